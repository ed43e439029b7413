"""Planted mistakes: plausible bugs in (copies of) the oracle must fail a pin.

These tests show that the pins are strong enough: a dropped term, a wrong
index, a transposed operand or an off-by-one in the causal limit each trips at
least one check.  The mistakes are planted in local copies on the CPU; the
oracle itself is not modified.
"""
import numpy as np
import pytest

import pins
import test_oracle_allocator as TA
from oracle import attention as A
from oracle import layout
from oracle.allocator import PoolModel


def _attn_variant(kind):
    def attn(kc, vc, q, scale, return_probs=False):
        n, hkv, d = kc.shape
        hq = q.shape[0]
        g = hq // hkv
        out = np.empty((hq, d))
        lse = np.empty(hq)
        probs = np.empty((hq, n))
        for h in range(hq):
            kvh = h % hkv if kind == "gqa_modulo" else h // g
            s = 1.0 if kind == "no_scale" else scale
            keys = vc if kind == "k_is_v" else kc
            x = s * (keys[:, kvh, :] @ q[h])
            m = np.max(x)
            e = np.exp(x - m)
            z = float(n) if kind == "mean_normaliser" else np.sum(e)
            p = e / z
            vals = kc if kind == "v_is_k" else vc
            out[h] = p @ vals[:, kvh, :]
            lse[h] = np.log(np.sum(e)) if kind == "lse_without_max" else m + np.log(np.sum(e))
            if kind == "lse_sign":
                lse[h] = m - np.log(np.sum(e))
            probs[h] = p
        if return_probs:
            return out, lse, probs
        return out, lse
    return attn


def _fails_some_check(attn):
    failures = 0
    for check in pins.ATTN_CHECKS:
        try:
            check(attn)
        except AssertionError:
            failures += 1
    try:
        pins.check_probs_sum_to_one(lambda k, v, q, s: attn(k, v, q, s, return_probs=True))
    except AssertionError:
        failures += 1
    return failures


@pytest.mark.parametrize("kind", ["gqa_modulo", "no_scale", "k_is_v", "v_is_k",
                                  "mean_normaliser", "lse_without_max", "lse_sign"])
def test_planted_attention_mistakes_are_caught(kind):
    assert _fails_some_check(_attn_variant(kind)) >= 1


def test_correct_copy_passes_every_check():
    assert _fails_some_check(_attn_variant("none")) == 0


def test_planted_verify_off_by_one_is_caught():
    def verify_excluding_self(kc, vc, q, scale):
        n, kd = kc.shape[0], q.shape[0]
        outs, lses = [], []
        for i in range(kd):
            ni = n - kd + i          # drops the draft's own row
            o, l_ = A.softmax_attention(kc[:ni], vc[:ni], q[i], scale)
            outs.append(o)
            lses.append(l_)
        return np.stack(outs), np.stack(lses)
    with pytest.raises(AssertionError):
        pins.check_verify_causal(verify_excluding_self, A.softmax_attention)


def _run_trace_invariants(seed=3):
    from traces import random_trace
    ops = random_trace(seed, n_ops=80)
    m = PoolModel(30, 2, 8, "f32", 8, 16, free_order=np.random.default_rng(seed).permutation(30))
    logical = {}
    TA.replay_model(ops, m, np.random.default_rng(seed + 1), logical)
    TA.check_invariants(m, logical)


def test_planted_layout_mistake_is_caught(monkeypatch):
    def bad_read_row(kpool, vpool, b, t, dtype):
        hkv, nchunk, _, x = kpool.shape[1], kpool.shape[2], kpool.shape[3], kpool.shape[4]
        k = kpool[b, :, :, t, :].transpose(0, 2, 1).reshape(hkv, -1)   # chunk order swapped
        return k.copy(), vpool[b, :, :, t].copy()
    monkeypatch.setattr(layout, "read_row", bad_read_row)
    with pytest.raises(AssertionError):
        _run_trace_invariants()


def test_planted_cow_short_copy_is_caught(monkeypatch):
    real = layout.copy_rows

    def short_copy(kpool, vpool, src, dst, n_rows):
        real(kpool, vpool, src, dst, max(0, n_rows - 1))
    monkeypatch.setattr(layout, "copy_rows", short_copy)
    with pytest.raises(AssertionError):
        for seed in range(3, 12):
            _run_trace_invariants(seed)


def test_planted_release_order_mistake_is_caught(monkeypatch):
    real_truncate = PoolModel.truncate

    def reversed_release(self, seq, new_len):
        keep = (new_len + 15) // 16
        tab = self.tables[seq]
        for b in reversed(tab[keep:]):
            self._release(b)
        del tab[keep:]
        self.lens[seq] = new_len
    monkeypatch.setattr(PoolModel, "truncate", reversed_release)
    with pytest.raises(AssertionError):
        TA.test_hand_worked_trace()
    monkeypatch.setattr(PoolModel, "truncate", real_truncate)
