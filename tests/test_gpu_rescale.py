"""GPU parity where the online-softmax running maximum must move.

The attention kernels keep a per-row reference maximum and move it only when
a score beats it by more than 8 (log2 units); when it moves, the accumulator
and the running sum are rescaled by 2^(m_old - m_new).  Inputs drawn N(0, 1)
almost never move it after the first 32-token pair, so these cases plant keys
aligned with a query (``workloads.with_rising_scores``): at 40 and 100 tokens
into every span of ``pt`` tokens, at gains 1 and 2.5, each raising that row's
best score by far more than 8 log2 units.  Every case first checks, from the
float64 scores of the oracle's gathered rows, that some row's maximum does rise
by more than 8 after the first 32 tokens of each span, so the rescale provably
runs; then it compares outputs and lse with the oracle.

Online softmax itself is this library's reading: the pages describe one fused
pass that keeps scores and probabilities on chip ("Les noyaux d'attention",
ranksignal.fr post 218), which needs the running maximum and the rescale.
"""
import math

import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch, prefix_pass_ran
from oracle import attention as A
from oracle.numerics import to_f64
from workloads import make_custom, with_rising_scores

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)
SLACK = 8.0  # log2 units a score must beat the reference maximum by to move it


def _say(msg):
    print(msg, flush=True)


def _scores_log2(pair, seq, q_bits, scale):
    """[K, Hq, n] scores in log2 units from the oracle's gather of ``seq``."""
    m = pair.model
    sc = (m.k_scale, m.v_scale) if m.dtype == "fp8" else None
    kc, _ = A.gather(m.kpool, m.vpool, m.table(seq), m.length(seq), m.dtype, sc)
    q = to_f64(q_bits, "bf16" if m.dtype == "fp8" else m.dtype)  # [K, Hq, D]
    g = q.shape[1] // kc.shape[1]
    x = np.einsum("khd,nhd->khn", q, np.repeat(kc, g, axis=1)) * scale * LOG2E
    return x


def _assert_rises(pair, seqs, q_bits, scale, every, k_draft=1):
    """Every span [b, b + every) that reaches past its first planted key (40
    tokens in) has a row whose maximum over the span's first 32 tokens is
    beaten by more than SLACK later in the span."""
    spans = 0
    for i, s in enumerate(seqs):
        x = _scores_log2(pair, s, q_bits[i], scale)
        n = x.shape[-1]
        for b in range(0, n, every):
            best = -np.inf
            for d in range(k_draft):
                vis = n - k_draft + d + 1
                e = min(b + every, vis)
                if e - b <= 40:
                    continue
                first = x[d, :, b:b + 32].max(axis=-1)
                rest = x[d, :, b + 32:e].max(axis=-1)
                best = max(best, float(np.max(rest - first)))
            if best > -np.inf:
                spans += 1
                assert best > SLACK, f"seq {s} span {b}: largest rise {best:.2f} log2 units"
    assert spans > 0


def _ws(pair, seqs, k_draft, pt):
    if pt < 0:
        return None, 0
    w = pair.w
    ws = pair.gpu.make_workspace(len(seqs), w.num_q_heads, int(max(pair.model.length(s) for s in seqs)),
                                 k_draft=k_draft, partition_tokens=pt)
    if ws is not None:
        ws.fill_(float("nan"))
    return ws, pt


def _attend(pair, seqs, q_bits, k_draft, pt, dtype):
    w = pair.w
    qd = "bf16" if dtype == "fp8" else dtype
    q = to_torch(q_bits, qd)
    ws, pt = _ws(pair, seqs, k_draft, pt)
    if k_draft == 1:
        out, lse = pair.gpu.decode(seqs, q.reshape(len(seqs), w.num_q_heads, w.head_dim).contiguous(), w.scale,
                                   partition_tokens=pt, workspace=ws)
        return out[:, None], lse[:, None]
    return pair.gpu.verify(seqs, q.contiguous(), w.scale, partition_tokens=pt, workspace=ws)


def _pair(w, dtype):
    if dtype == "fp8":
        return Pair(w, cache_dtype="fp8", kv_scales=(np.full(w.num_kv_heads, 0.05, np.float32),
                                                     np.full(w.num_kv_heads, 0.02, np.float32)))
    return Pair(w)


# pt -1: no workspace (unsplit); 256: split, merged inside the attention launch;
# 64: up to 30 partitions, merged by merge_kernel
@pytest.mark.parametrize("pt", [-1, 256, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "fp8"])
def test_rescale_decode(dtype, pt):
    _say(f"rescale decode {dtype} pt={pt}")
    wd = "bf16" if dtype == "fp8" else dtype
    every = 256 if pt < 0 else pt
    base = make_custom(lengths=[33, 150, 700, 1900], mode="append_decode", num_q_heads=16, num_kv_heads=4,
                       head_dim=128, dtype=wd, seed=101)
    w = with_rising_scores(base, every)
    pair = _pair(w, dtype)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    _assert_rises(pair, seqs, w.q, w.scale, every)
    out, lse = _attend(pair, seqs, w.q, 1, pt, dtype)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, dtype, f"rescale decode pt={pt}")


@pytest.mark.parametrize("head_dim", [64, 256])
def test_rescale_decode_head_dims(head_dim):
    _say(f"rescale decode D={head_dim}")
    base = make_custom(lengths=[120, 900], mode="append_decode", num_q_heads=8, num_kv_heads=2,
                       head_dim=head_dim, dtype="bf16", seed=102)
    w = with_rising_scores(base, 256)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    seqs = [0, 1]
    _assert_rises(pair, seqs, w.q, w.scale, 256)
    for pt in (-1, 256):
        out, lse = _attend(pair, seqs, w.q, 1, pt, "bf16")
        ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
        assert_close(out, lse, ro, rl, "bf16", f"rescale D={head_dim} pt={pt}")


# verify: 5 drafts x G 4 = 20 rows per kv head, two 16-row tiles per wave
@pytest.mark.parametrize("pt", [-1, 256])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rescale_verify(dtype, pt):
    _say(f"rescale verify {dtype} pt={pt}")
    every = 256 if pt < 0 else pt
    base = make_custom(lengths=[150, 700, 1300], mode="verify", num_q_heads=16, num_kv_heads=4, head_dim=128,
                       dtype="bf16", seed=103, k_draft=5)
    w = with_rising_scores(base, every)
    pair = _pair(w, dtype)
    pair.fill()
    pair.append_step_rows()
    seqs = list(range(w.batch))
    _assert_rises(pair, seqs, w.q, w.scale, every, k_draft=5)
    out, lse = _attend(pair, seqs, w.q, 5, pt, dtype)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=5)
    assert_close(out, lse, ro, rl, dtype, f"rescale verify pt={pt}")


# chunked prefill: 40 tokens x G 4 = 160 rows, row tiles of 128 (tile_kernel)
@pytest.mark.parametrize("pt", [-1, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "fp8"])
def test_rescale_prefill_row_tiles(dtype, pt):
    _say(f"rescale prefill {dtype} pt={pt}")
    wd = "bf16" if dtype == "fp8" else dtype
    every = 256 if pt < 0 else pt
    base = make_custom(lengths=[300, 1500], mode="verify", num_q_heads=8, num_kv_heads=2, head_dim=128,
                       dtype=wd, seed=104, k_draft=40)
    w = with_rising_scores(base, every)
    pair = _pair(w, dtype)
    pair.fill()
    pair.append_step_rows()
    seqs = [0, 1]
    _assert_rises(pair, seqs, w.q, w.scale, every, k_draft=40)
    q = to_torch(w.q, wd).contiguous()
    ws, ptu = _ws(pair, seqs, 40, pt)
    out, lse = pair.gpu.prefill(seqs, q, w.scale, partition_tokens=ptu, workspace=ws)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=40)
    assert_close(out, lse, ro, rl, dtype, f"rescale prefill pt={pt}")


# shared-prefix pass: six forks of a 1,100-token prefix, 512-token partitions;
# the prefix's spikes are aligned with sequence 0's queries
@pytest.mark.parametrize("dtype,k_draft", [("bf16", 5), ("bf16", 1), ("fp8", 5)])
def test_rescale_shared_prefix_pass(dtype, k_draft):
    _say(f"rescale shared prefix {dtype} k={k_draft}")
    base = make_custom(lengths=[16, 77, 200, 512, 31, 100], mode="verify" if k_draft > 1 else "append_decode",
                       num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16", seed=105, k_draft=k_draft,
                       prefix_len=1100)
    w = with_rising_scores(base, 512)
    pair = _pair(w, dtype)
    pair.fill()
    pair.append_step_rows()
    seqs = list(range(w.batch))
    _assert_rises(pair, seqs[:1], w.q[:1], w.scale, 512, k_draft=k_draft)
    out, lse = _attend(pair, seqs, w.q, k_draft, 512, dtype)
    torch.cuda.synchronize()
    assert prefix_pass_ran(pair.gpu), "the shared-prefix pass did not run"
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=k_draft)
    assert_close(out, lse, ro, rl, dtype, "rescale shared prefix")


# one launch appends and attends; the appended row itself carries the largest
# score, so the tail step that splices it in rescales too
@pytest.mark.parametrize("pt", [-1, 256, 0])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rescale_append_attend(dtype, pt):
    _say(f"rescale append_attend {dtype} pt={pt}")
    every = 256 if pt <= 0 else pt
    base = make_custom(lengths=[15, 200, 513, 1000, 47, 1], mode="append_decode", num_q_heads=32, num_kv_heads=8,
                       head_dim=128, dtype="bf16", seed=106)
    w = with_rising_scores(base, every, new_row_gain=4.0)
    pair = _pair(w, dtype)
    pair.fill()
    seqs = list(range(w.batch))
    nk = to_torch(w.new_k.reshape(-1, w.num_kv_heads, w.head_dim), "bf16")
    nv = to_torch(w.new_v.reshape(-1, w.num_kv_heads, w.head_dim), "bf16")
    q = to_torch(w.q, "bf16").contiguous()
    ws, ptu = _ws(pair, seqs, 1, pt)
    pair.gpu.profile_enable(True)
    out, lse = pair.gpu.append_attend(seqs, nk, nv, q, w.scale, partition_tokens=ptu, workspace=ws)
    torch.cuda.synchronize()
    _, n_app = pair.gpu.profile_read(2)
    pair.gpu.profile_enable(False)
    assert n_app == 0, "the append ran as a launch of its own, not inside the attention launch"
    pair.model.append(seqs, [1] * w.batch, w.new_k.reshape(-1, w.num_kv_heads, w.head_dim),
                      w.new_v.reshape(-1, w.num_kv_heads, w.head_dim))
    pair.check_pools_and_tables()
    _assert_rises(pair, seqs, w.q, w.scale, every)
    # the last row beats everything before it in every sequence longer than a pair
    for i, s in enumerate(seqs):
        x = _scores_log2(pair, s, w.q[i], w.scale)[0]
        if x.shape[-1] > 32:
            assert np.max(x[:, -1] - x[:, :-1].max(axis=-1)) > SLACK
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, dtype, f"rescale append_attend pt={pt}")


@pytest.mark.parametrize("pt", [-1, 256])
def test_large_scale_underflowing_probabilities(pt):
    """scale 1 instead of 1/sqrt(128): scores spread over about +-50 log2
    units, most probabilities underflow, and the row maxima keep moving."""
    _say(f"large scale pt={pt}")
    base = make_custom(lengths=[90, 600, 2000], mode="append_decode", num_q_heads=16, num_kv_heads=4,
                       head_dim=128, dtype="bf16", seed=107, scale=1.0)
    w = with_rising_scores(base, 256, offsets=(), gains=())  # values halved only: one row dominates each output
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    seqs = [0, 1, 2]
    _assert_rises(pair, seqs, w.q, w.scale, 256 if pt < 0 else pt)
    out, lse = _attend(pair, seqs, w.q, 1, pt, "bf16")
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "bf16", f"scale 1 pt={pt}")
