"""Seeded random configurations through the C ABI against the oracle: head
dims 64 / 128 / 256, 1-4 kv heads, groups of 1-8, 1-20 query tokens per
sequence, bf16 / f16 / E4M3 pools, shared copy-on-write prefixes, partition
lengths from 32 tokens to the library's choice.  Each case checks pools and
tables bit-exactly and outputs / lse at the dtype's tolerance, so paths that
the targeted tests reach one at a time (row tiles, the shared-prefix pass,
split merges, absorbed remainders) also meet in combinations."""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for case in range(n):
        prefix = int(rng.choice([0, 0, 300, 530, 1100]))
        b = int(rng.integers(1, 9))
        out.append(dict(
            D=int(rng.choice([64, 128, 256])), hkv=int(rng.choice([1, 2, 4])), G=int(rng.choice([1, 2, 4, 8])),
            kd=int(rng.choice([1, 1, 2, 5, 20])), dtype=str(rng.choice(["bf16", "f16", "fp8"])), prefix=prefix,
            lengths=[int(x) for x in rng.integers(0, 1400, size=max(b, 6) if prefix else b)],
            pt=int(rng.choice([0, 32, 64, 256, 512, 608])),
            scales=(rng.uniform(0.01, 3.0, size=4).astype(np.float32), rng.uniform(0.01, 3.0, size=4).astype(np.float32)),
            seed=2000 + case))
    return out


@pytest.mark.parametrize("c", _cases(24, 20261203), ids=lambda c: f"D{c['D']}-h{c['hkv']}-g{c['G']}-k{c['kd']}-"
                         f"{c['dtype']}-p{c['prefix']}-pt{c['pt']}")
def test_random_configuration(c):
    print(f"random {c['dtype']} D={c['D']} hkv={c['hkv']} G={c['G']} kd={c['kd']} prefix={c['prefix']} "
          f"lens={c['lengths']} pt={c['pt']}", flush=True)
    wd = "bf16" if c["dtype"] == "fp8" else c["dtype"]
    w = make_custom(lengths=c["lengths"], mode="verify" if c["kd"] > 1 else "append_decode",
                    num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"], head_dim=c["D"], dtype=wd, seed=c["seed"],
                    k_draft=c["kd"], prefix_len=c["prefix"])
    if c["dtype"] == "fp8":
        pair = Pair(w, cache_dtype="fp8", kv_scales=(c["scales"][0][:c["hkv"]], c["scales"][1][:c["hkv"]]))
    else:
        pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    q = to_torch(w.q, wd)
    ws = pair.gpu.make_workspace(len(seqs), w.num_q_heads, int(max(pair.model.length(s) for s in seqs)),
                                 k_draft=c["kd"], partition_tokens=c["pt"])
    if ws is not None:
        ws.fill_(float("nan"))
    if c["kd"] == 1:
        out, lse = pair.gpu.decode(seqs, q.reshape(len(seqs), w.num_q_heads, c["D"]).contiguous(), w.scale,
                                   partition_tokens=c["pt"], workspace=ws)
        out, lse = out[:, None], lse[:, None]
    else:
        out, lse = pair.gpu.verify(seqs, q.contiguous(), w.scale, partition_tokens=c["pt"], workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=c["kd"])
    assert_close(out, lse, ro, rl, c["dtype"], "random configuration")


def _fused_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for case in range(n):
        d = int(rng.choice([64, 128, 256]))
        g = int(rng.choice([1, 2, 4, 8]))
        kd = int(rng.choice([1, 1, 2, 3, 5]))
        if g * kd > (64 if d <= 128 else 32):
            kd = 1
        prefix = int(rng.choice([0, 0, 300, 530, 1100, 2100]))
        b = int(rng.integers(4, 10)) if prefix else int(rng.integers(1, 10))
        out.append(dict(
            D=d, hkv=int(rng.choice([1, 2, 4, 8])), G=g, kd=kd, dtype=str(rng.choice(["bf16", "f16", "fp8"])),
            prefix=prefix, lengths=[int(x) for x in rng.integers(0 if prefix else 1, 1400, size=b)],
            pt=int(rng.choice([0, 0, 32, 64, 256, 512, 608])), rising=bool(rng.random() < 0.3),
            scales=(rng.uniform(0.01, 3.0, size=8).astype(np.float32), rng.uniform(0.01, 3.0, size=8).astype(np.float32)),
            seed=6000 + case))
    return out


@pytest.mark.parametrize("c", _fused_cases(16, 20261204), ids=lambda c: f"D{c['D']}-h{c['hkv']}-g{c['G']}-k{c['kd']}-"
                         f"{c['dtype']}-p{c['prefix']}-pt{c['pt']}{'-rising' if c['rising'] else ''}")
def test_random_fused_step(c):
    """The same kind of draws through pa_append_attend (append and attention in
    one call: fused when one unit takes all query rows, the shared-prefix units
    inside the attention launch and the merge launch after it), with kv heads up
    to 8 and, in some cases, scores that rise after the first pair."""
    from workloads.synth import with_rising_scores

    print(f"random fused {c}", flush=True)
    wd = "bf16" if c["dtype"] == "fp8" else c["dtype"]
    w = make_custom(lengths=c["lengths"], mode="verify" if c["kd"] > 1 else "append_decode",
                    num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"], head_dim=c["D"], dtype=wd, seed=c["seed"],
                    k_draft=c["kd"], prefix_len=c["prefix"])
    if c["rising"]:
        w = with_rising_scores(w, every=2)
    if c["dtype"] == "fp8":
        pair = Pair(w, cache_dtype="fp8", kv_scales=(c["scales"][0][:c["hkv"]], c["scales"][1][:c["hkv"]]))
    else:
        pair = Pair(w)
    pair.fill()
    seqs = list(range(w.batch))
    n, t, hkv, d = len(seqs), w.new_k.shape[1], c["hkv"], c["D"]
    kn, vn = w.new_k.reshape(-1, hkv, d), w.new_v.reshape(-1, hkv, d)
    ws = pair.gpu.make_workspace(n, w.num_q_heads, int(max(pair.model.length(s) for s in seqs)) + t,
                                 k_draft=c["kd"], partition_tokens=c["pt"])
    if ws is not None:
        ws.fill_(float("nan"))
    out, lse = pair.gpu.append_attend(seqs, to_torch(kn, wd), to_torch(vn, wd), to_torch(w.q, wd).contiguous(),
                                      w.scale, partition_tokens=c["pt"], workspace=ws)
    pair.model.append(seqs, [t] * n, kn, vn)
    pair.check_pools_and_tables()
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=c["kd"])
    assert_close(out, lse, ro, rl, c["dtype"], "random fused step")
