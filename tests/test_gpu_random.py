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
