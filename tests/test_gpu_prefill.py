"""GPU parity of chunked prefill (many query tokens per sequence, causal) against
the float64 oracle, through the C ABI.

A chunk of C prompt tokens is appended, then each chunk token i attends to
positions [0, length - C + i].  C * G query rows per KV head exceed one
attention unit (64 rows, 32 at head_dim 256), so the library runs one unit
per tile of rows; each tile stops at the last position its rows see.
"""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch, prefix_pass_ran
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _prefill(pair, seqs, pt=0, api="prefill"):
    w = pair.w
    c = w.k_draft
    q = to_torch(w.q, w.dtype).contiguous()
    ws = pair.gpu.make_workspace(len(seqs), w.num_q_heads, int(max(pair.model.length(s) for s in seqs)),
                                 k_draft=c, partition_tokens=pt)
    if ws is not None:
        ws.fill_(float("nan"))
    if api == "prefill":
        return pair.gpu.prefill(seqs, q, w.scale, partition_tokens=pt, workspace=ws)
    return pair.gpu.verify(seqs, q, w.scale, partition_tokens=pt, workspace=ws)


@pytest.mark.parametrize("dtype,head_dim,g,chunk,pt", [
    ("bf16", 128, 4, 100, 0),     # 400 rows: 7 tiles of 64 (the last 16)
    ("bf16", 128, 4, 100, 64),    # split into 64-token partitions, merged by merge_kernel
    ("f16", 64, 8, 33, 0),        # 264 rows: last tile 8 rows
    ("f16", 64, 8, 33, 96),
    ("bf16", 256, 4, 20, 0),      # 80 rows in tiles of 32
    ("f32", 128, 2, 50, 0),       # fp32 body, 100 rows
    ("f32", 64, 4, 40, 64),
])
def test_prefill_chunk_matches_oracle(dtype, head_dim, g, chunk, pt):
    """Sequences with 0 (a whole prompt as one chunk), 37 and 300 cached
    tokens each take a chunk; pools and tables bit-exact, outputs and lse
    against the oracle for every chunk token and query head."""
    _say(f"prefill {dtype} D={head_dim} G={g} C={chunk} pt={pt}")
    hkv = 2
    w = make_custom(lengths=[0, 37, 300], mode="verify", num_q_heads=g * hkv, num_kv_heads=hkv,
                    head_dim=head_dim, dtype=dtype, seed=70 + chunk + head_dim, k_draft=chunk)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    out, lse = _prefill(pair, seqs, pt)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=chunk)
    assert_close(out, lse, ro, rl, dtype, f"prefill C={chunk}")


@pytest.mark.parametrize("dtype,head_dim,g,chunk,cached,pt", [
    ("bf16", 128, 4, 70, 1500, 0),     # 280 rows, tiles of 128, unsplit: 99 blocks, two table chunks
    ("f16", 256, 2, 40, 1300, 4096),   # 80 rows, tiles of 64, forced unsplit: 84 blocks, 8 loads per thread
    ("bf16", 64, 8, 30, 2100, 0),      # 240 rows; first partition 1,920 tokens (two chunks), merged
])
def test_prefill_long_context_crosses_table_chunks(dtype, head_dim, g, chunk, cached, pt):
    """Row tiles over contexts longer than one 64-entry chunk of the table:
    the LDS ring of pairs drains and refills at each chunk boundary.  Outputs
    and lse against the oracle for every chunk token and query head."""
    _say(f"prefill long {dtype} D={head_dim} G={g} C={chunk} cached={cached} pt={pt}")
    hkv = 2
    w = make_custom(lengths=[cached, cached // 3], mode="verify", num_q_heads=g * hkv, num_kv_heads=hkv,
                    head_dim=head_dim, dtype=dtype, seed=90 + head_dim, k_draft=chunk)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    out, lse = _prefill(pair, seqs, pt)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=chunk)
    assert_close(out, lse, ro, rl, dtype, f"prefill long C={chunk}")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_row_tiles_short_last_table_chunk(cache):
    """Row tiles whose table row ends just past a 64-entry chunk: the second
    chunk's ring holds one pair (65 and 66 blocks) or two (67 blocks), and a
    unit of exactly 64 blocks ends on the boundary.  The pipelined ring loop
    is then all prologue and epilogue: its first step, the PV of the last
    pair after the loop, and a V mask on a pair past the end.  160 query rows
    per kv head (two tiles of 128; the second tile's units see 8 positions
    more than the first's), unsplit.  Outputs and lse against the oracle for
    every chunk token and query head."""
    _say(f"row tiles, short last table chunk, {cache}")
    chunk = 40
    w = make_custom(lengths=[985, 1001, 1017, 984], mode="verify", num_q_heads=8, num_kv_heads=2, head_dim=128,
                    dtype="bf16", seed=97, k_draft=chunk)
    kw = {}
    if cache == "fp8":
        kw = dict(cache_dtype="fp8", kv_scales=(np.array([0.02, 0.5], np.float32), np.array([1.5, 0.03], np.float32)))
    pair = Pair(w, **kw)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    assert [int(pair.model.length(s)) for s in seqs] == [1025, 1041, 1057, 1024]
    out, lse = _prefill(pair, seqs, 4096)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=chunk)
    assert_close(out, lse, ro, rl, cache, f"row tiles, short last chunk, {cache}")


def test_prefill_equals_verify_bitwise_and_repeats():
    """pa_prefill is pa_verify with k_draft = chunk: bitwise equal results,
    and a second identical call repeats them."""
    w = make_custom(lengths=[5, 700], mode="verify", num_q_heads=16, num_kv_heads=4, head_dim=128,
                    dtype="bf16", seed=77, k_draft=48)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    seqs = [0, 1]
    a, la = _prefill(pair, seqs, 256, "prefill")
    torch.cuda.synchronize()
    a, la = a.clone(), la.clone()
    b, lb = _prefill(pair, seqs, 256, "verify")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    c, lc = _prefill(pair, seqs, 256, "prefill")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16)) and torch.equal(la, lc)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=48)
    assert_close(a, la, ro, rl, "bf16", "prefill 48")


def test_prefill_through_append_attend():
    """pa_append_attend with a 40-token chunk (160 rows, more than one tile:
    the append runs as its own launch) equals append + prefill and the oracle."""
    w = make_custom(lengths=[0, 100, 17], mode="verify", num_q_heads=32, num_kv_heads=8, head_dim=128,
                    dtype="bf16", seed=78, k_draft=40)
    seqs = list(range(w.batch))
    nk = to_torch(w.new_k.reshape(-1, w.num_kv_heads, w.head_dim), "bf16")
    nv = to_torch(w.new_v.reshape(-1, w.num_kv_heads, w.head_dim), "bf16")
    q = to_torch(w.q, "bf16").contiguous()
    res = []
    for one_call in (False, True):
        pair = Pair(w)
        pair.fill()
        if one_call:
            out, lse = pair.gpu.append_attend(seqs, nk, nv, q, w.scale)
        else:
            pair.gpu.append(seqs, [40] * w.batch, nk, nv)
            out, lse = pair.gpu.prefill(seqs, q, w.scale)
        pair.model.append(seqs, [40] * w.batch, w.new_k.reshape(-1, w.num_kv_heads, w.head_dim),
                          w.new_v.reshape(-1, w.num_kv_heads, w.head_dim))
        torch.cuda.synchronize()
        pair.check_pools_and_tables()
        res.append((pair, out.clone(), lse.clone()))
    (_, o1, l1), (pair, o2, l2) = res
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=40)
    assert_close(o2, l2, ro, rl, "bf16", "append_attend chunk")


def test_prefill_fp8_pool():
    """A 64-token chunk over an E4M3 pool with per-head scales."""
    w = make_custom(lengths=[10, 250], mode="verify", num_q_heads=16, num_kv_heads=4, head_dim=128,
                    dtype="bf16", seed=79, k_draft=64)
    ks = np.array([0.5, 0.03, 1.0, 2.5], np.float32)
    vs = np.array([0.01, 1.0, 0.25, 4.0], np.float32)
    pair = Pair(w, cache_dtype="fp8", kv_scales=(ks, vs))
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    out, lse = _prefill(pair, [0, 1], 128)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, [0, 1], w.q, w.scale, k_draft=64)
    assert_close(out, lse, ro, rl, "fp8", "fp8 prefill")


@pytest.mark.parametrize("head_dim,g,chunk,cached", [(64, 8, 20, 1400), (256, 2, 48, 1200)])
def test_prefill_fp8_long_context_row_tiles(head_dim, g, chunk, cached):
    """Row tiles of an E4M3 pool (pairs shared through the LDS ring as 8-bit
    codes, decoded per wave) over a context longer than one 64-entry table
    chunk, unsplit."""
    w = make_custom(lengths=[cached, 60], mode="verify", num_q_heads=g * 2, num_kv_heads=2, head_dim=head_dim,
                    dtype="bf16", seed=80 + head_dim, k_draft=chunk)
    ks = np.array([0.03, 2.5], np.float32)
    vs = np.array([4.0, 0.01], np.float32)
    pair = Pair(w, cache_dtype="fp8", kv_scales=(ks, vs))
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    out, lse = _prefill(pair, [0, 1], 4096)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, [0, 1], w.q, w.scale, k_draft=chunk)
    assert_close(out, lse, ro, rl, "fp8", "fp8 prefill, long context")


def test_prefill_shared_prefix_forks():
    """Six forks of a 1,100-token prompt prefix each take a 24-token chunk:
    the prefix's whole partitions go through the shared-prefix pass (rows of
    several tiles packed across the forks), the rest per tile."""
    w = make_custom(lengths=[16, 77, 200, 0, 31, 100], mode="verify", num_q_heads=16, num_kv_heads=4,
                    head_dim=128, dtype="bf16", seed=80, k_draft=24, prefix_len=1100)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    seqs = list(range(w.batch))
    out, lse = _prefill(pair, seqs, 512)
    torch.cuda.synchronize()
    assert prefix_pass_ran(pair.gpu)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=24)
    assert_close(out, lse, ro, rl, "bf16", "prefill over a shared prefix")
