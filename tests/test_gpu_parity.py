"""GPU parity: the gfx950 library against the float64 oracle, through the C ABI.

Pools, block tables and lengths must match the oracle's model bit for bit;
attention outputs within max-abs 2e-3 (fp16), 1e-2 (bf16), 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

from gpu_harness import (FILL, Pair, assert_close, contiguous_reference, oracle_decode, pool_bits,
                         prefix_pass_ran, to_torch)
from paged_kv_cache_216_amd import PaInvalid, PaNoMem
from workloads import make_custom, make_gqa70b, make_highbatch, make_long, make_tiny, make_verify
from workloads.synth import _to_storage as to_storage

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _decode(pair, seqs, q_bits, scale, pt=0, ws=True, k_draft=1):
    w = pair.w
    q = to_torch(q_bits, w.dtype)
    workspace = None
    if ws:
        workspace = pair.gpu.make_workspace(len(seqs), w.num_q_heads, int(max(pair.model.length(s) for s in seqs)),
                                            k_draft=k_draft, partition_tokens=pt)
        if workspace is not None:
            workspace.fill_(float("nan"))  # a partial read before it is written shows up
    if k_draft == 1:
        out, lse = pair.gpu.decode(seqs, q.reshape(len(seqs), w.num_q_heads, w.head_dim).contiguous(), scale,
                                   partition_tokens=pt, workspace=workspace)
        return out[:, None], lse[:, None]
    return pair.gpu.verify(seqs, q.contiguous(), scale, partition_tokens=pt, workspace=workspace)


# ---------------------------------------------------------------------------
def test_tiny_end_to_end():
    """4 sequences {17, 33, 64, 100}, fp32, D=64, 64-block pool: decode, append
    one row each (64 -> 65 opens a fifth block), decode again."""
    _say("tiny: fill")
    w = make_tiny()
    pair = Pair(w, max_seqs=4)
    pair.fill()
    pair.check_pools_and_tables()
    seqs = [0, 1, 2, 3]
    out, lse = _decode(pair, seqs, w.q, w.scale)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "f32", "tiny decode")
    pair.append_step_rows()
    pair.check_pools_and_tables()
    assert len(pair.model.table(2)) == 5
    out2, lse2 = _decode(pair, seqs, w.q2, w.scale)
    ro2, rl2 = oracle_decode(pair, seqs, w.q2, w.scale)
    assert_close(out2, lse2, ro2, rl2, "f32", "tiny decode after append")


@pytest.mark.parametrize("pt", [0, 256, 4096])
def test_gqa_group8_fp16(pt):
    """G = 8 (64 query heads over 8 KV heads), fp16, ragged lengths across
    partition edges; split and unsplit against the oracle."""
    _say(f"gqa fp16 pt={pt}")
    w = make_custom(lengths=[17, 512, 513, 1000, 1537, 33, 2048, 1], num_q_heads=64, num_kv_heads=8,
                    head_dim=128, dtype="f16", seed=21)
    pair = Pair(w)
    pair.fill()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    out, lse = _decode(pair, seqs, w.q, w.scale, pt=pt)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "f16", f"gqa pt={pt}")


def test_unsplit_paths_are_bitwise_equal():
    """A partition size above every length and 'no workspace' both run the
    unsplit kernel: bitwise identical results."""
    w = make_custom(lengths=[700, 1500, 64], num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=22)
    pair = Pair(w)
    pair.fill()
    seqs = [0, 1, 2]
    a, la = _decode(pair, seqs, w.q, w.scale, pt=2048)
    b, lb = _decode(pair, seqs, w.q, w.scale, pt=0, ws=False)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_highbatch_bf16_append_then_decode():
    """Log-normal lengths (median 200), bf16, 32/8 heads: append one row per
    sequence, then decode over the grown cache."""
    _say("highbatch small")
    w = make_custom(lengths=40, lengths_fn=lambda r, b: np.clip(np.rint(r.lognormal(np.log(200), 1.0, b)), 16, 2048),
                    mode="append_decode", num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=23)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    seqs = list(range(w.batch))
    out, lse = _decode(pair, seqs, w.q, w.scale)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "bf16", "highbatch small")


def test_long_split_fp16():
    """Contexts of 4096 and 3000 tokens in 512-token partitions, merged by lse."""
    _say("long small")
    w = make_custom(lengths=[4096, 3000], num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="f16", seed=24,
                    partition_tokens=512)
    pair = Pair(w)
    pair.fill()
    seqs = [0, 1]
    out, lse = _decode(pair, seqs, w.q, w.scale, pt=512)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "f16", "long split")


@pytest.mark.parametrize("prefix_len", [256, 250])
def test_shared_prefix_verify_bf16(prefix_len):
    """Sequences forked from one prefix (block-aligned and not: 250 leaves a
    shared partial block that each sequence copies on its first write), private
    suffixes, 5 drafts verified causally."""
    _say(f"verify prefix={prefix_len}")
    w = make_custom(lengths=[16, 77, 200, 512, 31, 100], mode="verify", num_q_heads=32, num_kv_heads=8,
                    head_dim=128, dtype="bf16", seed=25, k_draft=5, prefix_len=prefix_len)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    pair.check_pools_and_tables()
    full = prefix_len // 16
    assert pair.model.refcount(pair.model.table(3)[0]) == w.batch
    if prefix_len % 16:
        assert pair.model.table(3)[full] != pair.model.table(4)[full]  # the partial block was copied
    seqs = list(range(w.batch))
    out, lse = _decode(pair, seqs, w.q, w.scale, k_draft=5)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=5)
    assert_close(out, lse, ro, rl, "bf16", "verify")


def test_verify_k1_equals_decode_bitwise():
    w = make_custom(lengths=[300, 45], num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=26)
    pair = Pair(w)
    pair.fill()
    q = to_torch(w.q, "bf16")
    a, la = pair.gpu.decode([0, 1], q[:, 0].contiguous(), w.scale)
    b, lb = pair.gpu.verify([0, 1], q.contiguous(), w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b[:, 0].view(torch.int16)) and torch.equal(la, lb[:, 0])


def test_draft_i_equals_decode_of_fork():
    """Verify draft i equals a decode of a child forked at L + i + 1 tokens."""
    w = make_custom(lengths=[90], mode="verify", num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="f16",
                    seed=27, k_draft=4)
    pair = Pair(w, max_seqs=8)
    pair.fill()
    pair.append_step_rows()
    n = pair.model.length(0)
    q = to_torch(w.q, "f16")
    out, lse = pair.gpu.verify([0], q.contiguous(), w.scale)
    for i in range(4):
        pair.alloc(1 + i, 0, n - 4 + i + 1)
        o, l_ = pair.gpu.decode([1 + i], q[:, i].contiguous(), w.scale)
        torch.cuda.synchronize()
        assert torch.allclose(o.float(), out[:, i].float(), atol=2e-3, rtol=0)
        assert torch.allclose(l_, lse[:, i], atol=1e-4, rtol=0)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_placement_permutation_bitwise(dtype):
    """Two physical placements of the same logical cache: bitwise equal outputs."""
    w = make_custom(lengths=[5, 16, 31, 700], num_q_heads=16, num_kv_heads=4, head_dim=64, dtype=dtype, seed=28)
    outs = []
    for order in (np.arange(w.num_blocks), w.free_order):
        pair = Pair(w, free_order=order)
        pair.fill()
        o, l_ = _decode(pair, [0, 1, 2, 3], w.q, w.scale)
        torch.cuda.synchronize()
        outs.append((o.clone(), l_.clone()))
    it = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(outs[0][0].view(it), outs[1][0].view(it)) and torch.equal(outs[0][1], outs[1][1])


def test_shared_prefix_equals_private_copies_bitwise():
    w = make_custom(lengths=[10, 60, 3], mode="verify", num_q_heads=16, num_kv_heads=4, head_dim=128,
                    dtype="bf16", seed=29, k_draft=2, prefix_len=100)
    shared = Pair(w)
    shared.fill()
    shared.append_step_rows()
    # private copies need room for three full prefixes
    nb = 4 * w.num_blocks
    private = Pair(w, free_order=np.random.default_rng(1).permutation(nb), num_blocks=nb)
    for s in range(3):
        private.alloc(s)
        k = np.concatenate([w.prefix_k, w.k_rows[s], w.new_k[s]])
        v = np.concatenate([w.prefix_v, w.v_rows[s], w.new_v[s]])
        private.append([s], [k.shape[0]], k, v)
    a, la = _decode(shared, [0, 1, 2], w.q, w.scale, k_draft=2)
    b, lb = _decode(private, [0, 1, 2], w.q, w.scale, k_draft=2)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_single_token_returns_its_value_row_exactly(dtype):
    w = make_custom(lengths=[1, 1], num_q_heads=4, num_kv_heads=2, head_dim=128, dtype=dtype, seed=30)
    pair = Pair(w)
    pair.fill()
    out, _ = _decode(pair, [0, 1], w.q, w.scale)
    torch.cuda.synchronize()
    got = pool_bits(out, dtype).reshape(2, 4, 128)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[s, h], w.v_rows[s][0, h // 2].view(got.dtype))


@pytest.mark.parametrize("head_dim,g,kd", [(64, 1, 1), (64, 16, 4), (256, 4, 1), (256, 8, 4), (128, 16, 4),
                                           (128, 3, 7)])
def test_shapes_head_dims_and_row_tiles(head_dim, g, kd):
    """head_dim 64/128/256, 1..4 tiles of 16 query rows (group x drafts)."""
    _say(f"shape D={head_dim} G={g} K={kd}")
    w = make_custom(lengths=[33, 130, 600], mode="verify" if kd > 1 else "decode", num_q_heads=2 * g,
                    num_kv_heads=2, head_dim=head_dim, dtype="bf16", seed=31, k_draft=kd)
    pair = Pair(w)
    pair.fill()
    if kd > 1:
        pair.append_step_rows()
    seqs = [0, 1, 2]
    out, lse = _decode(pair, seqs, w.q, w.scale, k_draft=kd)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale, k_draft=kd)
    assert_close(out, lse, ro, rl, "bf16", f"D={head_dim} G={g} K={kd}")


def test_rollback_then_append():
    """Verify 5 drafts, accept 2, truncate, append the corrected token: pools,
    tables and free list follow the oracle's model exactly."""
    w = make_custom(lengths=[40, 47], mode="verify", num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="f16",
                    seed=32, k_draft=5)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    for s in (0, 1):
        pair.truncate(s, int(w.lengths[s]) + 2)
    r = np.random.default_rng(0)
    fix = r.standard_normal((2, 2, 64)).astype(np.float16)
    pair.append([0, 1], [1, 1], fix, fix[::-1].copy())
    pair.check_pools_and_tables()


def test_nomem_and_invalid_calls_change_nothing():
    w = make_custom(lengths=[20, 20], num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="bf16", seed=33,
                    num_blocks=5)
    w.max_blocks_per_seq = 8          # long enough that only the pool can run out
    pair = Pair(w)
    pair.fill()
    pair.check_pools_and_tables()
    big = np.zeros((40, 2, 64), np.uint16)
    with pytest.raises(PaNoMem):
        pair.gpu.append([0, 1], [20, 20], to_torch(big, "bf16"), to_torch(big, "bf16"))
    pair.check_pools_and_tables()
    pair.alloc(2)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(PaInvalid):
        pair.gpu.decode([2], q, 1.0)                    # empty context
    with pytest.raises(PaInvalid):
        pair.gpu.decode([0], torch.zeros((1, 3, 64), dtype=torch.bfloat16, device="cuda"), 1.0)
    out, _ = pair.gpu.decode([], torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda"), 1.0)
    assert out.shape == (0, 4, 64)
    pair.check_pools_and_tables()


# ---------------------------------------------------------------------------
# full-size workloads: every sequence checked against the oracle over its own
# logical rows (prefix, private rows, appended rows)
def _logical_rows(w, s):
    parts_k, parts_v = [], []
    if w.prefix_len:
        parts_k.append(w.prefix_k)
        parts_v.append(w.prefix_v)
    parts_k.append(w.k_rows[s])
    parts_v.append(w.v_rows[s])
    if w.new_k is not None and w.mode in ("append_decode", "verify"):
        parts_k.append(w.new_k[s])
        parts_v.append(w.new_v[s])
    return np.concatenate(parts_k), np.concatenate(parts_v)


def _check_all(w, out, lse, k_draft=1):
    o_all = out.detach().float().cpu()
    l_all = lse.detach().cpu()
    worst = 0.0
    for s in range(w.batch):
        k, v = _logical_rows(w, s)
        ro, rl = contiguous_reference(k, v, w.q[s], w.scale, w.dtype, k_draft)
        worst = max(worst, assert_close(o_all[s:s + 1], l_all[s:s + 1], ro[None], rl[None], w.dtype,
                                        f"{w.name} seq {s}"))
    _say(f"full {w.name}: all {w.batch} sequences within tolerance (max err {worst:.2e})")


def _full(w):
    """Fill, append the step's rows, then one attention call at the library's
    partition choice: every output row and lse against the oracle."""
    _say(f"full {w.name}: fill")
    pair = Pair(w, track_data=False)
    pair.fill()
    if w.new_k is not None:
        pair.append_step_rows()
    pair.check_tables()
    seqs = list(range(w.batch))
    out, lse = _decode(pair, seqs, w.q, w.scale, k_draft=w.k_draft)
    torch.cuda.synchronize()
    _say(f"full {w.name}: oracle on all {w.batch} sequences")
    _check_all(w, out, lse, w.k_draft)
    return pair


def _full_step(w):
    """The step bench.py times: pa_append_attend (append the step's rows and
    attend, one launch when possible) at the library's partition choice with a
    workspace sized as the bench sizes it.  Every output row and lse against
    the oracle, tables bit-exact."""
    _say(f"full step {w.name}: fill")
    pair = Pair(w, track_data=False)
    pair.fill()
    pair.check_tables()
    seqs = list(range(w.batch))
    t = w.new_k.shape[1]
    nk = to_torch(w.new_k.reshape(-1, w.num_kv_heads, w.head_dim), w.dtype)
    nv = to_torch(w.new_v.reshape(-1, w.num_kv_heads, w.head_dim), w.dtype)
    q = to_torch(w.q, w.dtype).contiguous()
    ws = pair.gpu.make_workspace(w.batch, w.num_q_heads, int(w.final_lengths().max()), k_draft=t)
    ws.fill_(float("nan"))
    pair.gpu.profile_enable(True)
    out, lse = pair.gpu.append_attend(seqs, nk, nv, q, w.scale, workspace=ws)
    torch.cuda.synchronize()
    n_append = pair.gpu.profile_read(2)[1]
    pair.gpu.profile_enable(False)
    assert n_append == 0, "the append ran as a launch of its own"
    pair.model.append(seqs, [t] * w.batch)
    pair.check_tables()
    _say(f"full step {w.name}: oracle on all {w.batch} sequences")
    _check_all(w, out, lse, t)
    return pair


def test_full_gqa70b():
    _full(make_gqa70b())


def test_full_highbatch():
    _full(make_highbatch())


def test_full_long():
    _full(make_long())


def test_full_highbatch_step():
    """Batch 256, log-normal lengths: the fused append + decode launch with
    the in-launch merge of split sequences, exactly as timed."""
    pair = _full_step(make_highbatch())
    pt, _ = pair.gpu.last_partition()
    assert pt == 512, pt


def _check_verify_partition(pair):
    # The library chose the partition: the shared-prefix pass runs in
    # four-wave workgroups of 128 query rows (1,280 rows = 10 row blocks),
    # in the attention launch beside its 64 x 8 attention units (128
    # workgroups of four).  At the default 512 tokens the launch would need
    # 8 partitions x 10 x 8 + 128 = 768 workgroups, more than one round of
    # the 2 per CU the device holds at once; the chosen length (a multiple of
    # 32, at most twice the default) fits it into one round.  The pass takes
    # the whole 4,096-token prefix (its last partition ends at 4,096).
    pt, prefix_wgs = pair.gpu.last_partition()
    resident = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    assert pt % 32 == 0 and 512 <= pt <= 1024, pt
    assert prefix_wgs == -(-4096 // pt) * 10 * 8, (pt, prefix_wgs)
    if 8 * 10 * 8 + 128 > resident:
        assert prefix_wgs + 128 <= resident, (pt, prefix_wgs, resident)
    st = pair.gpu.last_call_stats()
    assert st["prefix_kv_tokens"] == 4096
    # the splits (64 members x 8 kv heads x 5 groups of 4 rows) are merged by
    # a launch of their own, four waves per workgroup
    assert st["merge_workgroups"] == 64 * 8 * 5 // 4, st


def test_full_verify():
    _check_verify_partition(_full(make_verify()))


def test_full_verify_step():
    """64 forks of a 4,096-token prefix, 5 drafts appended and verified in one
    pa_append_attend call: shared-prefix pass, fused append + attention, merge."""
    _check_verify_partition(_full_step(make_verify()))


def test_many_partitions_fused_merge_and_repeat():
    """129 partitions of 32 tokens for one sequence (more than one wave of
    partials per merge), mixed with unsplit ones; a second identical call must
    give bitwise the same result (the merge counters reset themselves)."""
    w = make_custom(lengths=[4100, 70, 2000, 31], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="f16",
                    seed=34)
    pair = Pair(w)
    pair.fill()
    seqs = [0, 1, 2, 3]
    out, lse = _decode(pair, seqs, w.q, w.scale, pt=32)
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "f16", "129 partitions")
    out2, lse2 = _decode(pair, seqs, w.q, w.scale, pt=32)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_split_merge_reads_this_calls_partials(dtype):
    """Splits of 2..8 partitions (merged inside the attention launch): three
    calls on one workspace with different queries each match the oracle, so no
    call reads partials or counters left by the one before; the third call
    repeats the first bitwise."""
    w = make_custom(lengths=[1000, 2048, 300, 700, 90], num_q_heads=16, num_kv_heads=4, head_dim=128,
                    dtype=dtype, seed=35)
    pair = Pair(w)
    pair.fill()
    seqs = list(range(5))
    ws = pair.gpu.make_workspace(5, w.num_q_heads, 2048, partition_tokens=256)
    ws.fill_(float("nan"))
    rng = np.random.default_rng(36)
    q2_bits = to_storage(rng.standard_normal(w.q.shape, dtype=np.float32), dtype)
    outs = []
    for q_bits in (w.q, q2_bits, w.q):
        q = to_torch(q_bits, dtype).reshape(5, w.num_q_heads, w.head_dim).contiguous()
        out, lse = pair.gpu.decode(seqs, q, w.scale, partition_tokens=256, workspace=ws)
        torch.cuda.synchronize()
        ro, rl = oracle_decode(pair, seqs, q_bits, w.scale)
        assert_close(out[:, None], lse[:, None], ro, rl, dtype, "split, in-launch merge")
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[2][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[2][1])


@pytest.mark.parametrize("prefix_len,k_draft,dtype", [(1100, 5, "bf16"), (1024, 1, "f16"), (2100, 3, "bf16")])
def test_shared_prefix_pass(prefix_len, k_draft, dtype):
    """Six forks of one prefix: the whole partitions of the prefix (512 tokens
    each) are computed once for all six in the shared-prefix launch, the rest
    per sequence; the result matches the oracle and a pool where each sequence
    holds a private copy of the prefix (no sharing, so no shared-prefix pass)."""
    _say(f"shared-prefix pass prefix={prefix_len} k={k_draft} {dtype}")
    w = make_custom(lengths=[16, 77, 200, 512, 31, 100], mode="verify", num_q_heads=16, num_kv_heads=4,
                    head_dim=128, dtype=dtype, seed=37, k_draft=k_draft, prefix_len=prefix_len)
    shared = Pair(w)
    shared.fill()
    shared.append_step_rows()
    seqs = list(range(w.batch))
    a, la = _decode(shared, seqs, w.q, w.scale, pt=512, k_draft=k_draft)
    torch.cuda.synchronize()
    assert prefix_pass_ran(shared.gpu), "the shared-prefix pass did not run"
    ro, rl = oracle_decode(shared, seqs, w.q, w.scale, k_draft=k_draft)
    assert_close(a, la, ro, rl, dtype, "shared-prefix pass")
    nb = (len(seqs) + 1) * w.num_blocks
    private = Pair(w, free_order=np.random.default_rng(2).permutation(nb), num_blocks=nb)
    for s in seqs:
        private.alloc(s)
        k = np.concatenate([w.prefix_k, w.k_rows[s], w.new_k[s]])
        v = np.concatenate([w.prefix_v, w.v_rows[s], w.new_v[s]])
        private.append([s], [k.shape[0]], k, v)
    b, lb = _decode(private, seqs, w.q, w.scale, pt=512, k_draft=k_draft)
    torch.cuda.synchronize()
    assert not prefix_pass_ran(private.gpu)
    assert_close(b, lb, ro, rl, dtype, "private copies")


@pytest.mark.parametrize("pt,lengths", [(512, [640, 641, 1152, 1153, 1025, 1]), (256, [320, 321, 576, 577, 257, 64])])
def test_last_partition_absorbs_remainder_boundaries(pt, lengths):
    """Lengths at and just past the point where a sequence's last partition
    stops absorbing the remainder (a quarter partition): 640 tokens is one
    unit at 512-token partitions, 641 is 512 + 129, 1152 is 512 + 640, 1153
    is 512 + 512 + 129.  Decode, merged inside the launch, against the oracle."""
    w = make_custom(lengths=[n - 1 for n in lengths], mode="append_decode", num_q_heads=16, num_kv_heads=4,
                    head_dim=128, dtype="bf16", seed=42 + pt)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    seqs = list(range(w.batch))
    out, lse = _decode(pair, seqs, w.q, w.scale, pt=pt)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "bf16", f"absorbed remainders pt={pt}")


def test_shared_prefix_forks_with_short_members():
    """Decode over six forks of a 530-token prefix at 512-token partitions:
    the members' first appends copied the partly filled 34th block, so they
    share 528 positions; the pass takes them whole (a 512-token partition and
    a 16-token one) and each member keeps its own rest, unsplit as a short
    sequence would be.  Outputs match the oracle, and the structure is what the
    library reports."""
    w = make_custom(lengths=[10, 60, 100, 30, 200, 5], mode="append_decode", num_q_heads=16, num_kv_heads=4,
                    head_dim=128, dtype="bf16", seed=41, prefix_len=530)
    pair = Pair(w)
    pair.fill()
    pair.append_step_rows()
    seqs = list(range(w.batch))
    out, lse = _decode(pair, seqs, w.q, w.scale, pt=512)
    torch.cuda.synchronize()
    st = pair.gpu.last_call_stats()
    assert st["prefix_kv_tokens"] == 528 and st["prefix_workgroups"] > 0, st
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, "bf16", "forks with short members")


def test_shared_prefix_pass_fused_append_decode():
    """Decode step of eight forks of a 1,536-token prefix as one
    pa_append_attend call: shared-prefix launch, then the fused append +
    attention launch over the rest; matches the two-call path and the oracle."""
    w = make_custom(lengths=[5, 40, 300, 17, 600, 90, 1, 250], mode="append_decode", num_q_heads=32,
                    num_kv_heads=8, head_dim=128, dtype="bf16", seed=38, prefix_len=1536)
    _fused_vs_separate(w)


def _fused_vs_separate(w, prefix_fork_partial=False, pending_fork=False):
    """Run the same step as append + attend (two calls) and as one
    pa_append_attend call: pools, tables and outputs must be bitwise equal."""
    pairs = []
    for fused in (False, True):
        pair = Pair(w, max_seqs=2 * w.batch + 2)
        pair.fill()
        if pending_fork:
            # a child sharing only full blocks of sequence 1: its table entries
            # are still pending, and no write needs a copy
            full = (int(pair.model.length(1)) // 16) * 16
            pair.alloc(w.batch, 1, full)
        seqs = list(range(w.batch))
        t = w.new_k.shape[1]
        nk = to_torch(w.new_k.reshape(-1, w.num_kv_heads, w.head_dim), w.dtype)
        nv = to_torch(w.new_v.reshape(-1, w.num_kv_heads, w.head_dim), w.dtype)
        q = to_torch(w.q, w.dtype)
        ws = pair.gpu.make_workspace(w.batch, w.num_q_heads, int(w.final_lengths().max()), k_draft=t)
        if ws is not None:
            ws.fill_(float("nan"))
        if fused:
            out, lse = pair.gpu.append_attend(seqs, nk, nv, q.contiguous(), w.scale, workspace=ws)
        else:
            pair.gpu.append(seqs, [t] * w.batch, nk, nv)
            if t == 1:
                out, lse = pair.gpu.decode(seqs, q[:, 0].contiguous(), w.scale, workspace=ws)
                out, lse = out[:, None], lse[:, None]
            else:
                out, lse = pair.gpu.verify(seqs, q.contiguous(), w.scale, workspace=ws)
        pair.model.append(seqs, [t] * w.batch, w.new_k.reshape(-1, w.num_kv_heads, w.head_dim),
                          w.new_v.reshape(-1, w.num_kv_heads, w.head_dim))
        torch.cuda.synchronize()
        pair.check_pools_and_tables()
        pairs.append((pair, out.clone(), lse.clone()))
    it = torch.int32 if w.dtype == "f32" else torch.int16
    (_, o1, l1), (p2, o2, l2) = pairs
    assert torch.equal(o1.view(it), o2.view(it)), "fused and separate outputs differ"
    assert torch.equal(l1, l2)
    return p2, o2, l2


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_append_attend_decode_matches_separate_and_oracle(dtype):
    w = make_custom(lengths=[15, 16, 31, 200, 513, 1000, 1, 47], mode="append_decode", num_q_heads=32,
                    num_kv_heads=8, head_dim=128, dtype=dtype, seed=40)
    pair, out, lse = _fused_vs_separate(w)
    seqs = list(range(w.batch))
    ro, rl = oracle_decode(pair, seqs, w.q, w.scale)
    assert_close(out, lse, ro, rl, dtype, "fused decode step")


def test_append_attend_verify_shared_prefix():
    w = make_custom(lengths=[16, 77, 5, 300], mode="verify", num_q_heads=32, num_kv_heads=8, head_dim=128,
                    dtype="bf16", seed=41, k_draft=5, prefix_len=256)
    pair, out, lse = _fused_vs_separate(w)
    ro, rl = oracle_decode(pair, list(range(w.batch)), w.q, w.scale, k_draft=5)
    assert_close(out, lse, ro, rl, "bf16", "fused verify")


def test_append_attend_copy_on_write_falls_back():
    # a 250-token shared prefix leaves a shared partial block: the first write
    # into it needs a copy, so the library issues separate launches
    w = make_custom(lengths=[0, 0, 0], mode="verify", num_q_heads=16, num_kv_heads=4, head_dim=64,
                    dtype="f16", seed=42, k_draft=3, prefix_len=250)
    _fused_vs_separate(w)


def test_append_attend_with_pending_table_falls_back():
    w = make_custom(lengths=[40, 90], mode="append_decode", num_q_heads=8, num_kv_heads=2, head_dim=128,
                    dtype="bf16", seed=43)
    _fused_vs_separate(w, pending_fork=True)


def test_append_attend_fp32():
    w = make_custom(lengths=[17, 64], mode="append_decode", num_q_heads=4, num_kv_heads=4, head_dim=64,
                    dtype="f32", seed=44, scale=0.125)
    pair, out, lse = _fused_vs_separate(w)
    ro, rl = oracle_decode(pair, [0, 1], w.q, w.scale)
    assert_close(out, lse, ro, rl, "f32", "fp32 append+attend")
