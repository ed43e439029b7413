"""Pins of the block-pool model: hand-worked traces, invariants, and the plain
definition of a sequence's contents (what was appended, cut back by truncation,
inherited from a parent on fork)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from oracle.allocator import InvalidError, NoMemError, PoolModel
from oracle.numerics import to_f64
from traces import random_trace


def _rows(r, n, hkv=1, d=4):
    return r.standard_normal((n, hkv, d)).astype(np.float32)


def test_hand_worked_trace():
    """Free order [5, 3, 0, 1, 4, 2]; every expected value below is worked by hand."""
    m = PoolModel(6, 1, 4, "f32", max_seqs=4, max_blocks_per_seq=4, free_order=[5, 3, 0, 1, 4, 2])
    r = np.random.default_rng(0)
    m.alloc(0)
    m.append([0], [20], _rows(r, 20), _rows(r, 20))       # blocks 5 (16 rows) + 3 (4 rows)
    assert m.table(0) == [5, 3] and m.length(0) == 20
    m.alloc(1, parent=0, shared_tokens=18)                  # shares 5 and the partial 3
    assert m.table(1) == [5, 3] and m.refcount(5) == 2 and m.refcount(3) == 2
    m.append([1], [1], _rows(r, 1), _rows(r, 1))            # 3 is shared: copy 2 rows into 0
    assert m.table(1) == [5, 0] and m.refcount(3) == 1 and m.refcount(0) == 1
    m.append([0], [1], _rows(r, 1), _rows(r, 1))            # 3 now private to seq 0: in place
    assert m.table(0) == [5, 3] and m.length(0) == 21
    assert m.num_free() == 3                                # 1, 4, 2 remain
    m.truncate(0, 10)                                       # releases 3 -> back of the deque
    assert m.table(0) == [5] and m.refcount(3) == 0
    m.free_seq(1)                                           # releases 5 (rc 2 -> 1) and 0
    assert m.refcount(5) == 1 and m.refcount(0) == 0
    assert list(m.free) == [1, 4, 2, 3, 0]
    m.append([0], [30], _rows(r, 30), _rows(r, 30))       # 6 rows into 5, then pops 1 and 4
    assert m.table(0) == [5, 1, 4] and m.length(0) == 40
    m.free_seq(0)                                           # releases 5, 1, 4 in logical order
    assert list(m.free) == [2, 3, 0, 5, 1, 4]
    assert all(m.refcount(b) == 0 for b in range(6))


def test_cow_copies_only_filled_rows_and_keeps_parent():
    r = np.random.default_rng(1)
    m = PoolModel(8, 2, 8, "f32", 4, 4, free_order=range(8), sentinel_bits=0x7FC0DEAD)
    m.alloc(0)
    k, v = _rows(r, 5, 2, 8), _rows(r, 5, 2, 8)
    m.append([0], [5], k, v)
    m.alloc(1, 0, 5)
    k1, v1 = _rows(r, 1, 2, 8), _rows(r, 1, 2, 8)
    m.append([1], [1], k1, v1)
    gk0, _ = m.gather(0)
    gk1, gv1 = m.gather(1)
    assert np.array_equal(gk0, k.view(np.uint32))
    assert np.array_equal(gk1, np.concatenate([k, k1]).view(np.uint32))
    assert np.array_equal(gv1, np.concatenate([v, v1]).view(np.uint32))
    # slots 6..15 of the copy still hold the fill pattern
    assert np.all(m.kpool[1, :, :, 6:, :] == 0x7FC0DEAD)


def test_nomem_is_all_or_nothing():
    m = PoolModel(3, 1, 4, "f32", 4, 8, free_order=[0, 1, 2])
    r = np.random.default_rng(2)
    m.alloc(0)
    m.alloc(1)
    m.append([0], [30], _rows(r, 30), _rows(r, 30))
    before = (list(m.free), list(m.rc), m.table(0), m.table(1), m.kpool.copy())
    with pytest.raises(NoMemError):
        m.append([1, 0], [1, 3], _rows(r, 4), _rows(r, 4))  # needs 2 blocks, 1 free
    assert (list(m.free), list(m.rc), m.table(0), m.table(1)) == before[:4]
    assert np.array_equal(m.kpool, before[4])


def test_invalid_calls():
    m = PoolModel(4, 1, 4, "f32", 2, 2)
    with pytest.raises(InvalidError):
        m.alloc(2)
    m.alloc(0)
    with pytest.raises(InvalidError):
        m.alloc(0)
    with pytest.raises(InvalidError):
        m.alloc(1, parent=0, shared_tokens=1)
    with pytest.raises(InvalidError):
        m.append([0, 0], [1, 1], np.zeros((2, 1, 4), np.float32), np.zeros((2, 1, 4), np.float32))
    with pytest.raises(InvalidError):
        m.append([0], [33], np.zeros((33, 1, 4), np.float32), np.zeros((33, 1, 4), np.float32))
    with pytest.raises(InvalidError):
        m.truncate(0, 1)
    with pytest.raises(InvalidError):
        PoolModel(4, 1, 4, "f32", 2, 2, free_order=[0, 1, 1, 2])


def replay_model(ops, m: PoolModel, r, logical):
    """Replay a trace on the model and on the plain per-sequence row lists."""
    codes = []
    for op in ops:
        try:
            if op[0] == "alloc":
                _, s, p, sh = op
                m.alloc(s, p, sh)
                logical[s] = [] if p < 0 else list(logical[p][:sh])
            elif op[0] == "append":
                _, ss, ns = op
                tot = sum(ns)
                k = _rows(r, tot, m.hkv, m.d)
                v = _rows(r, tot, m.hkv, m.d)
                m.append(ss, ns, k, v)
                i = 0
                for s, n in zip(ss, ns):
                    for _ in range(n):
                        logical[s].append((k[i], v[i]))
                        i += 1
            elif op[0] == "truncate":
                _, s, nl = op
                m.truncate(s, nl)
                logical[s] = logical[s][:nl]
            elif op[0] == "free":
                m.free_seq(op[1])
                logical.pop(op[1])
            codes.append(0)
        except InvalidError:
            codes.append(-1)
        except NoMemError:
            codes.append(-2)
    return codes


def check_invariants(m: PoolModel, logical):
    refs = [0] * m.num_blocks
    for s, tab in m.tables.items():
        n = m.length(s)
        assert len(tab) == (n + 15) // 16
        assert len(tab) * 16 - n <= 15          # only the blocks needed
        for b in tab:
            refs[b] += 1
    assert refs == m.rc
    assert len(set(m.free)) == len(m.free)
    assert set(m.free) == {b for b in range(m.num_blocks) if m.rc[b] == 0}
    for s in m.tables:
        gk, gv = m.gather(s)
        want = logical[s]
        assert gk.shape[0] == len(want)
        for t, (k, v) in enumerate(want):
            assert np.array_equal(gk[t], k.view(np.uint32))
            assert np.array_equal(gv[t], v.view(np.uint32))


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.integers(6, 30))
def test_random_traces_keep_invariants(seed, num_blocks):
    ops = random_trace(seed)
    r = np.random.default_rng(seed)
    order = r.permutation(num_blocks)
    m = PoolModel(num_blocks, 1, 4, "f32", 8, 16, free_order=order, sentinel_bits=0xFFFFFFFF)
    logical = {}
    replay_model(ops, m, np.random.default_rng(seed + 1), logical)
    check_invariants(m, logical)


def _decode_all(m, q, scale):
    return [A.decode_from_pool(m.kpool, m.vpool, m.table(s), m.length(s), q[s], scale, m.dtype)
            for s in sorted(m.tables)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_placement_permutation_invariance(dtype):
    """Two different physical placements give bitwise-identical attention."""
    r = np.random.default_rng(5)
    lens = [3, 16, 17, 40]
    ks = [r.standard_normal((n, 2, 8)).astype(np.float32) for n in lens]
    vs = [r.standard_normal((n, 2, 8)).astype(np.float32) for n in lens]
    q = r.standard_normal((4, 4, 8)).astype(np.float32)
    if dtype == "bf16":
        ks = [bf(x) for x in ks]
        vs = [bf(x) for x in vs]
        q = bf(q)
    outs = []
    for order in (np.arange(12), r.permutation(12)):
        m = PoolModel(12, 2, 8, dtype, 4, 4, free_order=order)
        for s in range(4):
            m.alloc(s)
        m.append(range(4), lens, np.concatenate(ks), np.concatenate(vs))
        outs.append(_decode_all(m, q, 0.35))
    for (o1, l1), (o2, l2) in zip(*outs):
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def bf(x):
    from workloads import bf16_bits_from_f32
    return bf16_bits_from_f32(x)


def test_shared_prefix_equals_private_copies():
    """Forked sequences reading a shared copy-on-write prefix give bitwise the
    same attention as sequences that hold private copies of it."""
    r = np.random.default_rng(6)
    pre_k, pre_v = _rows(r, 37, 2, 8), _rows(r, 37, 2, 8)
    suf = [(_rows(r, n, 2, 8), _rows(r, n, 2, 8)) for n in (1, 9, 30)]
    q = r.standard_normal((3, 4, 8)).astype(np.float32)
    shared = PoolModel(40, 2, 8, "f32", 4, 8, free_order=r.permutation(40))
    shared.alloc(0)
    shared.append([0], [37], pre_k, pre_v)
    for s in (1, 2):
        shared.alloc(s, 0, 37)
    shared.append([0, 1, 2], [len(k) for k, _ in suf],
                  np.concatenate([k for k, _ in suf]), np.concatenate([v for _, v in suf]))
    private = PoolModel(40, 2, 8, "f32", 4, 8, free_order=r.permutation(40))
    for s in range(3):
        private.alloc(s)
        private.append([s], [37 + len(suf[s][0])], np.concatenate([pre_k, suf[s][0]]),
                       np.concatenate([pre_v, suf[s][1]]))
    assert shared.refcount(shared.table(1)[0]) == 3      # full prefix blocks stay shared
    for (o1, l1), (o2, l2) in zip(_decode_all(shared, q, 0.3), _decode_all(private, q, 0.3)):
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_verify_equals_decode_of_forked_prefix():
    """Draft i of a verify equals a decode of a child forked at L + i + 1 tokens."""
    r = np.random.default_rng(7)
    m = PoolModel(20, 2, 8, "f32", 8, 8, free_order=r.permutation(20))
    m.alloc(0)
    m.append([0], [29], _rows(r, 29, 2, 8), _rows(r, 29, 2, 8))
    kd = 5
    q = r.standard_normal((kd, 4, 8)).astype(np.float32)
    o, lse = A.verify_from_pool(m.kpool, m.vpool, m.table(0), 29, q, 0.5, "f32")
    for i in range(kd):
        m.alloc(1 + i, 0, 29 - kd + i + 1)
        oi, li = A.decode_from_pool(m.kpool, m.vpool, m.table(1 + i), m.length(1 + i), q[i], 0.5, "f32")
        assert np.array_equal(o[i], oi) and np.array_equal(lse[i], li)


def test_rollback_then_append_matches_never_drafted():
    """Truncating rejected drafts then appending the corrected token gives the
    same logical cache as never appending the drafts ([P2] section 5.2)."""
    r = np.random.default_rng(8)
    base_k, base_v = _rows(r, 21, 1, 4), _rows(r, 21, 1, 4)
    drafts_k, drafts_v = _rows(r, 5, 1, 4), _rows(r, 5, 1, 4)
    fix_k, fix_v = _rows(r, 1, 1, 4), _rows(r, 1, 1, 4)
    a = PoolModel(10, 1, 4, "f32", 2, 4, free_order=r.permutation(10))
    a.alloc(0)
    a.append([0], [21], base_k, base_v)
    a.append([0], [5], drafts_k, drafts_v)
    a.truncate(0, 21 + 2)                       # two drafts accepted
    a.append([0], [1], fix_k, fix_v)
    b = PoolModel(10, 1, 4, "f32", 2, 4, free_order=r.permutation(10))
    b.alloc(0)
    b.append([0], [24], np.concatenate([base_k, drafts_k[:2], fix_k]),
             np.concatenate([base_v, drafts_v[:2], fix_v]))
    ga, gb = a.gather(0), b.gather(0)
    assert np.array_equal(ga[0], gb[0]) and np.array_equal(ga[1], gb[1])
    assert a.num_free() == b.num_free()
    assert np.array_equal(to_f64(ga[0], "f32"), to_f64(gb[0], "f32"))
