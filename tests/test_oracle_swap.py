"""Pins for the oracle's swap to host memory (PoolModel.swap_out / swap_in):
the round trip restores the rows bit for bit, the blocks come from the front
of the free list as an append's would, shared blocks stay with their other
holders, and a swap-in that cannot get its blocks changes nothing."""
import numpy as np
import pytest

from oracle.allocator import InvalidError, NoMemError, PoolModel


def _rows(rng, n):
    return rng.integers(0, 2 ** 16, size=(n, 2, 64)).astype(np.uint16)


def test_round_trip_and_block_order():
    rng = np.random.default_rng(0)
    m = PoolModel(12, 2, 64, "bf16", 4, 6, free_order=rng.permutation(12))
    k, v = _rows(rng, 37), _rows(rng, 37)
    m.alloc(0)
    m.append([0], [37], k, v)
    old = m.table(0)
    n, ks, vs = m.swap_out(0)
    assert n == 37 and np.array_equal(ks, k) and np.array_equal(vs, v)
    assert list(m.free)[-3:] == old          # released in logical order
    front = list(m.free)[:3]
    m.swap_in(2, n, ks, vs)
    assert m.table(2) == front and m.length(2) == 37
    k2, v2 = m.gather(2)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)


def test_shared_blocks_stay_with_their_other_holders():
    rng = np.random.default_rng(1)
    m = PoolModel(12, 2, 64, "bf16", 4, 6)
    k, v = _rows(rng, 40), _rows(rng, 40)
    m.alloc(0)
    m.append([0], [40], k, v)
    m.alloc(1, 0, 32)                       # shares the first two blocks
    shared = m.table(0)[:2]
    n, ks, vs = m.swap_out(1)
    assert n == 32 and np.array_equal(ks, k[:32])
    assert [m.refcount(b) for b in shared] == [1, 1] and not any(b in m.free for b in shared)


def test_swap_in_without_blocks_changes_nothing():
    rng = np.random.default_rng(2)
    m = PoolModel(4, 2, 64, "bf16", 4, 8)
    k = _rows(rng, 60)
    before = (list(m.free), dict(m.lens))
    with pytest.raises(NoMemError):
        m.swap_in(0, 65, np.concatenate([k, k[:5]]), np.concatenate([k, k[:5]]))
    assert (list(m.free), dict(m.lens)) == before
    with pytest.raises(InvalidError):
        m.swap_out(3)
