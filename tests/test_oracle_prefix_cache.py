"""Pins for the oracle's prefix-cache model (oracle/prefix_cache.py): the reuse
rule of the pages (from the first token to the first differing one, never
past it), whole-block granularity, reference counting, eviction order, and
copy-on-write of a cached block."""
import numpy as np
import pytest

from oracle.allocator import InvalidError, PoolModel
from oracle.prefix_cache import PrefixCacheModel


def _pool(nb=16, track=False):
    return PoolModel(nb, 1, 64, "bf16", 8, 8, track_data=track)


def _prompt(n, start=1):
    return list(range(start, start + n))


def test_reuse_stops_at_first_differing_token():
    m = _pool()
    c = PrefixCacheModel(m)
    a = _prompt(64)
    m.alloc(0)
    m.append([0], [64])
    assert c.insert(0, a) == 4
    assert c.match(a) == 64
    b = list(a)
    b[20] = 999           # inside block 1: blocks 2 and 3 agree again, still not reused
    assert c.match(b) == 16
    first = [999] + a[1:]  # the very first token differs: nothing is reused
    assert c.match(first) == 0


def test_whole_blocks_only():
    m = _pool()
    c = PrefixCacheModel(m)
    a = _prompt(40)
    m.alloc(0)
    m.append([0], [40])
    assert c.insert(0, a) == 2          # 40 tokens: two full blocks, the tail is not registered
    assert c.match(a[:20] + [7] * 20) == 16
    assert c.match(a[:15]) == 0         # two prompts sharing their first 15 tokens share no block
    assert c.match(a[:32]) == 32 and c.match(a[:31]) == 16


def test_references_and_release():
    m = _pool()
    c = PrefixCacheModel(m)
    a = _prompt(32)
    m.alloc(0)
    m.append([0], [32])
    blocks = m.table(0)
    c.insert(0, a)
    assert [m.refcount(b) for b in blocks] == [2, 2]
    assert c.alloc_from(1, a + [5, 6, 7]) == 32
    assert m.table(1) == blocks and m.length(1) == 32
    assert [m.refcount(b) for b in blocks] == [3, 3]
    m.free_seq(0)
    m.free_seq(1)
    assert [m.refcount(b) for b in blocks] == [1, 1]      # still held by the cache
    assert not any(b in m.free for b in blocks)
    assert c.evict(10) == 2 and len(c) == 0
    assert list(m.free)[-2:] == [blocks[1], blocks[0]]    # leaf first, then its parent


def test_eviction_is_least_recently_used_leaf_first():
    m = _pool(nb=32)
    c = PrefixCacheModel(m)
    a, b = _prompt(48), _prompt(48, start=500)
    for s, p in ((0, a), (1, b)):
        m.alloc(s)
        m.append([s], [48])
        c.insert(s, p)
    ta, tb = m.table(0), m.table(1)
    m.free_seq(0)
    m.free_seq(1)
    c.alloc_from(2, a)     # uses chain a again: chain b is now the least recently used
    m.free_seq(2)
    assert c.evict(1) == 1
    assert m.free[-1] == tb[2]           # b's deepest block, not b's first block
    assert c.match(b) == 32 and c.match(a) == 48
    assert c.evict(2) == 2
    assert list(m.free)[-2:] == [tb[1], tb[0]]
    assert c.match(a) == 48 and c.match(b) == 0
    assert all(m.refcount(x) == 1 for x in ta)


def test_shared_prompt_branches_keep_their_common_blocks():
    m = _pool(nb=32)
    c = PrefixCacheModel(m)
    a = _prompt(48)
    b = a[:32] + _prompt(16, start=900)   # same first two blocks, different third
    m.alloc(0)
    m.append([0], [48])
    c.insert(0, a)
    assert c.alloc_from(1, b) == 32
    m.append([1], [16])
    assert c.insert(1, b) == 1            # only the new third block
    assert c.evict(1) == 1                # a leaf: a's or b's third block, never a shared one
    assert c.match(a[:32]) == 32 and c.match(b[:32]) == 32


def test_writing_into_a_cached_block_copies_it():
    m = PoolModel(8, 1, 64, "bf16", 4, 4, track_data=True)
    c = PrefixCacheModel(m)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 2 ** 15, size=(32, 1, 64)).astype(np.uint16)
    m.alloc(0)
    m.append([0], [32], rows, rows)
    a = _prompt(32)
    c.insert(0, a)
    cached = m.table(0)[1]
    m.truncate(0, 20)                      # back into the second (cached, full) block
    new = rng.integers(0, 2 ** 15, size=(1, 1, 64)).astype(np.uint16)
    m.append([0], [1], new, new)
    assert m.table(0)[1] != cached         # copied before the write
    c.alloc_from(1, a)
    k, _ = m.gather(1)
    assert np.array_equal(k, rows)         # the cached rows are intact


def test_errors():
    m = _pool()
    c = PrefixCacheModel(m)
    with pytest.raises(InvalidError):
        c.insert(0, _prompt(16))           # not live
    m.alloc(0)
    with pytest.raises(InvalidError):
        c.alloc_from(0, _prompt(16))       # already live
    with pytest.raises(InvalidError):
        c.evict(-1)
