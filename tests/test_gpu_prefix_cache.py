"""GPU parity of prompts reusing cached prefix blocks: sequences started from
the prefix cache attend over the reused blocks plus their own rows exactly as
the oracle does, and a write into a reused block copies it first, leaving the
cached rows intact."""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch
from oracle.prefix_cache import PrefixCacheModel
from workloads import make_custom
from workloads.synth import _to_storage as to_storage

pytestmark = pytest.mark.gpu


def _rows(rng, n, w):
    shape = (n, w.num_kv_heads, w.head_dim)
    return (to_storage(rng.standard_normal(shape, dtype=np.float32), w.dtype),
            to_storage(rng.standard_normal(shape, dtype=np.float32), w.dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prompts_from_the_prefix_cache(dtype):
    w = make_custom(lengths=[300], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype=dtype, seed=90)
    pair = Pair(w, max_seqs=8, num_blocks=200, free_order=np.random.default_rng(2).permutation(200))
    cache = PrefixCacheModel(pair.model)
    rng = np.random.default_rng(91)
    prompt = [int(x) for x in rng.integers(0, 50000, size=300)]
    pair.fill()                                   # sequence 0 holds the 300-token prompt
    assert pair.gpu.prefix_insert(0, prompt) == cache.insert(0, prompt) == 18
    pair.truncate(0, 290)                         # its own decode continues elsewhere
    # three later prompts: the same one, one diverging at token 100, one at token 0
    variants = [prompt + [7, 8, 9], prompt[:100] + [1] * 60, [5] + prompt[1:]]
    for s, p in zip((1, 2, 3), variants):
        m = pair.gpu.alloc_from_prefix(s, p)
        assert m == cache.alloc_from(s, p) == {1: 288, 2: 96, 3: 0}[s]
        k, v = _rows(rng, len(p) - m, w)
        pair.append([s], [len(p) - m], k, v)
    pair.check_pools_and_tables()
    seqs = [0, 1, 2, 3]
    q_bits = to_storage(rng.standard_normal((4, 1, w.num_q_heads, w.head_dim), dtype=np.float32), dtype)
    q = to_torch(q_bits, dtype).reshape(4, w.num_q_heads, w.head_dim).contiguous()
    out, lse = pair.gpu.decode(seqs, q, w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, seqs, q_bits, w.scale)
    assert_close(out[:, None], lse[:, None], ro, rl, dtype, "prompts from the prefix cache")
    # a write into a reused block copies it; the cache still serves the old rows
    pair.truncate(1, 40)
    k, v = _rows(rng, 1, w)
    pair.append([1], [1], k, v)
    pair.gpu.free(2)
    pair.model.free_seq(2)
    assert pair.gpu.alloc_from_prefix(2, prompt) == cache.alloc_from(2, prompt) == 288
    pair.gpu.sync_tables()                        # host-side call: the mirror follows on the next device call
    pair.check_pools_and_tables()
    out, lse = pair.gpu.decode([1, 2], q[:2].contiguous(), w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(pair, [1, 2], q_bits[:2], w.scale)
    assert_close(out[:, None], lse[:, None], ro, rl, dtype, "after a copy-on-write of a cached block")
    # evicting the whole cache returns every block nobody else holds
    for s in (0, 1, 2, 3):
        pair.gpu.free(s)
        pair.model.free_seq(s)
    assert pair.gpu.prefix_evict(1000) == cache.evict(1000)
    pair.gpu.sync_tables()
    pair.check_tables()
    assert pair.gpu.num_free() == 200
