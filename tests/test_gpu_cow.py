"""GPU: copy-on-write copies and row writes into the same block in one call.

A longer sharer of a partly filled block copies its filled slots [0, off) to a
fresh block and drops its reference; a shorter sharer served later in the same
append then holds the block alone and writes its new rows straight into it,
at slots below the copier's off.  The oracle's model serves the sequences one
after the other, so the copy takes the slots as they were before the call.
Pools, tables and outputs must match the model bit for bit / within tolerance,
through pa_append_kv and through pa_append_attend (which falls back to separate
launches when a copy is needed).

Copy-on-write sharing of blocks among sequences of one prompt: "PagedAttention,
décodage spéculatif, MoE et Blackwell", section 1; kenji.blog
"llm-inference-optimization-kv-cache", section 4.2.
"""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch
from workloads import make_custom
from workloads.synth import _to_storage as to_storage

pytestmark = pytest.mark.gpu


def _rows(rng, n, hkv, d, dtype):
    return to_storage(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)


def _setup(how, dtype):
    # parent (seq 0) holds 20 tokens: block 0 full, block 1 slots 0..3
    w = make_custom(lengths=[20], num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=dtype, seed=60)
    w.max_blocks_per_seq = 8
    pair = Pair(w, max_seqs=4, num_blocks=16, free_order=np.random.default_rng(63).permutation(16))
    pair.fill()
    if how == "fork_shorter":
        pair.alloc(1, 0, 17)           # shares both blocks, length 17 (block 1 slot 0 valid)
    elif how == "truncated_fork":
        pair.alloc(1, 0, 20)
        pair.truncate(1, 17)           # still shares block 1 (refcount 2)
    elif how == "two_children":
        pair.alloc(1, 0, 17)
        pair.alloc(2, 0, 18)           # block 1 referenced three times
    return w, pair


@pytest.mark.parametrize("how,order,n_tok", [
    ("fork_shorter", [0, 1], [1, 1]),
    ("fork_shorter", [0, 1], [1, 3]),     # the child writes slots 1..3, all below the parent's copy of 0..3
    ("truncated_fork", [0, 1], [2, 1]),
    ("two_children", [0, 2, 1], [1, 1, 2]),
    ("fork_shorter", [1, 0], [1, 1]),     # child first: it copies [0, 1), the parent then writes slot 4
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_source_written_by_a_later_sharer(how, order, n_tok, dtype):
    print(f"cow race {how} order={order} n_tok={n_tok} {dtype}", flush=True)
    w, pair = _setup(how, dtype)
    rng = np.random.default_rng(61)
    total = int(sum(n_tok))
    k = _rows(rng, total, w.num_kv_heads, w.head_dim, dtype)
    v = _rows(rng, total, w.num_kv_heads, w.head_dim, dtype)
    pair.append(order, n_tok, k, v)
    pair.check_pools_and_tables()
    seqs = sorted(order)
    q_bits = to_storage(rng.standard_normal((len(seqs), 1, w.num_q_heads, w.head_dim), dtype=np.float32), dtype)
    q = to_torch(q_bits, dtype).reshape(len(seqs), w.num_q_heads, w.head_dim).contiguous()
    out, lse = pair.gpu.decode(seqs, q, w.scale)
    ro, rl = oracle_decode(pair, seqs, q_bits, w.scale)
    assert_close(out[:, None], lse[:, None], ro, rl, dtype, f"decode after {how}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_append_attend_copy_source_written(dtype):
    """The same hazard through pa_append_attend: parent and a shorter fork each
    append one row and decode in one call."""
    print(f"cow race append_attend {dtype}", flush=True)
    w, pair = _setup("fork_shorter", dtype)
    rng = np.random.default_rng(62)
    k = _rows(rng, 2, w.num_kv_heads, w.head_dim, dtype)
    v = _rows(rng, 2, w.num_kv_heads, w.head_dim, dtype)
    q_bits = to_storage(rng.standard_normal((2, 1, w.num_q_heads, w.head_dim), dtype=np.float32), dtype)
    out, lse = pair.gpu.append_attend([0, 1], to_torch(k, dtype), to_torch(v, dtype),
                                      to_torch(q_bits, dtype).contiguous(), w.scale)
    pair.model.append([0, 1], [1, 1], k, v)
    pair.check_pools_and_tables()
    ro, rl = oracle_decode(pair, [0, 1], q_bits, w.scale)
    assert_close(out, lse, ro, rl, dtype, "append_attend after fork at a shorter length")
