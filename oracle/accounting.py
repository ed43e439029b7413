"""Byte accounting the pages state (oracle; test infrastructure only).

  kv_cache_bytes        [P2] section 3.2: memory = 2 (K and V) x batch x sequence
                        length x layers x heads x head dim x bytes per value
  bandwidth_bound_time  [P2] section 2.3: moving B bytes at W bytes/s takes B / W
                        seconds; 140 GB at 2 TB/s is 0.07 s, about 14 tokens/s
  contiguous_unused     [P1] section 1: a 32,768-token reservation of which 200
                        are used leaves more than 99 % empty
  paged_unused_slots    [P2] section 4.2: allocating only the blocks needed leaves
                        fewer than one block of slots unused per sequence
  decode_step_bytes     the bytes one paged decode step must move at least: every
                        cached K and V row of every key/value head once, the
                        queries, the outputs and the block-table entries used
"""
from __future__ import annotations

import math

BLOCK = 16


def kv_cache_bytes(batch: int, seq_len: int, layers: int, heads: int, head_dim: int,
                   bytes_per_value: int) -> int:
    return 2 * batch * seq_len * layers * heads * head_dim * bytes_per_value


def bandwidth_bound_time(num_bytes: float, bytes_per_second: float) -> float:
    return num_bytes / bytes_per_second


def contiguous_unused(used_tokens: int, reserved_tokens: int) -> float:
    return 1.0 - used_tokens / reserved_tokens


def paged_unused_slots(length: int, block: int = BLOCK) -> int:
    return math.ceil(length / block) * block - length


def decode_step_bytes(lengths, num_kv_heads: int, num_q_heads: int, head_dim: int,
                      elem_bytes: int, k_draft: int = 1, shared_prefix_tokens: int = 0) -> int:
    """Minimum HBM bytes of one decode (or verify) launch.

    K and V rows: sum over sequences of the rows it holds, with a shared prefix
    counted once; Q read and O written once per query row; one 4-byte table
    entry per block used and one 4-byte length per sequence.
    """
    lengths = [int(n) for n in lengths]
    rows = sum(n - shared_prefix_tokens for n in lengths) + (shared_prefix_tokens if lengths else 0)
    kv = rows * num_kv_heads * head_dim * elem_bytes * 2
    qo = 2 * len(lengths) * k_draft * num_q_heads * head_dim * elem_bytes
    table = sum(math.ceil(n / BLOCK) for n in lengths) * 4 + 4 * len(lengths)
    return kv + qo + table


def append_bytes(total_rows: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Rows read from the caller's buffers and written into the pool, plus one
    4-byte slot index per row."""
    return 2 * 2 * total_rows * num_kv_heads * head_dim * elem_bytes + 4 * total_rows
