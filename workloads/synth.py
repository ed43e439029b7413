"""Seeded synthetic workloads for paged KV-cache decode and speculative verify.

Every array is drawn from one ``numpy.random.default_rng(seed)`` in a fixed
order so that the GPU path and the oracle see byte-identical inputs:

    lengths -> free_order -> (shared prefix rows) -> per-sequence K, V rows
    -> appended rows (K then V) -> queries -> (second-phase queries)

Values are N(0, 1) drawn in float32 and rounded to the storage dtype with
round-to-nearest-even ('f16' through numpy, 'bf16' through torch's CPU cast,
kept as raw uint16 bit patterns because numpy has no bfloat16).

The shapes follow the workloads the pages motivate: 16-token blocks placed
anywhere in a physical pool (page "PagedAttention, décodage spéculatif, MoE et
Blackwell", section 1), decode that reads the whole cache every step (page
"CUDA Graphs, modèles de raisonnement et service désagrégé", section 3 table),
and K draft tokens verified in one pass (kenji.blog page
"llm-inference-optimization-kv-cache", section 5.2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
_ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
BLOCK_SIZE = 16


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return the uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _to_storage(rng.standard_normal(size=shape, dtype=np.float32), dtype)


@dataclass
class Workload:
    """One seeded workload.

    mode:
      'decode'         cache holds ``lengths`` tokens, one query per sequence.
      'append_decode'  append ``new_k/new_v`` (1 row per sequence), then decode
                       over the grown cache.
      'decode_append'  decode with ``q``, append ``new_k/new_v``, decode again
                       with ``q2``.
      'verify'         sequences share a ``prefix_len``-token prefix (copy-on-
                       write forks of sequence 0), then hold private suffix
                       rows, then ``k_draft`` draft rows are appended and the
                       ``k_draft`` queries per sequence are verified causally.
    """

    name: str
    mode: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    free_order: np.ndarray
    lengths: np.ndarray               # private rows per sequence (suffix for 'verify')
    k_rows: List[np.ndarray]          # [n_s, Hkv, D] per sequence, storage dtype
    v_rows: List[np.ndarray]
    q: np.ndarray                     # [B, k_draft, Hq, D]
    scale: float
    k_draft: int = 1
    new_k: Optional[np.ndarray] = None   # [B, T_new, Hkv, D]
    new_v: Optional[np.ndarray] = None
    q2: Optional[np.ndarray] = None      # second-phase queries for 'decode_append'
    prefix_len: int = 0
    prefix_k: Optional[np.ndarray] = None  # [prefix_len, Hkv, D]
    prefix_v: Optional[np.ndarray] = None
    partition_tokens: int = 0
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.lengths))

    @property
    def elem_bytes(self) -> int:
        return _ELEM_BYTES[self.dtype]

    @property
    def block_size(self) -> int:
        return BLOCK_SIZE

    def final_lengths(self) -> np.ndarray:
        """Tokens each sequence holds when the attention phase runs."""
        n = self.lengths.astype(np.int64) + self.prefix_len
        if self.new_k is not None and self.mode in ("append_decode", "verify"):
            n = n + self.new_k.shape[1]
        return n


def _pool_size(blocks_needed: int, factor: float = 1.25) -> int:
    return int(math.ceil(factor * blocks_needed))


def _blocks(n) -> int:
    return int(np.sum((np.asarray(n, dtype=np.int64) + BLOCK_SIZE - 1) // BLOCK_SIZE))


def _rows_per_seq(rng, lengths, hkv, d, dtype):
    k_rows, v_rows = [], []
    for n in lengths:
        k_rows.append(_normal(rng, (int(n), hkv, d), dtype))
        v_rows.append(_normal(rng, (int(n), hkv, d), dtype))
    return k_rows, v_rows


def make_custom(
    *,
    name: str = "custom",
    mode: str = "decode",
    lengths,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str,
    seed: int,
    k_draft: int = 1,
    num_blocks: Optional[int] = None,
    pool_factor: float = 1.25,
    partition_tokens: int = 0,
    scale: Optional[float] = None,
    prefix_len: int = 0,
    lengths_fn=None,
) -> Workload:
    """General seeded generator; the named configurations below call it.

    ``lengths`` is either an explicit integer sequence or, when ``lengths_fn``
    is given, the batch size passed to ``lengths_fn(rng, batch)``.
    """
    assert dtype in DTYPES
    rng = np.random.default_rng(seed)
    if lengths_fn is not None:
        lengths = np.asarray(lengths_fn(rng, int(lengths)), dtype=np.int64)
    else:
        lengths = np.asarray(lengths, dtype=np.int64)
    b = len(lengths)
    hkv, d = num_kv_heads, head_dim
    t_new = 0
    if mode in ("append_decode", "decode_append"):
        t_new = 1
    elif mode == "verify":
        t_new = k_draft
    final = lengths + prefix_len + (t_new if mode in ("append_decode", "verify") else 0)
    if mode == "decode_append":
        final = lengths + t_new
    if mode == "verify" and prefix_len:
        # prefix blocks are stored once; each sequence owns its tail blocks
        prefix_blocks = (prefix_len + BLOCK_SIZE - 1) // BLOCK_SIZE
        own = _blocks(final) - b * prefix_blocks
        need = prefix_blocks + own + (b if prefix_len % BLOCK_SIZE else 0)
    else:
        need = _blocks(final)
    if num_blocks is None:
        num_blocks = _pool_size(need, pool_factor)
    max_blocks_per_seq = int((int(final.max(initial=1)) + BLOCK_SIZE - 1) // BLOCK_SIZE)
    free_order = rng.permutation(num_blocks).astype(np.int32)
    prefix_k = prefix_v = None
    if prefix_len:
        prefix_k = _normal(rng, (prefix_len, hkv, d), dtype)
        prefix_v = _normal(rng, (prefix_len, hkv, d), dtype)
    k_rows, v_rows = _rows_per_seq(rng, lengths, hkv, d, dtype)
    new_k = new_v = None
    if t_new:
        new_k = _normal(rng, (b, t_new, hkv, d), dtype)
        new_v = _normal(rng, (b, t_new, hkv, d), dtype)
    q = _normal(rng, (b, k_draft, num_q_heads, d), dtype)
    q2 = None
    if mode == "decode_append":
        q2 = _normal(rng, (b, 1, num_q_heads, d), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Workload(
        name=name, mode=mode, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=hkv,
        head_dim=d, num_blocks=int(num_blocks), max_blocks_per_seq=max_blocks_per_seq,
        free_order=free_order, lengths=lengths, k_rows=k_rows, v_rows=v_rows, q=q,
        scale=float(scale), k_draft=k_draft, new_k=new_k, new_v=new_v, q2=q2,
        prefix_len=prefix_len, prefix_k=prefix_k, prefix_v=prefix_v,
        partition_tokens=partition_tokens, seed=seed,
    )


# ---- the named workloads -------------------------------------------------

def make_tiny(seed: int = 1) -> Workload:
    """4 sequences of {17, 33, 64, 100} tokens, 4 heads (no grouping), D=64, fp32,
    a 64-block pool; decode, append one row per sequence, decode again."""
    return make_custom(
        name="tiny", mode="decode_append", lengths=[17, 33, 64, 100], num_q_heads=4,
        num_kv_heads=4, head_dim=64, dtype="f32", seed=seed, num_blocks=64,
        scale=1.0 / 8.0,
    )


def _uniform_lengths(lo, hi):
    return lambda rng, b: rng.integers(lo, hi + 1, size=b)


def _lognormal_lengths(median, sigma, lo, hi):
    def f(rng, b):
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=b)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return f


def make_gqa70b(seed: int = 2, batch: int = 32) -> Workload:
    """70B-like grouped-query layer: lengths U[512, 4096], 64 query heads over
    8 KV heads, D=128, fp16, pool of 1.25x the blocks needed."""
    return make_custom(
        name="gqa70b", mode="decode", lengths=batch, lengths_fn=_uniform_lengths(512, 4096),
        num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="f16", seed=seed,
    )


def make_highbatch(seed: int = 3, batch: int = 256) -> Workload:
    """High-batch short contexts: 256 sequences, log-normal lengths (median 200,
    sigma 1, clipped to [16, 2048]), 32 query / 8 KV heads, D=128, bf16; each step
    appends one row per sequence, then decodes."""
    return make_custom(
        name="highbatch", mode="append_decode", lengths=batch,
        lengths_fn=_lognormal_lengths(200, 1.0, 16, 2048), num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", seed=seed,
    )


def make_long(seed: int = 4, batch: int = 8, length: int = 32768) -> Workload:
    """Long contexts: 8 sequences of 32,768 tokens, 32 query / 8 KV heads, D=128,
    fp16, split into 512-token partitions merged by log-sum-exp."""
    return make_custom(
        name="long", mode="decode", lengths=[length] * batch, num_q_heads=32,
        num_kv_heads=8, head_dim=128, dtype="f16", seed=seed, partition_tokens=512,
    )


def make_verify(seed: int = 5, batch: int = 64, prefix_len: int = 4096,
                k_draft: int = 5) -> Workload:
    """Shared prefix + speculative verify: 64 sequences share a 4,096-token
    copy-on-write prefix, then private suffixes U[16, 512], then 5 drafts each;
    32 query / 8 KV heads, D=128, bf16."""
    return make_custom(
        name="verify", mode="verify", lengths=batch, lengths_fn=_uniform_lengths(16, 512),
        num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=seed,
        k_draft=k_draft, prefix_len=prefix_len,
    )


def make_prefill(seed: int = 6, batch: int = 4, cached: int = 8192, chunk: int = 512) -> Workload:
    """Chunked prefill of long prompts: 4 sequences hold 8,192 prompt tokens
    from earlier chunks and take their next 512-token chunk (each chunk token
    attends causally); 32 query / 8 KV heads, D=128, bf16."""
    return make_custom(
        name="prefill", mode="verify", lengths=[cached] * batch, num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", seed=seed, k_draft=chunk,
    )


def by_name(name: str, **kw) -> Workload:
    table = {
        "tiny": make_tiny, "gqa70b": make_gqa70b, "highbatch": make_highbatch,
        "long": make_long, "verify": make_verify, "prefill": make_prefill,
    }
    return table[name](**kw)


# ---- inputs whose scores grow along the sequence -----------------------------

def _storage_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float32 (bf16 bit patterns widened, f16 / f32 cast)."""
    if dtype == "bf16":
        return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(bits).astype(np.float32)


def with_rising_scores(w: Workload, every: int, offsets=(40, 100), gains=(1.0, 2.5), v_gain: float = 0.5,
                       query_head: int = 0, new_row_gain: Optional[float] = None) -> Workload:
    """A copy of ``w`` whose key rows make some query rows' largest score grow
    well after the start of every ``every``-token span of each sequence.

    At logical position ``b + offsets[j]`` (b a multiple of ``every``, the
    position inside the sequence: shared prefix, then private rows, then the
    appended rows) the key row of every kv head is set to ``gains[j]`` times
    the sequence's first query of head ``kvh * G + query_head``; the spans of
    the shared prefix take sequence 0's query.  Every value row is multiplied
    by ``v_gain`` so that outputs stay well inside the output type's range.
    With ``new_row_gain``, the last appended row of each sequence gets that
    gain instead (a rise at the very end of the sequence).  All new values are
    rounded to the storage type as the generator does.
    """
    import copy

    out = copy.deepcopy(w)
    g = w.num_q_heads // w.num_kv_heads
    d = w.dtype
    qf = _storage_to_f32(w.q, d)  # [B, K, Hq, D]

    def plant(rows: np.ndarray, start: int, seq: int) -> np.ndarray:
        """rows [n, Hkv, D] at logical positions start .. start + n - 1."""
        if rows is None or rows.shape[0] == 0:
            return rows
        f = _storage_to_f32(rows, d).copy()
        n = f.shape[0]
        for b in range(0, start + n, every):
            for off, gain in zip(offsets, gains):
                pos = b + off
                if start <= pos < start + n and off < every:
                    for kvh in range(w.num_kv_heads):
                        f[pos - start, kvh] = np.float32(gain) * qf[seq, 0, kvh * g + query_head]
        return _to_storage(f, d)

    def shrink(rows: np.ndarray) -> np.ndarray:
        if rows is None or rows.shape[0] == 0:
            return rows
        return _to_storage(_storage_to_f32(rows, d) * np.float32(v_gain), d)

    if w.prefix_len:
        out.prefix_k = plant(w.prefix_k, 0, 0)
        out.prefix_v = shrink(w.prefix_v)
    for s in range(w.batch):
        out.k_rows[s] = plant(w.k_rows[s], w.prefix_len, s)
        out.v_rows[s] = shrink(w.v_rows[s])
    if w.new_k is not None:
        nk, nv = out.new_k.copy(), out.new_v.copy()
        for s in range(w.batch):
            nk[s] = plant(w.new_k[s], w.prefix_len + int(w.lengths[s]), s)
            nv[s] = shrink(w.new_v[s])
            if new_row_gain is not None:
                f = _storage_to_f32(nk[s], d).copy()
                for kvh in range(w.num_kv_heads):
                    f[-1, kvh] = np.float32(new_row_gain) * qf[s, 0, kvh * g + query_head]
                nk[s] = _to_storage(f, d)
        out.new_k, out.new_v = nk, nv
    out.name = w.name + "_rising"
    return out
