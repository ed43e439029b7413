"""Block-pool model (oracle; test infrastructure only).

What it models, from the pages:
  * the KV cache of each sequence is cut into fixed-size blocks of 16 tokens that
    can sit anywhere in the physical pool; a block table maps logical blocks to
    physical ones ([P1] section 1; [P2] section 4.1);
  * only the blocks a sequence needs are allocated, so at most 15 slots per
    sequence are unused ([P2] section 4.2);
  * sequences derived from the same prompt point to the same physical blocks
    and are copied only on write ([P1] section 1; [P2] section 4.2);
  * a rejected speculative draft is discarded and generation restarts at the
    first error ([P2] section 5.2; [P4] "Spéculer"), i.e. the cache is cut back
    to the accepted prefix (``truncate``).

Where the pages are silent this model takes one plain reading, which the library
implements identically so that block tables can be compared bit-exactly:
  * free list = a deque seeded with a caller-given order; allocation pops the
    front, release pushes to the back, in increasing logical block order;
  * a block is copied lazily: only when a token is written into a block whose
    reference count exceeds one; the copy takes the slots already filled;
  * the sequences of one append call are served in the order given, each one
    token after the other;
  * an append that cannot get every block it needs fails and changes nothing.

The model also keeps the exact bytes of the K and V pools (in the layout of
``oracle.layout``) so that tests can compare the pool written by the GPU byte by
byte, including slots that must still hold the fill pattern.
"""
from __future__ import annotations

import copy
from collections import deque
from typing import Dict, List, Optional

import numpy as np

from . import layout
from .numerics import BITS_DTYPE, as_bits

BLOCK = layout.BLOCK


class PaError(Exception):
    code = -1


class InvalidError(PaError):
    code = -1


class NoMemError(PaError):
    code = -2


class StateError(PaError):
    code = -4


class PoolModel:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
                 max_seqs: int, max_blocks_per_seq: int, free_order=None,
                 sentinel_bits: int = 0, track_data: bool = True, kv_scales=None):
        if num_blocks <= 0 or num_kv_heads <= 0 or head_dim <= 0:
            raise InvalidError("sizes must be positive")
        if free_order is None:
            free_order = np.arange(num_blocks)
        free_order = [int(b) for b in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise InvalidError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.hkv = num_kv_heads
        self.d = head_dim
        self.dtype = dtype
        # 'fp8' pools: rows arrive as bf16 bits and are stored as E4M3 codes of
        # row * (1 / scale) per kv head, the reciprocal and product in float32
        if kv_scales is None:
            kv_scales = (np.ones(num_kv_heads, np.float32), np.ones(num_kv_heads, np.float32))
        self.k_scale = np.asarray(kv_scales[0], np.float32)
        self.v_scale = np.asarray(kv_scales[1], np.float32)
        self.max_seqs = max_seqs
        self.max_blocks = max_blocks_per_seq
        self.free: deque = deque(free_order)
        self.rc: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.track_data = track_data
        if track_data:
            bits = BITS_DTYPE[dtype]
            self.kpool = np.full(layout.k_shape(num_blocks, num_kv_heads, head_dim, dtype),
                                 sentinel_bits, dtype=bits)
            self.vpool = np.full(layout.v_shape(num_blocks, num_kv_heads, head_dim, dtype),
                                 sentinel_bits, dtype=bits)

    # ---- queries -------------------------------------------------------------
    def live(self, seq: int) -> bool:
        return seq in self.lens

    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lens[seq]

    def refcount(self, block: int) -> int:
        return self.rc[block]

    def num_free(self) -> int:
        return len(self.free)

    # ---- operations ----------------------------------------------------------
    def _pop(self) -> int:
        if not self.free:
            raise NoMemError("pool exhausted")
        b = self.free.popleft()
        assert self.rc[b] == 0
        self.rc[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.rc[b] -= 1
        assert self.rc[b] >= 0
        if self.rc[b] == 0:
            self.free.append(b)

    def _check_seq_id(self, seq: int) -> None:
        if not (0 <= seq < self.max_seqs):
            raise InvalidError(f"seq id {seq} out of range")

    def alloc(self, seq: int, parent: int = -1, shared_tokens: int = 0) -> None:
        """Create ``seq``; with a parent, share its first ceil(shared/16) blocks."""
        self._check_seq_id(seq)
        if self.live(seq):
            raise InvalidError(f"seq {seq} already exists")
        if parent < 0:
            if shared_tokens != 0:
                raise InvalidError("shared_tokens needs a parent")
            self.tables[seq] = []
            self.lens[seq] = 0
            return
        if not self.live(parent):
            raise InvalidError(f"parent {parent} does not exist")
        if not (0 <= shared_tokens <= self.lens[parent]):
            raise InvalidError("shared_tokens out of range")
        nb = (shared_tokens + BLOCK - 1) // BLOCK
        shared = self.tables[parent][:nb]
        for b in shared:
            self.rc[b] += 1
        self.tables[seq] = list(shared)
        self.lens[seq] = shared_tokens

    def _append_one(self, seq: int, k_row: Optional[np.ndarray], v_row: Optional[np.ndarray]) -> None:
        t = self.lens[seq]
        off = t % BLOCK
        tab = self.tables[seq]
        if off == 0:
            tab.append(self._pop())
        elif self.rc[tab[-1]] > 1:
            old = tab[-1]
            new = self._pop()
            if self.track_data:
                layout.copy_rows(self.kpool, self.vpool, old, new, off)
            self._release(old)
            tab[-1] = new
        if self.track_data:
            if self.dtype == "fp8":
                k_code, v_code = self._quantize(k_row, self.k_scale), self._quantize(v_row, self.v_scale)
            else:
                k_code, v_code = as_bits(k_row, self.dtype), as_bits(v_row, self.dtype)
            layout.write_row(self.kpool, self.vpool, tab[-1], off, k_code, v_code, self.dtype)
        self.lens[seq] = t + 1

    @staticmethod
    def _quantize(row_bf16: np.ndarray, scale: np.ndarray, bulk: bool = False) -> np.ndarray:
        """E4M3 codes of bf16 rows [..., Hkv, D]: E4M3(x * (1 / scale[h])).
        ``bulk`` takes the search encoder (the same codes, for whole caches)."""
        from .fp8 import encode, encode_by_search
        x = (as_bits(row_bf16, "bf16").astype(np.uint32) << np.uint32(16)).view(np.float32)
        inv = (np.float32(1.0) / scale.astype(np.float32)).astype(np.float32)
        return (encode_by_search if bulk else encode)((x * inv[:, None]).astype(np.float32))

    def append(self, seq_ids, n_tok, k_rows=None, v_rows=None) -> None:
        """Append n_tok[i] rows to seq_ids[i]; rows are packed in call order
        ([sum(n_tok), Hkv, D]).  All-or-nothing on pool exhaustion."""
        seq_ids = [int(s) for s in seq_ids]
        n_tok = [int(n) for n in n_tok]
        if len(n_tok) != len(seq_ids):
            raise InvalidError("one token count per sequence")
        if len(set(seq_ids)) != len(seq_ids):
            raise InvalidError("duplicate sequence in one append")
        for s, n in zip(seq_ids, n_tok):
            self._check_seq_id(s)
            if not self.live(s):
                raise InvalidError(f"seq {s} does not exist")
            if n < 0:
                raise InvalidError("negative token count")
            if self.lens[s] + n > self.max_blocks * BLOCK:
                raise InvalidError("sequence would exceed max_blocks_per_seq")
        saved = (copy.deepcopy(self.free), list(self.rc), copy.deepcopy(self.tables),
                 dict(self.lens))
        saved_pools = None
        if self.track_data:
            saved_pools = (self.kpool.copy(), self.vpool.copy())
        try:
            r = 0
            for s, n in zip(seq_ids, n_tok):
                for _ in range(n):
                    kr = k_rows[r] if self.track_data else None
                    vr = v_rows[r] if self.track_data else None
                    self._append_one(s, kr, vr)
                    r += 1
        except NoMemError:
            self.free, self.rc, self.tables, self.lens = saved
            if saved_pools is not None:
                self.kpool, self.vpool = saved_pools
            raise

    def truncate(self, seq: int, new_len: int) -> None:
        """Cut ``seq`` back to ``new_len`` tokens, releasing blocks it no longer needs."""
        self._check_seq_id(seq)
        if not self.live(seq):
            raise InvalidError(f"seq {seq} does not exist")
        if not (0 <= new_len <= self.lens[seq]):
            raise InvalidError("new_len out of range")
        keep = (new_len + BLOCK - 1) // BLOCK
        tab = self.tables[seq]
        for b in tab[keep:]:
            self._release(b)
        del tab[keep:]
        self.lens[seq] = new_len

    def free_seq(self, seq: int) -> None:
        self.truncate(seq, 0)
        del self.tables[seq]
        del self.lens[seq]

    # ---- swap to host memory -------------------------------------------------
    # A KV cache short of GPU memory can move a sequence's blocks to host RAM
    # and bring them back later ([P4] "Mettre en cache", tiers G1 / G2).  Here
    # swapping out keeps the sequence's rows (stored codes, bit for bit) and
    # ends it; swapping in starts a sequence and writes those rows into blocks
    # taken as an append of that many rows would take them.
    def swap_out(self, seq: int):
        """Rows of ``seq`` as stored ([n, Hkv, D] bit patterns); ``seq`` ends."""
        if not self.live(seq):
            raise InvalidError(f"seq {seq} does not exist")
        k, v = self.gather(seq) if self.track_data else (None, None)
        n = self.lens[seq]
        self.free_seq(seq)
        return n, k, v

    def swap_in(self, seq: int, n: int, k_bits=None, v_bits=None) -> None:
        """Start ``seq`` with ``n`` rows given as stored bit patterns."""
        self._check_seq_id(seq)
        if self.live(seq):
            raise InvalidError(f"seq {seq} already exists")
        if n < 0:
            raise InvalidError("length < 0")
        if (n + BLOCK - 1) // BLOCK > self.max_blocks:
            raise InvalidError("longer than a block table")
        if (n + BLOCK - 1) // BLOCK > len(self.free):
            raise NoMemError("pool exhausted")
        self.tables[seq] = []
        self.lens[seq] = 0
        for t in range(n):
            if t % BLOCK == 0:
                self.tables[seq].append(self._pop())
            if self.track_data:
                layout.write_row(self.kpool, self.vpool, self.tables[seq][-1], t % BLOCK, k_bits[t], v_bits[t],
                                 self.dtype)
            self.lens[seq] = t + 1

    # ---- views for comparison -----------------------------------------------
    def gather(self, seq: int):
        """Logical K, V rows of ``seq`` ([n, Hkv, D] bit patterns), read through
        its block table."""
        n = self.lens[seq]
        tab = self.tables[seq]
        ks, vs = [], []
        for t in range(n):
            k, v = layout.read_row(self.kpool, self.vpool, tab[t // BLOCK], t % BLOCK, self.dtype)
            ks.append(k)
            vs.append(v)
        bits = BITS_DTYPE[self.dtype]
        if not ks:
            e = np.zeros((0, self.hkv, self.d), dtype=bits)
            return e, e.copy()
        return np.stack(ks), np.stack(vs)
