"""PagedKVCache: torch tensors for device memory, every operation through the C ABI.

PyTorch provides the device buffers (pools, block table, lengths, queries,
outputs, workspace) and the current stream; the block bookkeeping, the row
scatter and the attention all run in libpa.so (host allocator + gfx950 kernels).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import abi

# "fp8": pools of E4M3 codes (uint8 tensors); rows, queries and outputs are bf16
TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.bfloat16}
POOL_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.uint8}
PA_DTYPES = {"f32": abi.PA_F32, "f16": abi.PA_F16, "bf16": abi.PA_BF16, "fp8": abi.PA_FP8_E4M3}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
BLOCK = 16


def k_pool_shape(num_blocks: int, hkv: int, d: int, dtype: str):
    x = 16 // ELEM_BYTES[dtype]
    return (num_blocks, hkv, d // x, BLOCK, x)


def v_pool_shape(num_blocks: int, hkv: int, d: int, dtype: str):
    return (num_blocks, hkv, d, BLOCK)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class PagedKVCache:
    """One physical K/V pool with its block tables.

    fill_bits: optional integer bit pattern written into every pool element at
    creation (tests use a NaN pattern to show that unused slots are never read
    into results and never overwritten).
    """

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str, max_seqs: int,
                 max_blocks_per_seq: int, free_order: Optional[Sequence[int]] = None,
                 device: str = "cuda", fill_bits: Optional[int] = None, host_only: bool = False):
        self.lib = abi.load()
        self.num_blocks, self.hkv, self.d, self.dtype = num_blocks, num_kv_heads, head_dim, dtype
        self.max_seqs, self.max_blocks = max_seqs, max_blocks_per_seq
        self.tdtype = TORCH_DTYPES[dtype]
        self.host_only = host_only
        if host_only:
            self.k_pool = self.v_pool = self.block_table = self.seq_len = None
        else:
            self.k_pool = torch.empty(k_pool_shape(num_blocks, num_kv_heads, head_dim, dtype),
                                      dtype=POOL_DTYPES[dtype], device=device)
            self.v_pool = torch.empty(v_pool_shape(num_blocks, num_kv_heads, head_dim, dtype),
                                      dtype=POOL_DTYPES[dtype], device=device)
            if fill_bits is not None:
                ibits = {4: torch.int32, 2: torch.int16, 1: torch.int8}[ELEM_BYTES[dtype]]
                val = int(fill_bits)
                nbits = 8 * ELEM_BYTES[dtype]
                if val >= 1 << (nbits - 1):
                    val -= 1 << nbits
                self.k_pool.view(ibits).fill_(val)
                self.v_pool.view(ibits).fill_(val)
            self.block_table = torch.full((max_seqs, max_blocks_per_seq), -1, dtype=torch.int32, device=device)
            self.seq_len = torch.zeros((max_seqs,), dtype=torch.int32, device=device)
        order = None
        if free_order is not None:
            order, n = abi.i32_array(free_order)
            if n != num_blocks:
                raise ValueError("free_order must list every block once")
        handle = ctypes.c_void_p()
        abi.check(self.lib.pa_create_pool(
            ctypes.byref(handle), num_blocks, BLOCK, num_kv_heads, head_dim, PA_DTYPES[dtype],
            _ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.block_table), _ptr(self.seq_len),
            max_seqs, max_blocks_per_seq, order))
        self.handle = handle

    def close(self):
        if getattr(self, "handle", None):
            self.lib.pa_destroy_pool(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_kv_scales(self, k_scale: Sequence[float], v_scale: Sequence[float]) -> None:
        """Per-kv-head scales of an "fp8" pool (before the first append)."""
        fa = ctypes.c_float * self.hkv
        abi.check(self.lib.pa_set_kv_scales(self.handle, fa(*[float(x) for x in k_scale]),
                                            fa(*[float(x) for x in v_scale])))

    # ---- block bookkeeping -------------------------------------------------
    def alloc(self, seq: int, parent: int = -1, shared_tokens: int = 0) -> None:
        abi.check(self.lib.pa_alloc_blocks(self.handle, seq, parent, shared_tokens))

    # ---- swap to host ------------------------------------------------------
    def swap_bytes(self, n_tokens: int) -> int:
        out = ctypes.c_size_t()
        abi.check(self.lib.pa_swap_bytes(self.handle, n_tokens, ctypes.byref(out)))
        return out.value

    def swap_out(self, seq: int, k_host: torch.Tensor, v_host: torch.Tensor, stream=None) -> int:
        """Copy ``seq`` into pinned host tensors and end it; returns its length."""
        n = ctypes.c_int()
        nbytes = min(k_host.numel() * k_host.element_size(), v_host.numel() * v_host.element_size())
        abi.check(self.lib.pa_swap_out(self.handle, seq, _ptr(k_host), _ptr(v_host), nbytes, ctypes.byref(n),
                                       _stream(stream)))
        return n.value

    def swap_in(self, seq: int, length: int, k_host: torch.Tensor, v_host: torch.Tensor, stream=None) -> None:
        nbytes = min(k_host.numel() * k_host.element_size(), v_host.numel() * v_host.element_size())
        abi.check(self.lib.pa_swap_in(self.handle, seq, length, _ptr(k_host), _ptr(v_host), nbytes,
                                      _stream(stream)))

    # ---- prefix cache ------------------------------------------------------
    def prefix_insert(self, seq: int, tokens) -> int:
        """Register the full blocks of ``seq`` named by ``tokens``; returns the
        number of newly registered blocks."""
        ids, n = abi.i32_array(tokens)
        out = ctypes.c_int()
        abi.check(self.lib.pa_prefix_insert(self.handle, seq, ids, n, ctypes.byref(out)))
        return out.value

    def prefix_match(self, tokens) -> int:
        ids, n = abi.i32_array(tokens)
        out = ctypes.c_int()
        abi.check(self.lib.pa_prefix_match(self.handle, ids, n, ctypes.byref(out)))
        return out.value

    def alloc_from_prefix(self, seq: int, tokens) -> int:
        """Start ``seq`` on the cached leading blocks of ``tokens``; returns its length."""
        ids, n = abi.i32_array(tokens)
        out = ctypes.c_int()
        abi.check(self.lib.pa_alloc_from_prefix(self.handle, seq, ids, n, ctypes.byref(out)))
        return out.value

    def prefix_evict(self, max_entries: int) -> int:
        out = ctypes.c_int()
        abi.check(self.lib.pa_prefix_evict(self.handle, max_entries, ctypes.byref(out)))
        return out.value

    def prefix_entries(self) -> int:
        out = ctypes.c_int()
        abi.check(self.lib.pa_prefix_entries(self.handle, ctypes.byref(out)))
        return out.value

    def append(self, seq_ids: Sequence[int], n_tok, k_new: Optional[torch.Tensor],
               v_new: Optional[torch.Tensor], stream=None) -> None:
        """k_new / v_new: [sum(n_tok), Hkv, D] device tensors in the pool dtype."""
        ids, n = abi.i32_array(seq_ids)
        if isinstance(n_tok, int):
            n_tok = [n_tok] * n
        toks, m = abi.i32_array(n_tok)
        if m != n:
            raise ValueError("one token count per sequence")
        if k_new is not None:
            self._check_rows(k_new, sum(int(x) for x in n_tok))
            self._check_rows(v_new, sum(int(x) for x in n_tok))
        st = None if self.host_only else _stream(stream)
        abi.check(self.lib.pa_append_kv(self.handle, ids, n, toks, _ptr(k_new), _ptr(v_new), st))

    def _check_rows(self, t: torch.Tensor, rows: int):
        if t.dtype != self.tdtype or not t.is_contiguous() or tuple(t.shape) != (rows, self.hkv, self.d):
            raise ValueError(f"rows must be a contiguous {self.tdtype} tensor of shape {(rows, self.hkv, self.d)}")

    def truncate(self, seq: int, new_len: int) -> None:
        abi.check(self.lib.pa_truncate(self.handle, seq, new_len))

    def truncate_batch(self, seq_ids, new_lens) -> None:
        ids, n = abi.i32_array(seq_ids)
        lens, m = abi.i32_array(new_lens)
        if m != n:
            raise ValueError("one length per sequence")
        abi.check(self.lib.pa_truncate_batch(self.handle, ids, n, lens))

    def free(self, seq: int) -> None:
        abi.check(self.lib.pa_free_seq(self.handle, seq))

    def sync_tables(self, stream=None) -> None:
        abi.check(self.lib.pa_sync_tables(self.handle, None if self.host_only else _stream(stream)))

    def block_table_of(self, seq: int):
        nb, ln = ctypes.c_int(), ctypes.c_int()
        abi.check(self.lib.pa_get_block_table(self.handle, seq, None, 0, ctypes.byref(nb), ctypes.byref(ln)))
        buf = (ctypes.c_int32 * max(1, nb.value))()
        abi.check(self.lib.pa_get_block_table(self.handle, seq, buf, nb.value, ctypes.byref(nb), ctypes.byref(ln)))
        return list(buf[: nb.value]), ln.value

    def length(self, seq: int) -> int:
        return self.block_table_of(seq)[1]

    def refcount(self, block: int) -> int:
        rc = ctypes.c_int()
        abi.check(self.lib.pa_get_refcount(self.handle, block, ctypes.byref(rc)))
        return rc.value

    def num_free(self) -> int:
        n = ctypes.c_int()
        abi.check(self.lib.pa_num_free_blocks(self.handle, ctypes.byref(n)))
        return n.value

    def last_partition(self):
        """(partition tokens, shared-prefix workgroups) of the last attention call."""
        pt, pu = ctypes.c_int(), ctypes.c_int()
        abi.check(self.lib.pa_last_partition(self.handle, ctypes.byref(pt), ctypes.byref(pu)))
        return pt.value, pu.value

    def last_call_stats(self) -> dict:
        """pa_call_stats of the last attention call, as a dict."""
        st = abi.CallStats()
        abi.check(self.lib.pa_last_call_stats(self.handle, ctypes.byref(st)))
        return {name: int(getattr(st, name)) for name, _ in st._fields_ if name != "reserved"}

    def free_list(self):
        n = ctypes.c_int()
        abi.check(self.lib.pa_get_free_list(self.handle, None, 0, ctypes.byref(n)))
        buf = (ctypes.c_int32 * max(1, n.value))()
        abi.check(self.lib.pa_get_free_list(self.handle, buf, n.value, ctypes.byref(n)))
        return list(buf[: n.value])

    # ---- attention -----------------------------------------------------------
    def workspace_size(self, n_seq: int, num_q_heads: int, max_tokens: int, k_draft: int = 1,
                       partition_tokens: int = 0) -> int:
        b = ctypes.c_size_t()
        abi.check(self.lib.pa_workspace_size(self.handle, n_seq, num_q_heads, k_draft, max_tokens,
                                             partition_tokens, ctypes.byref(b)))
        return b.value

    def make_workspace(self, n_seq: int, num_q_heads: int, max_tokens: int, k_draft: int = 1,
                       partition_tokens: int = 0, device="cuda") -> Optional[torch.Tensor]:
        nbytes = self.workspace_size(n_seq, num_q_heads, max_tokens, k_draft, partition_tokens)
        if nbytes == 0:
            return None
        return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device)

    def decode(self, seq_ids, q: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True, partition_tokens: int = 0,
               workspace: Optional[torch.Tensor] = None, stream=None):
        """q: [n_seq, Hq, D]; returns (out, lse)."""
        n_seq, hq, d = q.shape
        return self._attend(seq_ids, 1, q, hq, scale, out, lse, want_lse, partition_tokens, workspace, stream)

    def decode_noalloc(self, seq_ids, q: torch.Tensor, scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                       partition_tokens: int = 0, stream=None):
        """pa_decode_noalloc: q, out [n_seq, Hq, D] and lse [n_seq, Hq] (or None)
        are caller-allocated; the library's fixed device scratch holds the
        plan and the split partials."""
        if q.dtype != self.tdtype or not q.is_contiguous() or q.dim() != 3 or q.shape[-1] != self.d:
            raise ValueError("q must be a contiguous [n_seq, Hq, D] tensor in the pool dtype")
        if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor shaped like q")
        ids, n = abi.i32_array(seq_ids)
        if n != q.shape[0]:
            raise ValueError("one query set per sequence")
        abi.check(self.lib.pa_decode_noalloc(self.handle, ids, n, q.shape[1], float(scale), _ptr(q), _ptr(out),
                                             _ptr(lse), partition_tokens, _stream(stream)))
        return out, lse

    def verify(self, seq_ids, q: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True, partition_tokens: int = 0,
               workspace: Optional[torch.Tensor] = None, stream=None):
        """q: [n_seq, K, Hq, D]; returns (out, lse)."""
        n_seq, kd, hq, d = q.shape
        return self._attend(seq_ids, kd, q, hq, scale, out, lse, want_lse, partition_tokens, workspace, stream)

    def prefill(self, seq_ids, q: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = True, partition_tokens: int = 0,
                workspace: Optional[torch.Tensor] = None, stream=None):
        """Chunked prefill: q [n_seq, n_new, Hq, D] for the last n_new (already
        appended) rows of each sequence; returns (out, lse)."""
        if q.dim() != 4:
            raise ValueError("q must be [n_seq, n_new, Hq, D]")
        n_seq, n_new, hq, d = q.shape
        if q.dtype != self.tdtype or not q.is_contiguous() or d != self.d:
            raise ValueError("q must be contiguous, in the pool dtype, with the pool head_dim")
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        ids, n = abi.i32_array(seq_ids)
        if n != n_seq:
            raise ValueError("one query set per sequence")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        abi.check(self.lib.pa_prefill(self.handle, ids, n, n_new, hq, float(scale), _ptr(q), _ptr(out), _ptr(lse),
                                      partition_tokens, _ptr(workspace), ws_bytes, _stream(stream)))
        return out, lse

    def append_attend(self, seq_ids, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, scale: float,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      want_lse: bool = True, partition_tokens: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None):
        """Append n_new rows per sequence and attend, in one launch when possible.

        k_new / v_new: [n_seq * n_new, Hkv, D]; q: [n_seq, n_new, Hq, D].
        Returns (out, lse) shaped like q (lse without the last dim)."""
        if q.dim() != 4:
            raise ValueError("q must be [n_seq, n_new, Hq, D]")
        n_seq, n_new, hq, d = q.shape
        self._check_rows(k_new, n_seq * n_new)
        self._check_rows(v_new, n_seq * n_new)
        if q.dtype != self.tdtype or not q.is_contiguous() or d != self.d:
            raise ValueError("q must be contiguous, in the pool dtype, with the pool head_dim")
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        ids, n = abi.i32_array(seq_ids)
        if n != n_seq:
            raise ValueError("one query set per sequence")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        abi.check(self.lib.pa_append_attend(self.handle, ids, n, n_new, _ptr(k_new), _ptr(v_new), hq, float(scale),
                                            _ptr(q), _ptr(out), _ptr(lse), partition_tokens, _ptr(workspace),
                                            ws_bytes, _stream(stream)))
        return out, lse

    def graph_prepare(self, seq_ids, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, scale: float,
                      out: torch.Tensor, lse: Optional[torch.Tensor], partition_tokens: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> int:
        """pa_graph_prepare: the host part of a graph step (append n_new rows per
        sequence, then attend); returns the step's class (padded units)."""
        n_seq, n_new, hq, d = q.shape
        self._check_rows(k_new, n_seq * n_new)
        self._check_rows(v_new, n_seq * n_new)
        if q.dtype != self.tdtype or not q.is_contiguous() or d != self.d or out.shape != q.shape:
            raise ValueError("q and out must be contiguous [n_seq, n_new, Hq, D] tensors in the pool dtype")
        ids, n = abi.i32_array(seq_ids)
        if n != n_seq:
            raise ValueError("one query set per sequence")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        cls = ctypes.c_int()
        abi.check(self.lib.pa_graph_prepare(self.handle, ids, n, n_new, _ptr(k_new), _ptr(v_new), hq, float(scale),
                                            _ptr(q), _ptr(out), _ptr(lse), partition_tokens, _ptr(workspace),
                                            ws_bytes, _stream(stream), ctypes.byref(cls)))
        return cls.value

    def graph_launch(self, stream=None) -> None:
        """pa_graph_launch: enqueue (or, under capture, record) the last prepared step."""
        abi.check(self.lib.pa_graph_launch(self.handle, _stream(stream)))

    def _attend(self, seq_ids, kd, q, hq, scale, out, lse, want_lse, pt, ws, stream):
        if q.dtype != self.tdtype or not q.is_contiguous() or q.shape[-1] != self.d:
            raise ValueError("q must be contiguous, in the pool dtype, with the pool head_dim")
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        ids, n = abi.i32_array(seq_ids)
        if n != q.shape[0]:
            raise ValueError("one query set per sequence")
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
        st = _stream(stream)
        if kd == 1 and q.dim() == 3:
            rc = self.lib.pa_decode(self.handle, ids, n, hq, float(scale), _ptr(q), _ptr(out), _ptr(lse), pt,
                                    _ptr(ws), ws_bytes, st)
        else:
            rc = self.lib.pa_verify(self.handle, ids, n, kd, hq, float(scale), _ptr(q), _ptr(out), _ptr(lse),
                                    pt, _ptr(ws), ws_bytes, st)
        abi.check(rc)
        return out, lse

    # ---- timing ----------------------------------------------------------------
    def profile_enable(self, on: bool = True) -> None:
        abi.check(self.lib.pa_profile_enable(self.handle, 1 if on else 0))

    def profile_read(self, which: int = 0):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        abi.check(self.lib.pa_profile_read(self.handle, which, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value
