"""Benchmark: paged-attention decode step on one MI355X.

Default workload (the configuration the headline metric is quoted on): 256
sequences with log-normal lengths (median 200, sigma 1, clipped to [16, 2048]),
32 query / 8 key-value heads, head_dim 128, bf16.  One step = append one K/V
row per sequence (kv_append), then decode one query per sequence over the grown
cache, then roll the lengths back on the host so every step sees the same
workload.  Steps rotate over several pool replicas so that the working set
(~0.4 GB per replica) streams from HBM rather than the 256 MB Infinity Cache.

Prints one JSON line.  `value` is effective GB/s of the whole step (algorithmic
bytes of append + decode / step time); `roofline` reports the attention kernel
alone, timed with HIP events recorded on the launch stream; `cpu_baseline` times
the float64 CPU oracle on a bounded sample of the same workload; `graph_step`
(workloads whose step appends) times the same step replayed from captured
graphs (pa_graph_prepare, then the replay), device us/step and host enqueue.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode effective HBM GB/s (% of MI355X peak); µs/step at batch 256"
METRIC_PREFILL = "paged-attn chunked-prefill attention TFLOP/s (% of MI355X dense bf16/fp16 MFMA peak)"
PEAK_GBS = 8000.0  # MI355X HBM3E, AMD public specification
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense MFMA (fp32: vector), AMD public figures
FILL = {"f32": 0x7FBADBAD, "f16": 0x7E5A, "bf16": 0x7FDA, "fp8": 0x7F}
EB = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="highbatch",
                    choices=["highbatch", "gqa70b", "long", "verify", "tiny", "prefill"])
    ap.add_argument("--swap", action="store_true",
                    help="measure block swap instead: every sequence of the workload out to pinned host "
                         "memory and back in, per step")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="split-KV partition length; 0: the workload's (or the library's) choice; -1: no split")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--kv-cache", default="same", choices=["same", "fp8"],
                    help="pool element type: the workload's own, or E4M3 codes with one scale per kv head "
                         "(bf16 workloads only; rows, queries and outputs stay bf16)")
    ap.add_argument("--separate", action="store_true",
                    help="issue the append and the attention as two calls instead of pa_append_attend")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed pass of the step (append workloads)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB before the timed region, so that "
                         "memory counters can be scaled against a copy of known size")
    ap.add_argument("--no-profile-events", action="store_true",
                    help="do not record HIP events around the attention kernel")
    return ap.parse_args()


def to_torch(arr, dtype, device="cuda"):
    import torch
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(arr.view(np.float16))
    else:
        t = torch.from_numpy(arr.view(np.float32))
    return t.to(device)


def step_lengths(w):
    """Cached tokens per sequence when the attention runs."""
    return [int(n) for n in w.final_lengths()]


def decode_bytes(w, kv_eb) -> int:
    """Algorithmic bytes of one attention launch: every K and V row of every KV
    head once (a shared prefix once) at kv_eb bytes per element, Q read, O
    written, block-table entries used and one length per sequence."""
    lens = step_lengths(w)
    e = EB[w.dtype]
    rows = sum(n - w.prefix_len for n in lens) + (w.prefix_len if lens else 0)
    kv = rows * w.num_kv_heads * w.head_dim * kv_eb * 2
    qo = 2 * len(lens) * w.k_draft * w.num_q_heads * w.head_dim * e
    tab = sum(math.ceil(n / 16) for n in lens) * 4 + 4 * len(lens)
    return kv + qo + tab


def is_prefill(w) -> bool:
    """Many query tokens per sequence: the attention is bound by the matrix
    cores, not by HBM, and is reported in TFLOP/s."""
    return w.k_draft >= 64


def attention_flops(w) -> int:
    """Multiply-add work of the attention: every query row of every query head
    against each position it sees, 2 D flops for QK and 2 D for PV."""
    lens = step_lengths(w)
    seen = 0
    for n in lens:
        first = n - w.k_draft + 1  # positions the first query sees
        seen += w.k_draft * first + w.k_draft * (w.k_draft - 1) // 2
    return 4 * w.head_dim * w.num_q_heads * seen


def append_bytes(w, kv_eb) -> int:
    """New K and V rows read in the workload's type and written at kv_eb bytes
    per element, plus one slot index per row."""
    if w.new_k is None or w.mode not in ("append_decode", "verify"):
        return 0
    rows = w.new_k.shape[0] * w.new_k.shape[1]
    return 2 * rows * w.num_kv_heads * w.head_dim * (EB[w.dtype] + kv_eb) + 4 * rows


def fp8_scales(w):
    """One scale per kv head for E4M3 pools: the largest magnitude of that
    head's rows (prefix, cached and new) maps to 448, the largest code."""
    def amax(parts):
        m = np.zeros(w.num_kv_heads)
        for a in parts:
            if a is None or a.size == 0:
                continue
            x = (np.asarray(a).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            x = x.reshape(-1, w.num_kv_heads, w.head_dim)
            m = np.maximum(m, np.abs(x).max(axis=(0, 2)))
        return np.maximum(m, 1e-6) / 448.0
    ks = amax([w.prefix_k] + list(w.k_rows) + [w.new_k])
    vs = amax([w.prefix_v] + list(w.v_rows) + [w.new_v])
    return ks.astype(np.float32), vs.astype(np.float32)


class Replica:
    """One filled pool plus the pre-marshalled arguments of a step."""

    def __init__(self, w, pt, separate=False, cache_dtype=None, scales=None):
        import torch
        from paged_kv_cache_216_amd.cache import PagedKVCache

        self.w = w
        b = w.batch
        cd = cache_dtype or w.dtype
        self.cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, cd, b, w.max_blocks_per_seq,
                                  free_order=w.free_order, fill_bits=FILL[cd])
        c = self.cache
        if scales is not None:
            c.set_kv_scales(*scales)
        if w.prefix_len:
            c.alloc(0)
            c.append([0], [w.prefix_len], to_torch(w.prefix_k, w.dtype), to_torch(w.prefix_v, w.dtype))
            for s in range(1, b):
                c.alloc(s, 0, w.prefix_len)
        else:
            for s in range(b):
                c.alloc(s)
        for lo in range(0, b, 32):
            grp = list(range(lo, min(b, lo + 32)))
            ns = [int(w.lengths[i]) for i in grp]
            c.append(grp, ns, to_torch(np.concatenate([w.k_rows[i] for i in grp]), w.dtype),
                     to_torch(np.concatenate([w.v_rows[i] for i in grp]), w.dtype))
        torch.cuda.synchronize()
        self.base_lens = [int(w.lengths[i]) + w.prefix_len for i in range(b)]
        self.ids = (ctypes.c_int32 * b)(*range(b))
        self.t_new = 0
        if w.new_k is not None and w.mode in ("append_decode", "verify"):
            self.t_new = w.new_k.shape[1]
            self.ntok = (ctypes.c_int32 * b)(*([self.t_new] * b))
            hk = w.new_k.reshape(-1, w.num_kv_heads, w.head_dim)
            hv = w.new_v.reshape(-1, w.num_kv_heads, w.head_dim)
            self.k_new = to_torch(hk, w.dtype)
            self.v_new = to_torch(hv, w.dtype)
            self.rollback = (ctypes.c_int32 * b)(*self.base_lens)
        q = to_torch(w.q, w.dtype)
        self.q = q if w.k_draft > 1 else q[:, 0].contiguous()
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:-1], dtype=torch.float32, device="cuda")
        max_len = max(step_lengths(w))
        # pt < 0: no workspace, so nothing splits
        self.ws = None if pt < 0 else c.make_workspace(b, w.num_q_heads, max_len, k_draft=w.k_draft,
                                                       partition_tokens=pt)
        pt = max(pt, 0)
        self.ws_bytes = 0 if self.ws is None else self.ws.numel() * 4
        self.pt = pt
        self.separate = separate

    def step(self, stream_handle):
        from paged_kv_cache_216_amd import abi
        c, w, lib = self.cache, self.w, self.cache.lib
        h = c.handle
        vp = ctypes.c_void_p
        ws = None if self.ws is None else vp(self.ws.data_ptr())
        if self.t_new and not self.separate:
            # append + attend in one call (one launch when possible)
            abi.check(lib.pa_append_attend(h, self.ids, w.batch, self.t_new, vp(self.k_new.data_ptr()),
                                           vp(self.v_new.data_ptr()), w.num_q_heads, w.scale,
                                           vp(self.q.data_ptr()), vp(self.out.data_ptr()), vp(self.lse.data_ptr()),
                                           self.pt, ws, self.ws_bytes, stream_handle))
            abi.check(lib.pa_truncate_batch(h, self.ids, w.batch, self.rollback))
            return
        if self.t_new:
            abi.check(lib.pa_append_kv(h, self.ids, w.batch, self.ntok, vp(self.k_new.data_ptr()),
                                       vp(self.v_new.data_ptr()), stream_handle))
        if w.k_draft == 1:
            rc = lib.pa_decode(h, self.ids, w.batch, w.num_q_heads, w.scale, vp(self.q.data_ptr()),
                               vp(self.out.data_ptr()), vp(self.lse.data_ptr()), self.pt, ws, self.ws_bytes,
                               stream_handle)
        else:
            rc = lib.pa_verify(h, self.ids, w.batch, w.k_draft, w.num_q_heads, w.scale, vp(self.q.data_ptr()),
                               vp(self.out.data_ptr()), vp(self.lse.data_ptr()), self.pt, ws, self.ws_bytes,
                               stream_handle)
        abi.check(rc)
        if self.t_new:
            abi.check(lib.pa_truncate_batch(h, self.ids, w.batch, self.rollback))


    def graph_prepare(self, stream_handle, pt):
        """pa_graph_prepare of this replica's step; returns its class."""
        from paged_kv_cache_216_amd import abi
        c, w, lib = self.cache, self.w, self.cache.lib
        vp = ctypes.c_void_p
        ws = None if self.ws is None else vp(self.ws.data_ptr())
        cls = ctypes.c_int()
        abi.check(lib.pa_graph_prepare(c.handle, self.ids, w.batch, self.t_new, vp(self.k_new.data_ptr()),
                                       vp(self.v_new.data_ptr()), w.num_q_heads, w.scale, vp(self.q.data_ptr()),
                                       vp(self.out.data_ptr()), vp(self.lse.data_ptr()), pt, ws, self.ws_bytes,
                                       stream_handle, ctypes.byref(cls)))
        return cls.value

    def roll_back(self):
        from paged_kv_cache_216_amd import abi
        abi.check(self.cache.lib.pa_truncate_batch(self.cache.handle, self.ids, self.w.batch, self.rollback))


def graph_steps(reps, stream, steps, warmup, pt):
    """The step as a graph replay: pa_graph_prepare (host bookkeeping; the
    step's metadata and plan copied to the device on the stream), replay of the
    launch captured once per (replica, class) from pa_graph_launch, then the
    host rollback.  Returns device us/step and host enqueue us/step."""
    import torch
    from paged_kv_cache_216_amd import abi

    sh = ctypes.c_void_p(stream.cuda_stream)
    cap = torch.cuda.Stream()
    graphs = {}

    def one(i):
        j = i % len(reps)
        r = reps[j]
        cls = r.graph_prepare(sh, pt)
        g = graphs.get((j, cls))
        if g is None:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                abi.check(r.cache.lib.pa_graph_launch(r.cache.handle, ctypes.c_void_p(cap.cuda_stream)))
            graphs[(j, cls)] = g
        g.replay()
        r.roll_back()

    for i in range(max(warmup, len(reps))):
        one(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        one(i)
    t_enq = time.perf_counter() - t0
    stop.record(stream)
    torch.cuda.synchronize()
    stats = reps[0].cache.last_call_stats()
    return {"us_per_step": round(start.elapsed_time(stop) * 1e3 / steps, 2),
            "host_enqueue_us_per_step": round(1e6 * t_enq / steps, 2),
            "classes": sorted({c for _, c in graphs}), "partition_tokens": stats["partition_tokens"],
            "attention_workgroups": stats["attention_workgroups"]}


def make_workload(name):
    from workloads import by_name
    return by_name(name)


def describe(w) -> str:
    d = {"highbatch": "256 seqs, lengths lognormal(median 200, sigma 1) clipped to [16, 2048], 32 q / 8 kv heads, "
                      "head_dim 128, bf16; step = append 1 row/seq + decode",
         "gqa70b": "32 seqs, lengths U[512, 4096], 64 q / 8 kv heads, head_dim 128, fp16; step = decode",
         "long": "8 seqs x 32768 tokens, 32 q / 8 kv heads, head_dim 128, fp16, 512-token split-KV; step = decode",
         "verify": "64 seqs sharing a 4096-token copy-on-write prefix + suffix U[16, 512], 32 q / 8 kv heads, "
                   "head_dim 128, bf16; step = append 5 drafts/seq + causal verify",
         "tiny": "4 seqs {17, 33, 64, 100}, 4 heads, head_dim 64, fp32; step = append + decode",
         "prefill": "4 seqs x 8192 cached prompt tokens + a 512-token chunk each, 32 q / 8 kv heads, head_dim 128, "
                    "bf16; step = append the chunk + causal chunk attention"}
    return d[w.name]


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, budget_s, cache_dtype, scales):
    """The float64 oracle as it stands, on the first sequences of the same
    workload: first with one BLAS thread until about half of `budget_s`
    seconds of work, then the same sample with the BLAS library's own thread
    count (all the cores it uses).  Reported in the metric's unit."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention as A
    from oracle.allocator import PoolModel

    lens = step_lengths(w)

    def one(s):
        m = PoolModel(w.num_blocks, w.num_kv_heads, w.head_dim, cache_dtype, 1, w.max_blocks_per_seq,
                      free_order=w.free_order, kv_scales=scales)
        m.alloc(0)
        parts_k, parts_v = [], []
        if w.prefix_len:
            parts_k.append(w.prefix_k)
            parts_v.append(w.prefix_v)
        parts_k.append(w.k_rows[s])
        parts_v.append(w.v_rows[s])
        if w.new_k is not None and w.mode in ("append_decode", "verify"):
            parts_k.append(w.new_k[s])
            parts_v.append(w.new_v[s])
        k, v = np.concatenate(parts_k), np.concatenate(parts_v)
        t0 = time.perf_counter()
        m.append([0], [k.shape[0]], k, v)
        if w.k_draft == 1:
            A.decode_from_pool(m.kpool, m.vpool, m.table(0), m.length(0), w.q[s, 0], w.scale, cache_dtype, scales)
        else:
            A.verify_from_pool(m.kpool, m.vpool, m.table(0), m.length(0), w.q[s], w.scale, cache_dtype, scales)
        return time.perf_counter() - t0

    sample, t1 = [], 0.0
    with threadpool_limits(limits=1):
        for s in range(w.batch):
            t1 += one(s)
            sample.append(s)
            if t1 >= budget_s / 2:
                break
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    tn = sum(one(s) for s in sample)
    done_bytes = done_flops = ntok = 0
    for s in sample:
        n = lens[s]
        done_bytes += (n * w.num_kv_heads * w.head_dim * EB[cache_dtype] * 2
                       + 2 * w.k_draft * w.num_q_heads * w.head_dim * EB[w.dtype] + math.ceil(n / 16) * 4 + 4)
        done_flops += 4 * w.head_dim * w.num_q_heads * (w.k_draft * (n - w.k_draft + 1)
                                                        + w.k_draft * (w.k_draft - 1) // 2)
        ntok += n
    if is_prefill(w):
        unit, work, scale = "TFLOP/s", done_flops, 1e12
    else:
        unit, work, scale = "GB/s", done_bytes, 1e9
    return {
        "value": round(work / tn / scale, 6), "unit": unit, "cores": threads, "kind": "oracle",
        "sample": f"first {len(sample)} of {w.batch} sequences ({ntok} cached tokens): append into the float64 "
                  f"oracle's pool model, then gather + softmax attention, per sequence in Python; "
                  f"{tn:.1f} s with the BLAS library's {threads} threads, {t1:.1f} s with one",
        "single_thread": {"value": round(work / t1 / scale, 6), "unit": unit, "cores": 1},
        "cpu": cpu_model(), "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
    }


def kernel_source_id() -> str:
    """Hash of the kernel sources and of the host code that plans their
    launches (partition choice, work units): counter figures recorded for
    other sources no longer describe the kernels."""
    import hashlib
    h = hashlib.sha256()
    for f in ("kernels.hip", "kernels.hpp", "pa_api.cpp"):
        with open(os.path.join(ROOT, "paged_kv_cache_216_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE records
    kept under profiles/ (a line `traffic-record: key=value ...`), scaled by the
    factors those records give; None when no record matches these sources."""
    import glob
    src = kernel_source_id()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                line = line.strip().strip("`")
                if not line.startswith("traffic-record:"):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("workload") == workload and kv.get("kernel") == kernel and kv.get("source") == src:
                    return int(1024 * (float(kv["fetch_kib"]) * float(kv["fetch_scale"])
                                       + float(kv["write_kib"]) * float(kv["write_scale"])))
    return None


def copy_reference():
    """A plain 1 GiB device-to-device copy on the same GPU, timed with events
    after the timed region: what a simple streaming kernel reaches on this GPU
    (bytes read + written / time), as context for the fraction of the 8 TB/s
    specification the attention reaches."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    reps = 10
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"copy_gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_GBS, 4),
            "what": "1 GiB device-to-device copy (torch copy_), read + written bytes / time, 10 repetitions"}


PCIE_GBS = 64.0  # PCIe 5.0 x16, one direction, the MI355X host link


def run_swap(args, w):
    """Block swap to pinned host memory: a step swaps every sequence of one
    pool out (pa_swap_out, device -> host) and back in (pa_swap_in, host ->
    device).  Reported in GB/s of K/V bytes moved over the host link."""
    import torch
    rep = Replica(w, 0)
    c = rep.cache
    lens = [int(n) for n in w.lengths + w.prefix_len]
    imgs = []
    for n in lens:
        nb = c.swap_bytes(n)
        imgs.append((torch.empty(nb, dtype=torch.uint8, pin_memory=True),
                     torch.empty(nb, dtype=torch.uint8, pin_memory=True)))
    stream = torch.cuda.current_stream()

    def step():
        for s, (ki, vi) in enumerate(imgs):
            c.swap_out(s, ki, vi, stream)
        for s, (ki, vi) in enumerate(imgs):
            c.swap_in(s, lens[s], ki, vi, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    moved = 2 * sum(2 * c.swap_bytes(n) for n in lens)  # K and V images, out and in
    gbs = moved / (ms * 1e-3) / 1e9
    line = {
        "metric": "block swap GB/s (device <-> pinned host, K/V images out and back in)", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {describe(w)}; step = every sequence swapped out, then back in",
                   "bytes_per_step": moved, "sequences": len(lens)},
        "roofline": {"bound": "pcie", "achieved": round(gbs, 2), "peak": PCIE_GBS, "unit": "GB/s",
                     "frac": round(gbs / PCIE_GBS, 4), "traffic": None,
                     "note": "the out and in copies run one after the other, each bound by one direction"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sharding by sequence or by key/value head is not implemented)", flush=True)
        sys.exit(2)
    import torch

    from paged_kv_cache_216_amd import abi
    abi.load()
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    w = make_workload(args.workload)
    if args.swap:
        return run_swap(args, w)
    pt = args.partition_tokens if args.partition_tokens else (w.partition_tokens or 0)
    cd, scales, wkey = w.dtype, None, w.name
    if args.kv_cache == "fp8":
        if w.dtype != "bf16":
            print("bench.py: --kv-cache fp8 takes bf16 workloads", flush=True)
            sys.exit(2)
        cd, scales, wkey = "fp8", fp8_scales(w), w.name + "_fp8"
    print(f"bench: building {args.replicas} replica pools for '{wkey}'", file=sys.stderr, flush=True)
    reps = [Replica(w, pt, args.separate, cd, scales) for _ in range(args.replicas)]
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        reps[i % len(reps)].step(sh)
    torch.cuda.synchronize()

    # Timed region: K steps, nothing else on the stream.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        reps[i % len(reps)].step(sh)
    t_enq = time.perf_counter() - t0
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    # Kernel durations: the same K steps again with the library's HIP events
    # recorded around every launch on the launch stream (events between the
    # kernels stretch the step, so the step time above is taken without them).
    kern = {0: [0.0, 0], 1: [0.0, 0], 2: [0.0, 0], 3: [0.0, 0]}
    if not args.no_profile_events:
        for r in reps:
            for k in kern:
                r.cache.profile_read(k)
            r.cache.profile_enable(True)
        for i in range(args.steps):
            reps[i % len(reps)].step(sh)
        torch.cuda.synchronize()
        for r in reps:
            r.cache.profile_enable(False)
            for k in kern:
                ms, n = r.cache.profile_read(k)
                kern[k][0] += ms
                kern[k][1] += n
    # Per-step distribution: one more pass with an event pair around each step
    # (a step's own events add a little to it).
    pct = None
    if not args.no_profile_events:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            evs[i][0].record(stream)
            reps[i % len(reps)].step(sh)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        st = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        pct = {"p50": round(float(np.percentile(st, 50)), 2), "p90": round(float(np.percentile(st, 90)), 2),
               "p99": round(float(np.percentile(st, 99)), 2), "mean": round(float(st.mean()), 2)}
    pt_used, prefix_wgs = reps[0].cache.last_partition()
    stats = reps[0].cache.last_call_stats()
    hbm_ref = None if args.no_profile_events else copy_reference()
    kv_eb, e = EB[cd], EB[w.dtype]
    dec_b = decode_bytes(w, kv_eb)
    app_b = append_bytes(w, kv_eb)
    step_b = dec_b + app_b
    flops = attention_flops(w)
    prefill = is_prefill(w)
    value = step_b / (ms_step * 1e-3) / 1e9
    if prefill:
        value = flops / (ms_step * 1e-3) / 1e12
    # calls of several row tiles take the append and the attention as two launches
    one_tile = (w.num_q_heads // w.num_kv_heads) * w.k_draft <= (64 if w.head_dim <= 128 else 32)
    fused = bool(reps[0].t_new) and not args.separate and one_tile
    multi_wave = not one_tile and cd in ("f16", "bf16", "fp8")  # LDS-shared row tiles
    attn_name = "attn_append_kernel" if fused else ("tile_kernel" if multi_wave else "attn_kernel")

    # Each launch of the step with its own algorithmic bytes: the shared-prefix
    # pass reads the shared positions once and the queries of the rows it
    # serves; the attention launch the rest of the step's bytes (with the
    # append's when fused).  Split partials are not algorithmic: reported as
    # overhead (written once, read once by the merge).
    D, hkv = w.head_dim, w.num_kv_heads
    prefix_kv_b = stats["prefix_kv_tokens"] * hkv * D * 2 * kv_eb
    prefix_b = prefix_kv_b + stats["prefix_query_rows"] * hkv * D * e if stats["prefix_workgroups"] else 0
    attn_b = dec_b - prefix_kv_b + (app_b if fused else 0)
    if prefix_b and not kern[3][1] and kern[0][1]:
        # the shared-prefix units ran inside the attention launch: it moves
        # the whole step's bytes (the prefix once, q once)
        attn_name, attn_b = "attn_prefix_kernel", dec_b + (app_b if fused else 0)
    merge_name = "merge_rows_kernel" if attn_name == "attn_prefix_kernel" else "merge_kernel"
    own = {3: ("prefix_kernel", prefix_b), 0: (attn_name, attn_b), 2: ("append_kernel", app_b), 1: (merge_name, 0)}
    kernels, kernel_us_step, traffic = [], 0.0, 0
    for k in (3, 2, 0, 1):
        ms, n = kern[k]
        if not n:
            continue
        name, b = own[k]
        avg_us = 1e3 * ms / n
        per_step = n / args.steps
        kernel_us_step += avg_us * per_step
        t = measured_traffic(wkey, name)
        traffic = None if (t is None or traffic is None) else traffic + t * per_step
        kernels.append({"kernel": name, "avg_us": round(avg_us, 2), "launches_per_step": round(per_step, 3),
                        "bytes": b, "gbs": round(b / (avg_us * 1e-6) / 1e9, 1) if b else None,
                        "frac_hbm": round(b / (avg_us * 1e-6) / 1e9 / PEAK_GBS, 4) if b else None,
                        "traffic": t})
    roof = None
    if kernels:
        # Summed kernel time of a step: the per-launch events (which stretch
        # each launch a little) and the timed region / steps (which adds the
        # gaps between launches) both bound it from above; the smaller is used.
        step_us = kernel_us_step
        timing = "HIP events around each launch on its stream (second pass of the timed steps), summed per step"
        if ms_step * 1e3 < step_us:
            step_us = ms_step * 1e3
            timing = "HIP events on the launch stream around the timed region / steps (launch gaps included)"
        one_launch = len(kernels) == 1 and kernels[0]["launches_per_step"] == 1
        what = kernels[0]["kernel"] if one_launch else "step: " + " + ".join(k["kernel"] for k in kernels)
        achieved = step_b / (step_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": None if traffic is None else int(traffic),
                "kernel": what, "avg_us": round(step_us, 2), "bytes_per_launch": step_b, "timing": timing,
                "kernel_us_events": round(kernel_us_step, 2)}
        peak = PEAK_TFLOPS[w.dtype if cd != "fp8" else "bf16"]
        tf = flops / (step_us * 1e-6) / 1e12
        mfma = {"achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                "flops_per_step": flops}
        if prefill:
            roof.update({"bound": "mfma", "achieved": mfma["achieved"], "peak": peak, "unit": "TFLOP/s",
                         "frac": mfma["frac"], "flops_per_launch": flops, "hbm_gbs": round(achieved, 1)})
        elif w.k_draft > 1:
            roof["mfma"] = mfma  # verify: G x K_d query rows per kv head, reported against both roofs
    line = {
        "metric": METRIC_PREFILL if prefill else METRIC, "value": round(value, 2),
        "unit": "TFLOP/s" if prefill else "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_peak": round(100 * value / (PEAK_TFLOPS[w.dtype] if prefill else PEAK_GBS), 2),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{wkey}: {describe(w)}" + (
                       "; key/value pools in E4M3 with one scale per kv head (amax / 448)" if cd == "fp8" else ""),
                   "kv_cache": cd, "batch": w.batch, "seed": w.seed,
                   "replicas": args.replicas,
                   "partition_tokens": pt if pt > 0 else ("unsplit" if pt < 0 else "library choice"),
                   "partition_tokens_used": pt_used, "shared_prefix_workgroups": prefix_wgs,
                   "bytes_per_step": step_b, "decode_bytes": dec_b, "append_bytes": app_b,
                   "cached_tokens": int(sum(step_lengths(w))), "attention_flops": flops},
        "kernels": kernels,
        "split_overhead": {"partial_rows": stats["partial_rows"],
                           "partial_bytes_written": stats["partial_rows"] * (D + 2) * 4,
                           "what": "split-KV partials, written once and read once by the merge; not algorithmic"},
        "step_us_percentiles": pct,
        "host_wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "host_enqueue_us_per_step": round(1e6 * t_enq / args.steps, 2),
        "step_calls": ("pa_append_attend" if fused else
                       "pa_append_attend (append and attention launches)" if reps[0].t_new and not args.separate else
                       "pa_append_kv + attention" if reps[0].t_new else "attention"),
        "roofline": roof,
        "hbm_reference": hbm_ref,
    }
    if fused and not args.no_graph:
        # the same step replayed from captured graphs, at the partition length
        # the eager calls used (no shared-prefix pass in graph steps)
        print("bench: graph-replayed steps", file=sys.stderr, flush=True)
        g_pt = pt if pt > 0 else (pt_used or 0)
        try:
            gs = graph_steps(reps, stream, args.steps, args.warmup, g_pt)
            gs.update({"eager_us_per_step": line["us_per_step"],
                       "eager_host_enqueue_us_per_step": line["host_enqueue_us_per_step"],
                       "calls": "pa_graph_prepare, then replay of the graph captured from pa_graph_launch",
                       "timing": "HIP events on the stream around the timed steps (metadata copies included)"})
        except abi.PaError as exc:
            gs = {"error": str(exc)}
        line["graph_step"] = gs
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, cd, scales)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
