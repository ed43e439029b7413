"""Graph steps: the whole fused decode step (append + attention, split
partitions merged inside the launch) captured once per batch-size class into
a HIP graph (through torch.cuda.graph) and replayed over several steps, with
the host bookkeeping (pa_graph_prepare) run eagerly before every replay.

Each replay must equal the eager pa_append_attend call of the same step on a
twin pool bit for bit (outputs, lse), both pools and their tables must equal
the oracle's model, and the outputs must match the oracle.  The steps cross
block boundaries (table updates in the step's metadata), change class (a
second graph), come back to the first class, and include a copy-on-write
fork (the append then runs eagerly and the replay only attends), and
truncations between steps.  Capture and
replay of launches with in-place updated data, padded to batch classes:
"CUDA Graphs, modèles de raisonnement et service désagrégé", section 1.
"""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch
from workloads import make_custom
from workloads.synth import _to_storage as to_storage

pytestmark = pytest.mark.gpu


def _buffers(n, n_new, w, dtype):
    qd = "bf16" if dtype == "fp8" else dtype
    tq = torch.bfloat16 if qd == "bf16" else torch.float16
    return {
        "k": torch.empty((n * n_new, w.num_kv_heads, w.head_dim), dtype=tq, device="cuda"),
        "v": torch.empty((n * n_new, w.num_kv_heads, w.head_dim), dtype=tq, device="cuda"),
        "q": torch.empty((n, n_new, w.num_q_heads, w.head_dim), dtype=tq, device="cuda"),
        "out": torch.empty((n, n_new, w.num_q_heads, w.head_dim), dtype=tq, device="cuda"),
        "lse": torch.empty((n, n_new, w.num_q_heads), dtype=torch.float32, device="cuda"),
    }


@pytest.mark.parametrize("dtype,g,n_new,d", [("bf16", 4, 1, 128), ("f16", 8, 1, 128), ("bf16", 4, 5, 128),
                                             ("fp8", 4, 1, 128), ("bf16", 4, 1, 64), ("f16", 2, 3, 256)])
def test_graph_steps_replay_like_eager_calls(dtype, g, n_new, d):
    print(f"graph steps {dtype} G={g} n_new={n_new} D={d}", flush=True)
    wd = "bf16" if dtype == "fp8" else dtype
    lens = [int(x) for x in np.clip(np.rint(np.random.default_rng(90).lognormal(np.log(200), 1.0, 20)), 16, 1500)]
    w = make_custom(lengths=lens, num_q_heads=4 * g, num_kv_heads=4, head_dim=d, dtype=wd, seed=91)
    w.max_blocks_per_seq = 160
    nb = 2000
    order = np.random.default_rng(92).permutation(nb)
    kw = {}
    if dtype == "fp8":
        kw = dict(cache_dtype="fp8", kv_scales=(np.full(4, 0.02, np.float32), np.full(4, 0.03, np.float32)))
    pairs = [Pair(w, max_seqs=24, num_blocks=nb, free_order=order, **kw) for _ in range(2)]
    for pr in pairs:
        pr.fill()
    graph, eager = pairs
    rng = np.random.default_rng(93)
    ws = graph.gpu.make_workspace(20, w.num_q_heads, 2048, k_draft=n_new, partition_tokens=256)
    ws_e = eager.gpu.make_workspace(20, w.num_q_heads, 2048, k_draft=n_new, partition_tokens=256)
    stream = torch.cuda.Stream()
    graphs, bufs = {}, {}
    # phases: 12 sequences (one class), 20 (a larger class, with a fork of
    # sequence 15 -- 109 tokens, the fork shares 104 of them, so both append
    # into the shared, partly filled block: copies), 12 again.  Both pools use
    # the same partition length; the shared part is shorter than a partition,
    # so the eager call runs no shared-prefix pass either.
    pt = 256
    phases = [list(range(12))] * 3 + [list(range(19)) + [20]] * 3 + [list(range(12))] * 2
    forked = False
    for step, seqs in enumerate(phases):
        n = len(seqs)
        if n == 20 and not forked:
            for pr in pairs:
                pr.alloc(20, 15, int(pr.model.length(15)) - 5)
            forked = True
        if step in (1, 6):
            # truncations before a step: their length changes ride in the
            # step's metadata (sequence 13 is not in the first phase's steps)
            for pr in pairs:
                pr.truncate(2, int(pr.model.length(2)) - 3)
                pr.truncate(13, int(pr.model.length(13)) - 2)
        key = (n, n_new)
        if key not in bufs:
            bufs[key] = _buffers(n, n_new, w, dtype)
        b = bufs[key]
        k_bits = to_storage(rng.standard_normal((n * n_new, w.num_kv_heads, w.head_dim), dtype=np.float32), wd)
        v_bits = to_storage(rng.standard_normal((n * n_new, w.num_kv_heads, w.head_dim), dtype=np.float32), wd)
        q_bits = to_storage(rng.standard_normal((n, n_new, w.num_q_heads, w.head_dim), dtype=np.float32), wd)
        with torch.cuda.stream(stream):
            b["k"].copy_(to_torch(k_bits, wd))
            b["v"].copy_(to_torch(v_bits, wd))
            b["q"].copy_(to_torch(q_bits, wd))
            cls = graph.gpu.graph_prepare(seqs, b["k"], b["v"], b["q"], w.scale, b["out"], b["lse"],
                                          partition_tokens=pt, workspace=ws, stream=stream)
            if (cls, key) not in graphs:
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    graph.gpu.graph_launch(stream=stream)
                graphs[(cls, key)] = gr
            graphs[(cls, key)].replay()
        stream.synchronize()
        eo, el = eager.gpu.append_attend(seqs, to_torch(k_bits, wd), to_torch(v_bits, wd), to_torch(q_bits, wd),
                                         w.scale, partition_tokens=pt, workspace=ws_e)
        torch.cuda.synchronize()
        it = torch.int16
        assert torch.equal(b["out"].view(it), eo.view(it)), f"step {step}: replay and eager outputs differ"
        assert torch.equal(b["lse"], el), f"step {step}: lse"
        for pr in pairs:
            pr.model.append(seqs, [n_new] * n, k_bits, v_bits)
            pr.check_pools_and_tables()
        ro, rl = oracle_decode(graph, seqs, q_bits, w.scale, k_draft=n_new)
        assert_close(b["out"], b["lse"], ro, rl, dtype, f"graph step {step}")
    assert len({c for c, _ in graphs}) >= 2, "the steps never changed class"


def test_graph_prepare_rejections():
    w = make_custom(lengths=[700, 20], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16", seed=94)
    pair = Pair(w, max_seqs=4)
    pair.fill()
    b = _buffers(2, 1, w, "bf16")
    from paged_kv_cache_216_amd import PaInvalid
    from paged_kv_cache_216_amd.abi import PaStateError
    with pytest.raises(PaStateError):
        pair.gpu.graph_launch()                                   # nothing prepared
    with pytest.raises(PaInvalid):                                # 700 tokens split, no workspace
        pair.gpu.graph_prepare([0, 1], b["k"], b["v"], b["q"], w.scale, b["out"], b["lse"])
    pair.check_tables()                                           # nothing changed
    big = torch.empty((2, 20, 16, 128), dtype=torch.bfloat16, device="cuda")  # 80 rows per kv head
    kb = torch.empty((40, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(PaStateError):
        pair.gpu.graph_prepare([0, 1], kb, kb, big, w.scale, torch.empty_like(big), None)
    pair.check_tables()
