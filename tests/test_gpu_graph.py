"""A decode call captured into a HIP graph (through torch.cuda.graph) and
replayed after eager appends: every replay reads the lengths and block tables
current at replay time and equals an eager decode bitwise, and the oracle."""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch
from workloads import make_custom
from workloads.synth import _to_storage as to_storage

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k_draft", [1, 3])
def test_captured_decode_replays_over_grown_cache(k_draft):
    w = make_custom(lengths=[100, 37, 500, 16], num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                    seed=97)
    w.max_blocks_per_seq = 40            # room for the appends below
    pair = Pair(w, max_seqs=8, num_blocks=100, free_order=np.random.default_rng(4).permutation(100))
    pair.fill()
    seqs = [0, 1, 2, 3]
    rng = np.random.default_rng(98)
    q_bits = to_storage(rng.standard_normal((4, k_draft, w.num_q_heads, w.head_dim), dtype=np.float32), "bf16")
    q = to_torch(q_bits, "bf16").contiguous()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")

    def call(o, l_):
        if k_draft == 1:
            pair.gpu.decode(seqs, q[:, 0], w.scale, out=o[:, 0], lse=l_[:, 0])
        else:
            pair.gpu.verify(seqs, q, w.scale, out=o, lse=l_)

    if k_draft == 1:
        q = q.clone()  # q[:, 0] of a [4, 1, ...] tensor is contiguous
    call(out, lse)  # builds the work plan on the device, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    for step in range(3):
        n_new = [1 + step, 2, 17, 0][:4]
        k = to_storage(rng.standard_normal((sum(n_new), w.num_kv_heads, w.head_dim), dtype=np.float32), "bf16")
        v = to_storage(rng.standard_normal((sum(n_new), w.num_kv_heads, w.head_dim), dtype=np.float32), "bf16")
        pair.append(seqs, n_new, k, v)          # eager, outside the graph
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager_o = torch.empty_like(out)
        eager_l = torch.empty_like(lse)
        call(eager_o, eager_l)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_o.view(torch.int16)), f"replay {step}"
        assert torch.equal(lse, eager_l)
        ro, rl = oracle_decode(pair, seqs, q_bits, w.scale, k_draft=k_draft)
        assert_close(out, lse, ro, rl, "bf16", f"replay {step}")
