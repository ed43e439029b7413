"""GPU: pa_decode_noalloc (fixed device scratch, nothing allocated) against
pa_decode with a caller workspace, through the C ABI.

Two calls in a row on one pool, the second with a smaller input, each equal
to pa_decode bit for bit (same kernels, same plan) and to the oracle within
the dtype's tolerance; splits merged inside the attention launch and by the
merge launch; a shared-prefix pass; pending table updates carried in kernel
arguments; a partition whose partials exceed the scratch is rejected before
any launch.  Callers: those that cannot allocate device memory.
"""
import numpy as np
import pytest
import torch

from gpu_harness import Pair, assert_close, oracle_decode, to_torch, prefix_pass_ran
from paged_kv_cache_216_amd import PaInvalid
from workloads import make_custom
from workloads.synth import _to_storage as to_storage

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _both(pair, seqs, q_bits, pt):
    """pa_decode_noalloc first (so that it carries any pending table updates),
    then pa_decode with a workspace: bitwise equal, and within tolerance of
    the oracle."""
    w = pair.w
    q = to_torch(q_bits, w.dtype).reshape(len(seqs), w.num_q_heads, w.head_dim).contiguous()
    out = torch.full_like(q, float("nan"))
    lse = torch.full((len(seqs), w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    pair.gpu.decode_noalloc(seqs, q, w.scale, out, lse, partition_tokens=pt)
    torch.cuda.synchronize()
    out, lse = out.clone(), lse.clone()
    ws = pair.gpu.make_workspace(len(seqs), w.num_q_heads, int(max(pair.model.length(s) for s in seqs)),
                                 partition_tokens=pt)
    if ws is not None:
        ws.fill_(float("nan"))
    ref, ref_lse = pair.gpu.decode(seqs, q, w.scale, partition_tokens=pt, workspace=ws)
    torch.cuda.synchronize()
    it = torch.int32 if w.dtype == "f32" else torch.int16
    assert torch.equal(out.view(it), ref.view(it)), "noalloc output differs from pa_decode"
    assert torch.equal(lse, ref_lse), "noalloc lse differs from pa_decode"
    ro, rl = oracle_decode(pair, seqs, q_bits, w.scale)
    assert_close(out[:, None], lse[:, None], ro, rl, w.dtype, f"noalloc pt={pt}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_noalloc_two_calls_second_smaller(dtype):
    _say(f"noalloc two calls {dtype}")
    w = make_custom(lengths=[17, 530, 1000, 2048, 3000, 90, 1, 700], num_q_heads=16, num_kv_heads=4,
                    head_dim=128, dtype=dtype, seed=120)
    pair = Pair(w)
    pair.fill()
    seqs = list(range(w.batch))
    # first call: eight sequences, 64-token partitions (up to 47 of them: merge launch)
    _both(pair, seqs, w.q, 64)
    # second call: three shorter sequences, the library's partition (merged inside the launch)
    _both(pair, [5, 1, 2], w.q[[5, 1, 2]], 0)
    # and once more with a forced in-launch merge split
    _both(pair, [0, 3], w.q[[0, 3]], 256)


def test_noalloc_after_appends_and_forks():
    """Table updates left pending by forks (about 2,400 entries, more than one
    launch's arguments hold) reach the device through kernel arguments; the
    four forks and their parent take the shared-prefix pass."""
    _say("noalloc pending tables")
    w = make_custom(lengths=[40, 30000], num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16", seed=121,
                    num_blocks=3000)
    pair = Pair(w, max_seqs=8)
    pair.fill()
    for child in (2, 3, 4, 5):
        pair.alloc(child, 1, 16 * (child + 600))
    assert pair.gpu.lib is not None
    seqs = [0, 1, 2, 3, 4, 5]
    rng = np.random.default_rng(122)
    q_bits = to_storage(rng.standard_normal((6, 1, 8, 64), dtype=np.float32), "bf16")
    _both(pair, seqs, q_bits, 512)
    assert prefix_pass_ran(pair.gpu), "the shared-prefix pass did not run for pa_decode"
    pair.check_pools_and_tables()


def test_noalloc_rejects_partials_past_the_scratch():
    """An explicit partition whose partials exceed the 31 MiB partial region
    is rejected before any launch (outputs untouched); the library's own
    partition then runs and equals pa_decode."""
    _say("noalloc too large")
    w = make_custom(lengths=[4096] * 8, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16", seed=123)
    pair = Pair(w, track_data=False)
    pair.fill()
    seqs = list(range(8))
    q = to_torch(w.q, "bf16").reshape(8, 64, 128).contiguous()
    out = torch.zeros_like(q)
    lse = torch.zeros((8, 64), dtype=torch.float32, device="cuda")
    # 128 partitions x 8 kv heads x 8 rows x 130 floats x 4 bytes x 8 sequences = 34 MB
    with pytest.raises(PaInvalid):
        pair.gpu.decode_noalloc(seqs, q, w.scale, out, lse, partition_tokens=32)
    torch.cuda.synchronize()
    assert not out.any() and not lse.any()
    pair.gpu.decode_noalloc(seqs, q, w.scale, out, lse, partition_tokens=0)
    torch.cuda.synchronize()
    ws = pair.gpu.make_workspace(8, 64, 4096)
    ref, ref_lse = pair.gpu.decode(seqs, q, w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)) and torch.equal(lse, ref_lse)
