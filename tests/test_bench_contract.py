"""bench.py on the CPU: a request for more than one GPU ends with a message,
and the algorithmic byte and flop counts of the measurement follow the
counting rule (every K and V row of every kv head once, q read and out written,
the table entries used, one length per sequence; new rows read and written,
one slot each), checked against figures worked out by hand."""
import os
import subprocess
import sys

import bench
from workloads import make_highbatch, make_tiny

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_tiny_decode_bytes_and_flops_by_hand():
    w = make_tiny()  # lengths 17, 33, 64, 100; 4 q = 4 kv heads, D = 64, fp32
    # K and V: 214 tokens x 4 kv heads x 64 x 4 B x 2       = 438,272
    # q read and out written: 2 x 4 seqs x 4 heads x 64 x 4 B = 8,192
    # table entries used: (2 + 3 + 4 + 7) x 4 B               = 64
    # lengths: 4 x 4 B                                        = 16
    assert bench.decode_bytes(w, 4) == 446_544
    # QK and PV: 4 flops per (dim, query head, visible position)
    assert bench.attention_flops(w) == 219_136


def test_highbatch_append_bytes_by_hand():
    w = make_highbatch()
    # 256 new rows x 8 kv heads x 128 dims, K and V, read as bf16 (2 B) and
    # written at the pool's element size, plus one 4-byte slot per row
    assert bench.append_bytes(w, 2) == 2_097_152 + 1_024
    assert bench.append_bytes(w, 1) == 1_572_864 + 1_024  # E4M3 pools: one byte written per element
