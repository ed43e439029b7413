"""The seeded generators are deterministic and produce the stated shapes."""
import numpy as np

from workloads import make_custom, make_tiny, make_verify


def test_same_seed_same_bytes():
    a = make_custom(lengths=[5, 40], num_q_heads=4, num_kv_heads=2, head_dim=16, dtype="bf16", seed=9)
    b = make_custom(lengths=[5, 40], num_q_heads=4, num_kv_heads=2, head_dim=16, dtype="bf16", seed=9)
    assert np.array_equal(a.free_order, b.free_order)
    for x, y in zip(a.k_rows + a.v_rows, b.k_rows + b.v_rows):
        assert np.array_equal(x, y)
    assert np.array_equal(a.q, b.q)


def test_tiny_shapes():
    w = make_tiny()
    assert list(w.lengths) == [17, 33, 64, 100]
    assert w.num_blocks == 64 and sorted(w.free_order) == list(range(64))
    assert w.k_rows[3].shape == (100, 4, 64) and w.k_rows[0].dtype == np.float32
    assert w.q.shape == (4, 1, 4, 64) and w.q2.shape == (4, 1, 4, 64)
    assert w.new_k.shape == (4, 1, 4, 64)
    assert w.scale == 1 / 8


def test_verify_shapes_small():
    w = make_verify(batch=4, prefix_len=64, k_draft=3)
    assert w.prefix_k.shape == (64, 8, 128)
    assert w.new_k.shape == (4, 3, 8, 128)
    assert np.all((w.lengths >= 16) & (w.lengths <= 512))
    assert np.array_equal(w.final_lengths(), w.lengths + 64 + 3)
