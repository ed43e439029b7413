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


def test_rising_scores_plants_query_aligned_keys():
    """with_rising_scores: keys at 40 and 100 tokens into each span are the
    gain times the sequence's first query of the group's first head (rounded
    to storage), every other key row is untouched, values are scaled."""
    from workloads import with_rising_scores
    from workloads.synth import _storage_to_f32 as f32

    w = make_custom(lengths=[300, 20], mode="append_decode", num_q_heads=8, num_kv_heads=2, head_dim=16,
                    dtype="bf16", seed=11, prefix_len=0)
    r = with_rising_scores(w, 128, new_row_gain=3.0)
    q = f32(w.q, "bf16")
    planted = {40: 1.0, 100: 2.5, 168: 1.0, 228: 2.5, 296: 1.0}
    for t in range(300):
        for h in range(2):
            got = f32(r.k_rows[0][t, h], "bf16")
            if t in planted:
                want = f32(w.k_rows[0][t, h], "bf16") * 0 + planted[t] * q[0, 0, 4 * h]
                assert np.allclose(got, want, rtol=2 ** -8, atol=0)
            else:
                assert np.array_equal(r.k_rows[0][t, h], w.k_rows[0][t, h])
    assert np.array_equal(r.k_rows[1], w.k_rows[1])          # 20 tokens: no span reaches offset 40
    assert np.allclose(f32(r.v_rows[0], "bf16"), 0.5 * f32(w.v_rows[0], "bf16"), rtol=2 ** -8, atol=0)
    assert np.allclose(f32(r.new_k[1][-1, 1], "bf16"), 3.0 * q[1, 0, 4], rtol=2 ** -8, atol=0)
    assert np.array_equal(r.q, w.q)
