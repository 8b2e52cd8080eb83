"""Pins of RoPE on read (oracle/rope.py) and of the attention references with it.

Against closed forms: each channel pair turns as the complex number x_c + i x_{c+D/2} times
e^{i idx theta_c}; zero angle is the identity; norms are kept; q(i) . k(j) depends on j - i only
(to fp64 rounding: the angle is the exact product idx * theta_c, also at indices where an fp32 product
would move it by milliradians); theta_c is geometric with ratio base^(-2/D).  Against the
StreamingLLM + KIVI page ("RoPE caveat", "Implementation"): after eviction the sinks hold indices
0.., the window follows them without a gap, and a decode query sits at index n_sink + window - 1
however long the stream is.
"""
import numpy as np

from oracle import attention as oattn
from oracle import cache as ocache
from oracle import rope


def test_pairs_turn_as_complex_numbers():
    rng = np.random.default_rng(0)
    for D in (32, 64, 128):
        x = rng.standard_normal((7, D))
        idx = np.array([0, 1, 5, 17, 300, 4095, 65535])
        y = rope.rotate(x, idx)
        ang = rope.angles(idx, D).astype(np.float64)
        z = (x[:, : D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * ang)
        assert np.allclose(y[:, : D // 2], z.real, rtol=0, atol=1e-12)
        assert np.allclose(y[:, D // 2:], z.imag, rtol=0, atol=1e-12)
        assert np.array_equal(rope.rotate(x, np.zeros(7, np.int64)), x)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(1)
    D = 128
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for i, j in [(10, 3), (100, 0), (259, 4)]:
        base = rope.rotate(q, i) @ rope.rotate(k, j)
        for t in (1, 7, 1000, 3 * 65536 + 5):  # the last: an fp32 product would be off by 1e-2 rad
            shifted = rope.rotate(q, i + t) @ rope.rotate(k, j + t)
            assert abs(shifted - base) <= 1e-10 * np.abs(q).sum() * np.abs(k).max()
    # and q(i) . k(j) = q . k(j - i) exactly in the angle algebra (fp64 angles)
    th = rope.inv_freq(D).astype(np.float64)
    def rot64(x, ang):
        a, b = x[: D // 2], x[D // 2:]
        return np.concatenate([a * np.cos(ang) - b * np.sin(ang), b * np.cos(ang) + a * np.sin(ang)])
    assert abs(rot64(q, 9 * th) @ rot64(k, 4 * th) - q @ rot64(k, -5 * th)) < 1e-12


def test_angle_is_the_exact_product():
    """idx * theta_c to fp64 rounding: at index 65537 the fp32 product would differ by ~4e-3 rad."""
    th = rope.inv_freq(128).astype(np.float64)
    ang = rope.angles(np.array([65537, 12345678]), 128)
    for r, i in enumerate((65537, 12345678)):
        exact = np.array([float(i) * t for t in th])
        assert np.array_equal(ang[r], exact)
    f32 = (np.float32(65537) * rope.inv_freq(128)).astype(np.float64)
    assert np.abs(f32 - ang[0]).max() > 1e-3


def test_theta_is_geometric():
    for D, base in [(32, 10000.0), (128, 10000.0), (64, 500000.0)]:
        th = rope.inv_freq(D, base).astype(np.float64)
        assert th[0] == 1.0
        assert np.allclose(th[1:] / th[:-1], base ** (-2.0 / D), rtol=2e-7)
        assert abs(th[-1] - base ** (-(D - 2) / D)) <= 1e-7 * th[-1]


def test_indices_after_eviction():
    """first-N sinks + window: the sinks take 0..n_sink-1, the window follows, the query is last."""
    cfg = ocache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=1, head_dim=32, sink_mode="first_n", n_sink=4,
                        window=64, capacity=ocache.default_capacity(64), rope=True)
    m = ocache.CacheModel(cfg)
    rng = np.random.default_rng(2)
    for step in range(300):
        m.append(0, rng.standard_normal((1, 1, 1, 32)), rng.standard_normal((1, 1, 1, 32)))
        m.evict(0)
    pos = sorted(m.valid(0, 0).keys())
    P = m.P[0]
    assert [rope.index_of(pos, p) for p in range(4)] == [0, 1, 2, 3]
    assert [rope.index_of(pos, p) for p in range(P - 64, P)] == list(range(4, 68))
    assert rope.index_of(pos, P - 1) == 4 + 64 - 1
    # no eviction, no sinks: indices are the positions
    assert rope.index_of(list(range(50)), 37) == 37


def test_decode_attention_with_rope_equals_relative_form():
    """With W = 0 and no sinks the query sits at P-1 and row p at p, so the score of row p is
    q . R(p - (P-1)) k_p (fp64 angle algebra)."""
    cfg = ocache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=2, head_dim=64, fmt="kivi", k_bits=8,
                        v_bits=8, capacity=128, in_dtype="f32", rope=True)
    m = ocache.CacheModel(cfg)
    rng = np.random.default_rng(3)
    m.append(0, rng.standard_normal((1, 1, 40, 64)), rng.standard_normal((1, 1, 40, 64)))
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    out = oattn.decode_attention(m, 0, q)
    pos = list(range(40))
    kh = oattn.stream_values(m, 0, 0, 0, "k", pos)
    vh = oattn.stream_values(m, 0, 0, 0, "v", pos)
    th = rope.inv_freq(64).astype(np.float64)
    for j in range(2):
        s = np.array([q[0, j].astype(np.float64) @ np.concatenate([
            kh[p, :32] * np.cos((p - 39) * th) - kh[p, 32:] * np.sin((p - 39) * th),
            kh[p, 32:] * np.cos((p - 39) * th) + kh[p, :32] * np.sin((p - 39) * th)]) for p in pos]) / 8.0
        w = np.exp(s - s.max())
        ref = (w @ vh) / w.sum()
        assert np.allclose(out[0, j], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # the same rows without RoPE on read give another answer: the rotation is applied
    m2 = ocache.CacheModel(cfg.with_(rope=False))
    m2.append(0, m.K[0][:, :, :40], m.V[0][:, :, :40])
    assert np.abs(oattn.decode_attention(m2, 0, q) - out).max() > 1e-3


def test_prefill_last_query_equals_decode_with_rope():
    cfg = ocache.Config(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=32, fmt="kivi", k_bits=4, v_bits=4,
                        sink_mode="first_n", n_sink=3, window=40, residual=8, capacity=ocache.default_capacity(40),
                        rope=True)
    m = ocache.CacheModel(cfg)
    rng = np.random.default_rng(4)
    for n in (30, 25):
        m.append(0, rng.standard_normal((2, 2, n, 32)), rng.standard_normal((2, 2, n, 32)))
        m.evict(0)
    q = rng.standard_normal((2, 4, 25, 32)).astype(np.float16)
    pre = oattn.prefill_attention(m, 0, q)
    dec = oattn.decode_attention(m, 0, q[:, :, -1])
    assert np.allclose(pre[:, :, -1], dec, rtol=0, atol=1e-12)
