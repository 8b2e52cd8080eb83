"""Pins of TurboQuant at a head_dim that is not a power of two (TurboQuant spec, "Hadamard Transform
Detail": pad to the next power of two; "Codebook Generation": target dimensions 64, 96, 128, 160).

Reading: the rows are zero-padded to dp (96 -> 128, 160 -> 256), rotated by the dp-point Walsh-Hadamard
transform with dp signs, and every rotated coordinate is coded (the page's truncation would discard
the energy that lands in the extra coordinates, so it cannot be inverted); the codebooks are the
page's Beta(d/2, d/2) for the head_dim d.  Decode reads the first d channels of the inverse rotation.
"""
import numpy as np
import pytest
from scipy import integrate
from scipy.linalg import hadamard
from scipy.stats import beta as beta_dist

from oracle import attention, cache
from oracle import turboquant as tq


@pytest.mark.parametrize("d", [96, 160])
def test_codebooks_for_the_page_target_dimensions(d):
    for bits in (2, 3, 4):
        b, c, _ = tq.beta_lloyd_max(d, bits)
        L = 1 << bits
        edges = [0.0] + list(b) + [1.0]
        for i in range(L):  # Lloyd's fixed point of Beta(d/2, d/2) by independent quadrature
            pdf = lambda x: beta_dist.pdf(x, d / 2, d / 2)  # noqa: E731
            m = integrate.quad(pdf, edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13, limit=200)[0]
            mom = integrate.quad(lambda x: x * pdf(x), edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13,
                                 limit=200)[0]
            assert abs(mom / m - c[i]) < 1e-10
        kb, kc = tq.codebook(d, bits)
        assert np.array_equal(kc, -kc[::-1]) and kb[L // 2 - 1] == 0
        init = beta_dist.ppf((np.arange(L) + 0.5) / L, d / 2, d / 2)  # unique: a second start agrees
        _, c2, _ = tq.beta_lloyd_max(d, bits, init=init)
        assert np.array_equal((2 * c - 1).astype(np.float32), (2 * c2 - 1).astype(np.float32))


@pytest.mark.parametrize("d,dp", [(96, 128), (160, 256)])
def test_padded_rotation_is_orthogonal_and_invertible(d, dp):
    sg = tq.signs(5, dp)
    R = (hadamard(dp) / np.sqrt(dp)) @ np.diag(sg.astype(np.float64))
    rng = np.random.default_rng(d)
    x = rng.standard_normal((50, d)).astype(np.float32)
    xp = tq.pad(x, dp)
    assert xp.shape == (50, dp) and np.all(xp[:, d:] == 0) and np.array_equal(xp[:, :d], x)
    y = tq.rotate(xp, sg)
    assert np.allclose(y.astype(np.float64), xp.astype(np.float64) @ R.T, atol=1e-5)
    # energy is kept over the dp coordinates: |R [x; 0]| = |x|
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=2e-6)
    # the fp64 inverse returns x in the first d channels and zeros after them
    back = (y.astype(np.float64) @ R)
    assert np.allclose(back[:, :d], x, atol=2e-6) and np.allclose(back[:, d:], 0, atol=2e-6)


def test_padded_dequant_distortion_matches_the_codebook():
    """Relative round-trip error of padded rows = dp * 4 * E[(u - q(u))^2] with u distributed as a
    coordinate of a rotated dp-dimensional unit vector (Beta(dp/2, dp/2)) and q the d = 96 quantizer."""
    d, dp = 96, 128
    sg = tq.signs(7, dp)
    rng = np.random.default_rng(96)
    x = rng.standard_normal((4000, d)).astype(np.float32)
    for bits in (2, 4):
        kb, kc = tq.codebook(d, bits)
        b, c, _ = tq.beta_lloyd_max(d, bits)
        edges = [0.0] + list(b) + [1.0]
        mse_u = sum(integrate.quad(lambda u: (u - c[i]) ** 2 * beta_dist.pdf(u, dp / 2, dp / 2), edges[i],
                                   edges[i + 1], epsabs=1e-15)[0] for i in range(1 << bits))
        u, n = tq.quantize_rows(x, sg, kb)
        assert u.shape == (4000, dp)
        xh = tq.dequant64(u, n, kc, sg)[:, :d]
        rel = ((xh - x) ** 2).sum(1) / (x ** 2).sum(1)
        # the first d channels carry d/dp of the error of the dp coordinates
        assert abs(rel.mean() / (d * 4 * mse_u) - 1) < 0.05


def test_cache_at_head_dim_96_reads_through_the_rotated_domain():
    """Decode attention over the truncated reconstructions equals the rotated-domain product the fused
    kernel forms (the page's "Optimization: Fused dequant-dot"): q . x_hat = (R [q; 0]) . (n c[u])."""
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=2, head_dim=96, fmt="tq", k_bits=4, v_bits=2,
                       capacity=128, seed=3)
    assert cfg.store_dim == 128
    m = cache.CacheModel(cfg)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((1, 1, 70, 96)).astype(np.float16)
    v = rng.standard_normal((1, 1, 70, 96)).astype(np.float16)
    m.append(0, k, v)
    img = m.image(0, 0, 0)
    assert img["bulk"].shape[1] == 32 * 128 * 4 // 8 + 32 * 128 * 2 // 8 + 8 * 32
    pos = list(range(70))
    kk = attention.stream_values(m, 0, 0, 0, "k", pos)
    assert kk.shape == (70, 96)
    q = rng.standard_normal(96)
    sg = tq.signs(3, 128).astype(np.float64)
    R = (hadamard(128) / np.sqrt(128)) @ np.diag(sg)
    qt = R @ np.concatenate([q, np.zeros(32)])  # the padded query, rotated once
    qs = cache.quantize_stream(cfg, m.K[0][0, 0], m.V[0][0, 0], [], 70, m.tq)
    kc = m.tq.kc.astype(np.float64)[qs["k_codes"].reshape(-1, 128)[:70].astype(np.intp)]
    rot = qs["k_norm"].reshape(-1)[:70, None].astype(np.float64) * kc  # n c[u]: 128 rotated coordinates
    assert np.allclose(rot @ qt, kk @ q, rtol=0, atol=1e-9 * np.abs(kk @ q).max())
