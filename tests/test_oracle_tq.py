"""Pins of the TurboQuant variant (TurboQuant spec page)."""
import json
import os

import numpy as np
from scipy import integrate
from scipy.linalg import hadamard
from scipy.stats import beta as beta_dist

from oracle import layout
from oracle import turboquant as tq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_fwht_is_sylvester_hadamard():
    for d in (2, 8, 32, 128):
        H = tq.fwht(np.eye(d))
        assert np.array_equal(H, hadamard(d).astype(np.float64))


def test_rotation_orthogonal_and_inverse():
    for d in (32, 64, 128):
        sg = tq.signs(0x5EED0004, d)
        R = (hadamard(d) / np.sqrt(d)) @ np.diag(sg.astype(np.float64))  # signs first, then H/sqrt(d)
        assert np.allclose(R @ R.T, np.eye(d), atol=1e-12)
        # (H/sqrt(d))^2 = I and D^2 = I separately; R itself is not an involution
        Hn = hadamard(d) / np.sqrt(d)
        assert np.allclose(Hn @ Hn, np.eye(d), atol=1e-12) and np.all(sg * sg == 1)
        rng = np.random.default_rng(30)
        x = rng.standard_normal((20, d)).astype(np.float32)
        y = tq.rotate(x, sg)
        assert np.allclose(y.astype(np.float64), x.astype(np.float64) @ R.T, rtol=0, atol=1e-5)
        back = tq.inverse_rotate(y, sg)
        assert np.max(np.abs(back - x)) <= 1e-6 * np.max(np.abs(x)) * 4
        # fp32 orthogonality of the rotation applied to the identity
        Rf = tq.rotate(np.eye(d, dtype=np.float32), sg).T.astype(np.float64)
        assert np.allclose(Rf @ Rf.T, np.eye(d), atol=1e-6)


def _cell_moments(a, lo, hi):
    pdf = lambda x: beta_dist.pdf(x, a, a)  # noqa: E731
    m = integrate.quad(pdf, lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    mom = integrate.quad(lambda x: x * pdf(x), lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
    return m, mom


def test_codebook_fixed_point_by_quadrature_and_symmetry():
    d = 128
    for bits in (2, 3, 4):
        b, c, _ = tq.beta_lloyd_max(d, bits)
        L = 1 << bits
        edges = [0.0] + list(b) + [1.0]
        for i in range(L):
            m, mom = _cell_moments(d / 2, edges[i], edges[i + 1])
            assert abs(mom / m - c[i]) < 1e-10
        kb, kc = tq.codebook(d, bits)
        assert np.array_equal(kc, -kc[::-1]) and kb[L // 2 - 1] == 0
        assert np.all(np.diff(kc) > 0) and np.all(np.diff(kb) > 0)


def test_codebook_unique_from_another_start():
    for bits in (2, 3, 4):
        L = 1 << bits
        b1, c1, _ = tq.beta_lloyd_max(128, bits)
        init = beta_dist.ppf((np.arange(L) + 0.5) / L, 64, 64)  # quantile start
        b2, c2, _ = tq.beta_lloyd_max(128, bits, init=init)
        assert np.array_equal((2 * c1 - 1).astype(np.float32), (2 * c2 - 1).astype(np.float32))


def test_codebook_gaussian_limit():
    g = json.load(open(os.path.join(GOLD, "gaussian_lloyd_max_textbook.json")))
    sd = 1.0 / (2.0 * np.sqrt(129.0))
    _, c4 = tq.codebook(128, 2)
    _, c16 = tq.codebook(128, 4)
    assert np.allclose(c4[2:] / (2 * sd), g["n4"]["levels"], rtol=0.0035)
    assert np.allclose(c16[8:] / (2 * sd), g["n16"]["levels"], rtol=0.017)  # 1.59% at the outer level, plus the table's 4-digit rounding


def test_roundtrip_mse_matches_distortion():
    d = 128
    rng = np.random.default_rng(31)
    sg = tq.signs(7, d)
    x = rng.standard_normal((4000, d)).astype(np.float32)
    for bits in (2, 3, 4):
        kb, kc = tq.codebook(d, bits)
        b, c, _ = tq.beta_lloyd_max(d, bits)
        edges = [0.0] + list(b) + [1.0]
        mse_u = 0.0
        for i in range(1 << bits):
            mse_u += integrate.quad(lambda u: (u - c[i]) ** 2 * beta_dist.pdf(u, 64, 64), edges[i], edges[i + 1],
                                    epsabs=1e-15)[0]
        u, n = tq.quantize_rows(x, sg, kb)
        xh = tq.dequant32(u, n, kc, sg)
        rel = ((xh - x) ** 2).sum(1) / (x ** 2).sum(1)
        assert abs(rel.mean() / (d * 4 * mse_u) - 1) < 0.05


def test_edge_cases_zero_constant_large():
    d = 64
    sg = tq.signs(3, d)
    kb, kc = tq.codebook(d, 4)
    x = np.zeros((1, d), np.float32)
    u, n = tq.quantize_rows(x, sg, kb)
    assert n[0] == 0 and np.all(tq.dequant32(u, n, kc, sg) == 0)
    for scale in (1e-3, 1.0, 3e4):
        xc = np.full((2, d), scale, np.float32)
        u, n = tq.quantize_rows(xc, sg, kb)
        xh = tq.dequant32(u, n, kc, sg)
        assert np.all(np.isfinite(xh))
        assert np.linalg.norm(xh - xc) / np.linalg.norm(xc) < 0.3


def test_determinism_and_fused_dot_identity():
    d = 128
    rng = np.random.default_rng(32)
    x = rng.standard_normal((10, d)).astype(np.float32)
    kb, kc = tq.codebook(d, 4)
    a = tq.quantize_rows(x, tq.signs(99, d), kb)
    b = tq.quantize_rows(x, tq.signs(99, d), kb)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # q . R^T k~ = (R q) . k~  (rotated-domain decode)
    sg = tq.signs(99, d).astype(np.float64)
    R = (hadamard(d) / np.sqrt(d)) @ np.diag(sg)
    q = rng.standard_normal(d)
    kt = a[1][:, None] * kc[a[0]].astype(np.float64)
    lhs = (R.T @ kt.T).T @ q
    rhs = kt @ (R @ q)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    assert np.allclose(tq.dequant64(a[0], a[1], kc, tq.signs(99, d)), (R.T @ kt.T).T, atol=1e-12)


def test_turboquant_code_bytes_per_token():
    from oracle import layout
    g = json.load(open(os.path.join(GOLD, "turboquant_memory.json")))
    for row in g["rows"]:
        _, size, _ = layout.record_sections("tq", row["head_dim"], row["k_bits"], row["v_bits"])
        assert size["k_codes"] // 32 * row["heads"] == row["keys_bytes"]
        assert size["v_codes"] // 32 * row["heads"] == row["values_bytes"]
        # metadata: one fp32 norm each for K and V per head (the page's two range floats each)
        assert (size["k_meta"] + size["v_meta"]) // 32 * row["heads"] * 2 == row["range_metadata_bytes"]
    assert 128 * 7 == g["rotation_flops_d128"]  # d log2 d butterflies


def test_three_bit_codes_take_the_per_byte_packing():
    """[TQ] "Step 3: Packing": 3-bit codes go two per byte with two bits unused, so K3 keys of 16
    heads at dim 128 take 16 * 128 / 2 = 1024 bytes per token (the page's 768 B row assumes the
    dense 8-in-3 alternative it mentions), the same as 4-bit keys."""
    _, s3, _ = layout.record_sections("tq", 128, 3, 2)
    _, s4, _ = layout.record_sections("tq", 128, 4, 2)
    assert s3["k_codes"] == s4["k_codes"] and 16 * s3["k_codes"] // 32 == 1024
    codes = np.arange(8, dtype=np.uint8)[None, :].repeat(4, 0).reshape(1, 32)
    assert np.array_equal(layout.unpack_words(layout.pack_words(codes, layout.slot_bits(3)), 4), codes)
    assert layout.pack_words(codes, 4).size == 16  # 32 codes in 16 bytes: two per byte


def test_dense_three_bit_stream():
    """The page's "8 values into 3 bytes": K3/V2 keys of 16 heads at dim 128 take 768 bytes per token
    ([TQ] "Memory per token per layer"), and the stream puts code i at bits 3i..3i+2, LSB first."""
    _, s3, _ = layout.record_sections("tq", 128, 3, 2, dense3=True)
    assert 16 * s3["k_codes"] // 32 == 768
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 8, size=(5, 64)).astype(np.uint8)
    packed = layout.pack_bits3(codes)
    assert packed.shape == (5, 24)
    big = int.from_bytes(packed[2].tobytes(), "little")
    assert all(((big >> (3 * i)) & 7) == codes[2, i] for i in range(64))
    assert np.array_equal(layout.unpack_bits3(packed, 64), codes)
    for D in (32, 64, 128):
        k = rng.integers(0, 8, size=(2, 32, D)).astype(np.uint8)
        assert np.array_equal(layout.unpack_k_rows(layout.pack_k_rows(k, 3), D, 3), k)
        assert np.array_equal(layout.unpack_v_tiles(layout.pack_v_tiles(k, 3), D, 3), k)
        assert layout.pack_k_rows(k, 3).shape[-1] == 32 * D * 3 // 8
