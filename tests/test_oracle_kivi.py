"""Pins of the KIVI affine quantizer (StreamingLLM + KIVI page, 'Affine quantisation formula')."""
import numpy as np

from oracle import kivi
from oracle.numerics import EPS, from_f16_bits, to_f16_bits


def _grid_group(bits, z, k, u):
    s = np.float32(2.0 ** -k)
    return np.float32(z) + u.astype(np.float32) * s, s


def test_exact_on_grid_reconstruction_k_and_v():
    rng = np.random.default_rng(10)
    for bits in (2, 4, 8):
        L = (1 << bits) - 1
        for z, k in [(-1.5, 4), (0.25, 7), (-3.0, 2), (0.0, 9)]:
            # K: per channel over a 32-row block; each channel hits 0 and L
            u = rng.integers(0, L + 1, size=(32, 64))
            u[0, :], u[1, :] = 0, L
            x, s = _grid_group(bits, z, k, u)
            codes, s16, z16 = kivi.quantize_k_block(x, np.ones(32, bool), bits)
            assert np.all(from_f16_bits(s16) == s) and np.all(from_f16_bits(z16) == np.float32(z))
            assert np.array_equal(codes, u.astype(np.uint8))
            assert np.array_equal(kivi.affine_dequant32(codes, s16[None], z16[None]), x)
            # V: per token over 32-channel groups
            uv = rng.integers(0, L + 1, size=(5, 64))
            uv[:, 0], uv[:, 1], uv[:, 32], uv[:, 33] = 0, L, 0, L
            xv, _ = _grid_group(bits, z, k, uv)
            cv, sv, zv = kivi.quantize_v_rows(xv, np.ones(5, bool), bits)
            assert np.array_equal(cv, uv.astype(np.uint8))
            dq = kivi.affine_dequant32(cv, np.repeat(sv, 32, 1), np.repeat(zv, 32, 1))
            assert np.array_equal(dq, xv)


def test_constant_group_uses_eps_and_no_nan():
    # bug class 1 of the page: min == max must not divide by zero
    x = np.full((32, 32), 0.75, np.float32)
    codes, s16, z16 = kivi.quantize_k_block(x, np.ones(32, bool), 4)
    assert np.all(s16 == to_f16_bits(EPS)) and abs(float(from_f16_bits(s16[0])) - 1.0013580322265625e-05) == 0
    assert np.all(codes == 0)
    dq = kivi.affine_dequant32(codes, s16[None], z16[None])
    assert np.all(np.isfinite(dq)) and np.all(dq == np.float32(0.75))
    x0 = np.zeros((3, 64), np.float32)
    c, s, z = kivi.quantize_v_rows(x0, np.ones(3, bool), 2)
    assert np.all(c == 0) and np.all(from_f16_bits(z) == 0) and np.all(np.isfinite(from_f16_bits(s)))


def test_clamp_range_and_nearest_level_bruteforce():
    rng = np.random.default_rng(11)
    for bits in (2, 4, 8):
        L = (1 << bits) - 1
        x = (rng.standard_normal((32, 128)) * rng.uniform(0.1, 6, size=128)).astype(np.float32)
        codes, s16, z16 = kivi.quantize_k_block(x, np.ones(32, bool), bits)
        assert codes.min() == 0 and codes.max() <= L
        s = from_f16_bits(s16).astype(np.float64)
        z = from_f16_bits(z16).astype(np.float64)
        lv = z[None, None, :] + np.arange(L + 1)[:, None, None] * s[None, None, :]  # [L+1, 1, D]
        dist = np.abs(x[None].astype(np.float64) - lv)  # [L+1, 32, D]
        best = dist.min(axis=0)
        got = np.take_along_axis(dist, codes[None].astype(np.intp), axis=0)[0]
        # the chosen level is the nearest one, up to the fp32 rounding of (x - z)/s
        assert np.all(got - best <= 2e-6 * (np.abs(x) + s[None] * L))


def test_roundtrip_error_bound():
    rng = np.random.default_rng(12)
    for bits in (2, 4, 8):
        L = (1 << bits) - 1
        x = rng.standard_normal((7, 128)).astype(np.float32) * np.float32(4)
        c, s16, z16 = kivi.quantize_v_rows(x, np.ones(7, bool), bits)
        g = x.reshape(7, 4, 32)
        mn, mx = g.min(2), g.max(2)
        s32 = np.maximum(EPS, (mx - mn) / np.float32(L)).astype(np.float64)
        s = from_f16_bits(s16).astype(np.float64)
        z = from_f16_bits(z16).astype(np.float64)
        bound = s / 2 + L * np.abs(s - s32) + np.abs(z - mn) + 1e-6 * np.abs(g).max(2)
        dq = kivi.affine_dequant32(c, np.repeat(s16, 32, 1), np.repeat(z16, 32, 1)).reshape(7, 4, 32)
        err = np.abs(dq.astype(np.float64) - g).max(2)
        assert np.all(err <= bound)


def test_calibration_excludes_rows():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    x[5] *= 25
    calib = np.ones(32, bool)
    calib[5] = False
    c1, s1, z1 = kivi.quantize_k_block(x, calib, 2)
    c2, s2, z2 = kivi.quantize_k_block(np.delete(x, 5, 0), np.ones(31, bool), 2)
    assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
    assert np.array_equal(np.delete(c1, 5, 0), c2) and np.all(c1[5] == 0)
    # 'replace by the nearest non-sink row' inside the group leaves min and max unchanged
    xr = x.copy()
    xr[5] = x[4]
    c3, s3, z3 = kivi.quantize_k_block(xr, np.ones(32, bool), 2)
    assert np.array_equal(s3, s1) and np.array_equal(z3, z1)


def test_no_calibration_rows():
    c, s, z = kivi.quantize_k_block(np.ones((32, 32), np.float32), np.zeros(32, bool), 2)
    assert np.all(c == 0) and np.all(s == to_f16_bits(EPS)) and np.all(z == 0)
