"""Pins of the q2k format (q2k pull-request page: 'Summary', 'Memory math', 'Reference papers')."""
import json
import os

import numpy as np
from scipy import integrate
from scipy.stats import norm

from oracle import accounting, q2k
from oracle.numerics import from_f16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_gaussian_lloyd_max_textbook_and_quadrature():
    g = json.load(open(os.path.join(GOLD, "gaussian_lloyd_max_textbook.json")))["n4"]
    th, lv = q2k.gaussian_lloyd_max(4)
    assert np.allclose(np.abs(lv[2:]), g["levels"], atol=6e-4)
    assert np.allclose(th[1:], g["thresholds"], atol=1e-4)
    # Lloyd's centroid condition by an independent quadrature of x phi(x)
    edges = [-np.inf] + list(th) + [np.inf]
    for i in range(4):
        m = integrate.quad(norm.pdf, edges[i], edges[i + 1], epsabs=1e-14)[0]
        mom = integrate.quad(lambda x: x * norm.pdf(x), edges[i], edges[i + 1], epsabs=1e-14)[0]
        assert abs(mom / m - lv[i]) < 1e-9
    mse = sum(integrate.quad(lambda x: (x - lv[i]) ** 2 * norm.pdf(x), edges[i], edges[i + 1], epsabs=1e-14)[0]
              for i in range(4))
    assert abs(mse - g["mse"]) < 1e-4
    assert np.array_equal(q2k.THETA, th.astype(np.float32)) and q2k.THETA[1] == 0


def test_threshold_rule_equals_nearest_level():
    rng = np.random.default_rng(20)
    t = rng.standard_normal(200000).astype(np.float32) * np.float32(2)
    code = q2k.k_codes_from_t(t)
    near = np.argmin(np.abs(t[:, None].astype(np.float64) - q2k.LEVELS[None, :].astype(np.float64)), axis=1)
    mid = np.isin(t, q2k.THETA)
    assert np.array_equal(code[~mid], near[~mid])
    # exact thresholds go to the upper cell
    assert list(q2k.k_codes_from_t(q2k.THETA)) == [1, 2, 3]
    # symmetry: code(-t) = 3 - code(t) off the thresholds
    assert np.array_equal(q2k.k_codes_from_t(-t[~mid]), 3 - code[~mid])


def test_k_block_rms_and_codes():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((32, 64)) * np.geomspace(1, 74.9, 64)).astype(np.float32)
    calib = np.ones(32, bool)
    calib[[0, 3]] = False
    codes, r16 = q2k.quantize_k_block(x, calib)
    rms = np.sqrt((x[calib].astype(np.float64) ** 2).mean(0))
    assert np.all(np.abs(from_f16_bits(r16) - rms) <= 1e-3 * rms)
    assert np.all(codes[[0, 3]] == 0)
    dq = q2k.k_dequant32(codes, r16[None])
    # relative MSE near the Gaussian Lloyd-Max distortion 0.1175 on Gaussian data
    rel = ((dq[calib] - x[calib]) ** 2).mean(0) / rms ** 2
    assert 0.08 < rel.mean() < 0.16


def test_v_symmetric_4bit():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((9, 128)).astype(np.float32)
    codes, s16 = q2k.quantize_v_rows(x, np.ones(9, bool))
    assert codes.max() <= 15
    s = np.repeat(from_f16_bits(s16), 32, 1).astype(np.float64)
    dq = q2k.v_dequant32(codes, np.repeat(s16, 32, 1))
    # nearest integer multiple of s in [-8, 7]
    brute = np.clip(np.round(x / s), -8, 7) * s
    assert np.all(np.abs(dq - brute) <= 1e-6 * np.abs(x).max())
    # the absmax element of each group maps to +-7 (or -8) levels
    g = np.abs(x.reshape(9, 4, 32))
    amax_codes = np.take_along_axis(codes.reshape(9, 4, 32), g.argmax(2)[..., None], 2)[..., 0]
    assert np.all((amax_codes == 15) | (amax_codes <= 1))


def test_memory_math_448_bytes_per_cell():
    g = json.load(open(os.path.join(GOLD, "q2k_memory_math.json")))
    per_head = accounting.bytes_per_token_head("q2k", g["head_dim"], 2, 4)
    cell = per_head * g["kv_heads"]
    assert cell == g["bytes_per_cell"]["q2k"]
    fp16 = g["kv_heads"] * g["head_dim"] * 2 * 2
    assert fp16 == g["bytes_per_cell"]["fp16"]
    gib = lambda b: b * g["context"] * g["layers"] / 2 ** 30  # noqa: E731
    assert round(gib(cell), g["printed_decimals"]) == g["kv_total_gib_printed"]["q2k"]
    assert round(gib(fp16), g["printed_decimals"]) == g["kv_total_gib_printed"]["fp16"]
