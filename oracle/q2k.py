"""q2k format: 2-bit K per channel over 32-token blocks, 4-bit V per token (test infrastructure only).

Follows the q2k pull-request page ("Summary", "Why per-channel K and per-token
V", "Memory math", "Reference papers"): K at 2 bits per channel with a
Lloyd-Max codebook over the block RMS, fitted to the Gaussian grid; V at 4
bits per token in 32-element blocks with one fp16 scale each; 448 bytes per
cell at 2 KV heads x 256 channels.

Readings (the page names the formats but does not define them):

* 448 B/cell fixes the metadata as one fp16 scale per K (channel, 32-token
  block) and one per V (token, 32-channel group), with no zero points.
* K: r = max(1e-5, sqrt(sum x^2 / n)) over the block's n calibration rows,
  summed sequentially in token order; t = x / fp16(r); code = number of
  Gaussian Lloyd-Max thresholds <= t; value = level[code] * fp16(r).
* V (symmetric 4-bit): s = max(1e-5, absmax/7); q = clamp(rint(x/fp16(s)),
  -8, 7); stored u = q + 8; value = (u - 8) * fp16(s).

Parity: the codebook is pinned to textbook Gaussian Lloyd-Max values and to
an independent quadrature of the fixed-point equations; the quantizers are
pinned by brute-force nearest-level and symmetry checks
(tests/test_oracle_q2k.py).
"""

import math

import numpy as np
from scipy.special import ndtr

from .numerics import EPS, canon0, f32, from_f16_bits, to_f16_bits


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi) if math.isfinite(x) else 0.0


def _Phi(x):
    if x == math.inf:
        return 1.0
    if x == -math.inf:
        return 0.0
    return float(ndtr(x))


def gaussian_lloyd_max(levels=4, iters=100000, tol=1e-15):
    """Lloyd-Max quantizer of N(0, 1) in fp64: (thresholds, levels).

    Lloyd's two conditions: thresholds are midpoints of adjacent levels; each
    level is the conditional mean of its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    """
    lv = np.linspace(-1.5, 1.5, levels)
    for _ in range(iters):
        th = 0.5 * (lv[1:] + lv[:-1])
        edges = [-math.inf] + list(th) + [math.inf]
        new = np.array([(_phi(edges[i]) - _phi(edges[i + 1])) / (_Phi(edges[i + 1]) - _Phi(edges[i]))
                        for i in range(levels)])
        new = 0.5 * (new - new[::-1])  # enforce the symmetry of N(0, 1)
        step = np.max(np.abs(new - lv))
        lv = new
        if step < tol:
            break
    th = 0.5 * (lv[1:] + lv[:-1])
    th[levels // 2 - 1] = 0.0
    return th, lv


_TH64, _LV64 = gaussian_lloyd_max(4)
THETA = _TH64.astype(np.float32)   # fp32 thresholds {-0.98159883, 0, +0.98159883}
LEVELS = _LV64.astype(np.float32)  # fp32 levels {-1.5104176, -0.45278, +0.45278, +1.5104176}


def k_codes_from_t(t):
    """Code = number of thresholds <= t (ties go to the upper cell)."""
    t = f32(t)
    return ((t >= THETA[0]).astype(np.uint8) + (t >= THETA[1]).astype(np.uint8)
            + (t >= THETA[2]).astype(np.uint8))


def quantize_k_block(x, calib):
    """32-token K blocks: x fp32 [..., 32, D], calib bool [..., 32] ->
    codes uint8 [..., 32, D] (0 outside calib) and rms16 [..., D]."""
    x = f32(x)
    calib = np.asarray(calib, dtype=bool)
    n = calib.sum(axis=-1).astype(np.float32)[..., None]
    ss = np.zeros(x.shape[:-2] + (x.shape[-1],), dtype=np.float32)
    for t in range(x.shape[-2]):  # sequential sum in token order
        ss = np.where(calib[..., t, None], ss + x[..., t, :] * x[..., t, :], ss)
    has = n > 0
    mean = ss / np.where(has, n, np.float32(1.0))
    r32 = np.where(has, np.maximum(EPS, np.sqrt(mean)), EPS)
    r16 = to_f16_bits(r32)
    codes = k_codes_from_t(x / from_f16_bits(r16)[..., None, :])
    codes = np.where(calib[..., :, None], codes, np.uint8(0)).astype(np.uint8)
    return codes, r16


def k_dequant32(u, r16):
    return LEVELS[np.asarray(u, dtype=np.intp)] * from_f16_bits(r16)


def quantize_v_rows(x, quantized):
    """V rows [n, D]: codes uint8 [n, D] (u = q + 8) and scale16 [n, D/32]."""
    x = f32(x)
    n, D = x.shape
    grp = x.reshape(n, D // 32, 32)
    amax = canon0(np.abs(grp).max(axis=2))
    s16 = to_f16_bits(np.maximum(EPS, amax / np.float32(7.0)))
    q = np.clip(np.rint(grp / from_f16_bits(s16)[:, :, None]), np.float32(-8.0), np.float32(7.0))
    codes = (q + np.float32(8.0)).astype(np.uint8).reshape(n, D)
    m = np.asarray(quantized, dtype=bool)
    codes[~m] = 0
    s16 = s16.copy()
    s16[~m] = 0
    return codes, s16


def v_dequant32(u, s16):
    return (np.asarray(u, dtype=np.float32) - np.float32(8.0)) * from_f16_bits(s16)

