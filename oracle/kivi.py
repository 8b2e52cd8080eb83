"""KIVI asymmetric min/max group quantization (test infrastructure only).

Follows the StreamingLLM + KIVI page, "Affine quantisation formula":
scale = max(eps, (xMax - xMin)/(qMax - qMin)) with eps = 1e-5, zero = xMin,
codes from rounding (x - zero)/scale, dequant (q - qMin)*scale + zero.  K is
grouped per channel (here over 32-token blocks, the group-size freezing the
page's "Caveats" section names), V per token (here over 32-channel groups).

Readings where the page is silent:

* qMax - qMin = 2^b - 1 for b = 8, 4 (the page's -128/127 and -8/7) and 2
  (the kivi_sink page runs b = 2; the page itself has no int2).
* Codes are stored as the unsigned offset u = q - qMin in [0, 2^b-1], and u is
  rounded directly, u = rint((x - zero)/scale).  Adding qMin before rounding,
  as printed, can flip a half-way tie in fp32; the mapping is otherwise the
  same.
* The code is computed against the *stored* fp16 scale and zero, so that the
  stored metadata reconstructs exactly what was coded.
* Dequant casts the fp16 scale and zero to fp32 first (the page's bug class 2)
  and computes u*scale + zero in fp32 with two roundings.
* Rows excluded from calibration (sinks, rows not yet appended) get code 0;
  a K group with no calibration row gets scale fp16(1e-5) and zero +0.

Parity: pinned (exact on-grid reconstruction, eps path, clamp range, error
bound, brute-force nearest-level check) in tests/test_oracle_kivi.py.
"""

import numpy as np

from .numerics import EPS, ZERO32, canon0, f32, from_f16_bits, to_f16_bits


def n_levels(bits):
    """qMax - qMin for a b-bit code."""
    assert bits in (2, 4, 8)
    return (1 << bits) - 1


def affine_meta(mn, mx, bits):
    """fp16 (scale, zero) bit patterns from fp32 group minimum and maximum."""
    L = np.float32(n_levels(bits))
    s32 = np.maximum(EPS, (f32(mx) - f32(mn)) / L)
    return to_f16_bits(s32), to_f16_bits(f32(mn))


def affine_codes(x, s16, z16, bits):
    """u = clamp(rint((x - zero)/scale), 0, L) against the stored fp16 metadata."""
    L = np.float32(n_levels(bits))
    y = (f32(x) - from_f16_bits(z16)) / from_f16_bits(s16)
    return np.clip(np.rint(y), ZERO32, L).astype(np.uint8)


def affine_dequant32(u, s16, z16):
    """fp32 dequant u*scale + zero (two roundings, no FMA)."""
    return np.asarray(u, dtype=np.float32) * from_f16_bits(s16) + from_f16_bits(z16)


def quantize_k_block(x, calib, bits):
    """32-token K blocks, quantized per channel.

    x: fp32 [..., 32, D] rows of each block (rows outside ``calib`` may hold
    anything); calib: bool [..., 32], the rows present and not sinks.
    Returns codes uint8 [..., 32, D] (0 outside calib), scale16 [..., D],
    zero16 [..., D].  A block without calibration rows gets scale
    fp16(1e-5), zero +0 and all-zero codes.
    """
    x = f32(x)
    calib = np.asarray(calib, dtype=bool)
    cm = calib[..., :, None]
    inf = np.float32(np.inf)
    mn = canon0(np.where(cm, x, inf).min(axis=-2))
    mx = canon0(np.where(cm, x, -inf).max(axis=-2))
    has = calib.any(axis=-1)[..., None]
    mn = np.where(has, mn, ZERO32)
    mx = np.where(has, mx, ZERO32)
    s16, z16 = affine_meta(mn, mx, bits)
    codes = affine_codes(x, s16[..., None, :], z16[..., None, :], bits)
    codes = np.where(cm, codes, np.uint8(0)).astype(np.uint8)
    return codes, s16, z16


def quantize_v_rows(x, quantized, bits):
    """V rows quantized per token over 32-channel groups.

    x: fp32 [n, D]; quantized: bool [n] (False for sink rows, which keep
    code 0 and metadata 0).  Returns codes [n, D], scale16 [n, D/32],
    zero16 [n, D/32].
    """
    x = f32(x)
    n, D = x.shape
    grp = x.reshape(n, D // 32, 32)
    mn = canon0(grp.min(axis=2))
    mx = canon0(grp.max(axis=2))
    s16, z16 = affine_meta(mn, mx, bits)
    codes = affine_codes(grp, s16[:, :, None], z16[:, :, None], bits).reshape(n, D)
    q = np.asarray(quantized, dtype=bool)
    codes[~q] = 0
    s16 = s16.copy()
    z16 = z16.copy()
    s16[~q] = 0
    z16[~q] = 0
    return codes, s16, z16
