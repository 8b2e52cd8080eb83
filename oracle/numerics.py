"""Shared fp32/fp16 numerics of the oracle (test infrastructure only).

Rules the whole method is computed under:

* fp16 -> fp32 is exact; fp32 -> fp16 is IEEE round-to-nearest-even with
  subnormals (numpy's ``astype(float16)``; pinned against torch's conversion).
* Every code-deciding expression is evaluated in fp32, one rounding per
  operation, division and square root correctly rounded, ``rint`` rounding
  half to even.
* ``min``/``max`` results are canonicalised by adding +0.0, which turns a
  signed zero into +0 so that -0/+0 ties cannot make bytes differ.
* The sum of squares of a D-vector uses one fixed tree (``sumsq_canonical``):
  pair products first, then halving.  A sum has no single correct rounding, so
  this tree *is* the definition both sides follow.
"""

import numpy as np

F32 = np.float32
ZERO32 = np.float32(0.0)
EPS = np.float32(1e-5)  # the eps of the affine scale, StreamingLLM + KIVI page, "Affine quantisation formula"


def f32(x):
    """Array as float32 (exact for fp16 and fp32 input)."""
    return np.asarray(x, dtype=np.float32)


def to_f16_bits(x):
    """fp32 -> fp16 (RNE, subnormals kept), returned as uint16 bit patterns."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def from_f16_bits(bits):
    """uint16 fp16 bit patterns -> exact fp32 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def round_f16(x):
    """fp32 value of fp16(x) (RNE)."""
    return from_f16_bits(to_f16_bits(x))


def canon0(x):
    """+0.0 canonicalisation of a min/max result."""
    return np.asarray(x, dtype=np.float32) + ZERO32


def sumsq_canonical(x):
    """Sum of squares over the last axis (length a power of two >= 2) in fp32.

    Tree: a_l = x[2l]*x[2l] + x[2l+1]*x[2l+1] (two products, one add), then
    repeatedly a[:h] + a[h:] with h = len/2 until one value is left.
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    assert d >= 2 and (d & (d - 1)) == 0, "length must be a power of two"
    a = x[..., 0::2] * x[..., 0::2] + x[..., 1::2] * x[..., 1::2]
    while a.shape[-1] > 1:
        h = a.shape[-1] // 2
        a = a[..., :h] + a[..., h:]
    return a[..., 0]


def as_input(x, in_dtype):
    """Input rows as the caller hands them: fp16 (``'f16'``) or fp32 (``'f32'``), returned as fp32."""
    if in_dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    return np.asarray(x, dtype=np.float32)
