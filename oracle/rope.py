"""Rotary position embedding applied on read at a row's index in the compressed cache (test
infrastructure only).

Follows the StreamingLLM + KIVI page, "RoPE caveat — the vanilla StreamingLLM choice" and
"Caveats": StreamingLLM's own scheme gives every cached key the rotation of its index in the
compressed cache rather than of its original position, which needs the keys stored before RoPE and
the rotation applied when they are read.  Storing K before RoPE also keeps the per-channel K
quantisation on a stable basis ("The bug class the previous attempt hit", 5).

Readings where the pages are silent:

* The rotation is the rotary embedding in its rotate-half form: channel c < D/2 pairs with
  c + D/2, and the pair (x_c, x_{c+D/2}) turns by the angle idx * theta_c with
  theta_c = base^(-2c/D), base 10000 unless configured.  The pages name RoPE without fixing the
  pairing or the base.
* The index of a cached row is the number of valid positions before it (its slot in the
  compressed cache, sinks and window in position order); the index of a query is the number of
  valid positions before its own position (in decode its own row is the last valid one, so
  |valid| - 1).
* theta_c is rounded to fp32 (the table a kernel holds); the angle is the exact product
  idx * theta_c (taken in fp64, where it is exact to 2^-53 relative) and cos and sin are taken of it
  in fp64.  The rotary embedding defines the angle as that product; an fp32 rounding of it, as fp32
  frameworks form it, is an artefact of those frameworks that the pages do not ask for (it moves the
  angle by up to half an fp32 ulp, 2.4e-4 rad at index 4096 and 3.9e-3 rad at index 65536).
* The query is handed over before RoPE as well; only the cache knows its index.

Parity: pinned in tests/test_oracle_rope.py (the complex-multiplication form of each pair, zero
angle, norms, the relative-position identity, theta's geometric ratio, and the indices StreamingLLM
eviction leaves: sinks 0.., the window right after them, the query last).
"""

import numpy as np

DEFAULT_BASE = 10000.0


def inv_freq(D, base=DEFAULT_BASE):
    """theta_c = base^(-2c/D) for c < D/2, rounded to fp32."""
    c = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * c / D).astype(np.float32)


def angles(idx, D, base=DEFAULT_BASE):
    """Angles idx * theta_c (fp64), shape idx.shape + (D/2,)."""
    i = np.asarray(idx, dtype=np.float64)[..., None]
    return i * inv_freq(D, base).astype(np.float64)


def rotate(x, idx, base=DEFAULT_BASE):
    """Rows x [..., D] (fp64 result) turned by their indices idx (broadcast over the leading axes)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = angles(np.asarray(idx), D, base)
    cs, sn = np.cos(ang), np.sin(ang)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * cs - b * sn, b * cs + a * sn], axis=-1)


def index_of(valid_sorted, p):
    """Number of valid positions before p (valid_sorted ascending)."""
    return int(np.searchsorted(np.asarray(valid_sorted, dtype=np.int64), p, side="left"))
