"""TurboQuant format variant (test infrastructure only).

Follows the TurboQuant spec page: "As-Built Notes" (random +-1 signs applied
before the Walsh-Hadamard transform; normalisation by the vector L2 norm),
"Step 1: Random Orthogonal Rotation", "Step 2: Lloyd-Max Scalar Quantization",
"Codebook Generation" and "Hadamard Transform Detail" (in-place butterfly with
stages 1, 2, 4, ...; scale by 1/sqrt(d) after the transform), and
"Optimization: Fused dequant-dot" for the rotated-domain decode identity.

Readings:

* Signs: sigma_i = -1 when bit 63 of the i-th output of splitmix64 (the
  generator of Steele, Lea and Flood, 2014) seeded with ``seed`` is set,
  else +1.  The page only says the signs come from a seed.
* Rotation y = c_d * FWHT(sigma * x) with c_d = fp32(1/sqrt(d)).  Its inverse
  is sigma * (c_d * FWHT(y)): the transform first, then the signs (the page's
  "same operation" holds for each factor separately, not for the product).
* Norm n = sqrt(canonical sum of squares of y) in fp32, one fp32 value per
  (token, head) for K and one for V (the page keeps two range floats; the
  as-built norm scaling needs one).  t = y / n (t = 0 when n = 0).
* Codebook: Lloyd-Max for Beta(d/2, d/2) on [0, 1], mapped to t = 2u - 1,
  stored as fp32; code = number of boundaries <= t.  The page's uniform start
  and ~20 iterations do not converge for 16 levels (cells of zero mass), so
  the iteration starts from levels spread evenly over mean +- 3 sd and runs
  until the fp32 tables are stable.

Parity: rotation pinned by orthogonality and self-inverse checks in fp64;
codebook pinned by an independent quadrature of Lloyd's fixed-point
equations, symmetry, uniqueness from a second start, and its Gaussian limit
(tests/test_oracle_tq.py).
"""

import numpy as np
from scipy.special import betainc

from .numerics import f32, sumsq_canonical

MASK64 = (1 << 64) - 1


def splitmix64(seed, n):
    """First n outputs of splitmix64 seeded with ``seed`` (python ints)."""
    x = seed & MASK64
    out = []
    for _ in range(n):
        x = (x + 0x9E3779B97F4A7C15) & MASK64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def signs(seed, d):
    """The +-1 sign diagonal as fp32 [d]."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64(seed, d)], dtype=np.float32)


def c_d(d):
    """fp32 value of 1/sqrt(d)."""
    return np.float32(1.0 / np.sqrt(float(d)))


def fwht(x):
    """Unnormalised fast Walsh-Hadamard transform over the last axis, stages len = 1, 2, ..., d/2.

    Works in the dtype of ``x`` (fp32 or fp64): each stage replaces the pair
    (u, v) = (x[i+j], x[i+j+len]) by (u + v, u - v).
    """
    x = np.array(x, copy=True)
    d = x.shape[-1]
    lead = x.shape[:-1]
    ln = 1
    while ln < d:
        y = x.reshape(lead + (d // (2 * ln), 2, ln))
        u = y[..., 0, :]
        v = y[..., 1, :]
        x = np.stack([u + v, u - v], axis=-2).reshape(lead + (d,))
        ln *= 2
    return x


def rotate(x, sgn):
    """y = c_d * FWHT(sigma * x) in fp32."""
    x = f32(x)
    return fwht(x * sgn) * c_d(x.shape[-1])


def inverse_rotate(y, sgn):
    """x = sigma * (c_d * FWHT(y)) in fp32."""
    y = f32(y)
    return sgn * (fwht(y) * c_d(y.shape[-1]))


def beta_lloyd_max(d, bits, init=None, max_iters=400000, stable_iters=100, tol=1e-13):
    """Lloyd-Max quantizer of Beta(d/2, d/2) on [0, 1], in fp64.

    Returns (boundaries_u, centroids_u, iterations).  Centroid of the cell
    (lo, hi) = E[X | lo < X < hi] = (1/2) * (I_hi(a+1, a) - I_lo(a+1, a)) /
    (I_hi(a, a) - I_lo(a, a)), a = d/2, using x * Beta(a, a) density =
    (1/2) * Beta(a+1, a) density.  Boundaries are midpoints of centroids.
    """
    a = d / 2.0
    L = 1 << bits
    mu, sd = 0.5, 1.0 / (2.0 * np.sqrt(2.0 * a + 1.0))
    if init is None:
        c = mu - 3 * sd + 6 * sd * (np.arange(L) + 0.5) / L
    else:
        c = np.array(init, dtype=np.float64)
    last32, same = None, 0
    for it in range(1, max_iters + 1):
        b = 0.5 * (c[1:] + c[:-1])
        edges = np.concatenate([[0.0], b, [1.0]])
        mass = np.diff(betainc(a, a, edges))
        mom = 0.5 * np.diff(betainc(a + 1.0, a, edges))
        new = mom / mass
        new = 0.5 * (new + (1.0 - new[::-1]))  # symmetry about 1/2
        step = np.max(np.abs(new - c))
        c = new
        cur32 = (2.0 * c - 1.0).astype(np.float32)
        same = same + 1 if (last32 is not None and np.array_equal(cur32, last32)) else 0
        last32 = cur32
        if same >= stable_iters and step < tol:
            break
    b = 0.5 * (c[1:] + c[:-1])
    b[L // 2 - 1] = 0.5
    return b, c, it


def codebook(d, bits):
    """fp32 tables in t = 2u - 1 space: (boundaries [2^b - 1], centroids [2^b])."""
    b, c, _ = beta_lloyd_max(d, bits)
    return (2.0 * b - 1.0).astype(np.float32), (2.0 * c - 1.0).astype(np.float32)


def codes_from_t(t, boundaries):
    """Code = number of boundaries <= t (the binary search of the page, ties to the upper cell)."""
    t = f32(t)
    u = np.zeros(t.shape, dtype=np.uint8)
    for bnd in boundaries:
        u += (t >= bnd).astype(np.uint8)
    return u


def pad(x, dp):
    """Rows [..., d] zero-padded to [..., dp] (the rotation width, a power of two)."""
    x = f32(x)
    if x.shape[-1] == dp:
        return x
    out = np.zeros(x.shape[:-1] + (dp,), np.float32)
    out[..., :x.shape[-1]] = x
    return out


def quantize_rows(x, sgn, boundaries, quantized=None):
    """Rows [n, d] -> (codes uint8 [n, dp], norms fp32 [n]) with dp = len(sgn) >= d: rows are zero-padded
    to dp and every rotated coordinate is coded.  Rows with quantized=False get code 0, norm 0."""
    y = rotate(pad(x, len(sgn)), sgn)
    nrm = np.sqrt(sumsq_canonical(y))
    safe = np.where(nrm > 0, nrm, np.float32(1.0))
    t = np.where(nrm[:, None] > 0, y / safe[:, None], np.float32(0.0))
    u = codes_from_t(t, boundaries)
    if quantized is not None:
        m = np.asarray(quantized, dtype=bool)
        u[~m] = 0
        nrm = np.where(m, nrm, np.float32(0.0)).astype(np.float32)
    return u, nrm.astype(np.float32)


def dequant32(u, nrm, centroids, sgn):
    """fp32 reconstruction sigma * (c_d * FWHT(n * c[u]))."""
    w = f32(nrm)[:, None] * centroids[np.asarray(u, dtype=np.intp)]
    return inverse_rotate(w, sgn)


def dequant64(u, nrm, centroids, sgn):
    """Exact (fp64) reconstruction R^T (n * c[u]) with R = H/sqrt(d) * diag(sigma)."""
    w = np.asarray(nrm, dtype=np.float64)[:, None] * centroids.astype(np.float64)[np.asarray(u, dtype=np.intp)]
    d = w.shape[-1]
    return sgn.astype(np.float64) * (fwht(w) / np.sqrt(float(d)))
