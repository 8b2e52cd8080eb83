"""The StreamingLLM + KIVI page's own KIVI cache, K scales over the whole stored T (test infrastructure only).

Follows the StreamingLLM + KIVI page:

* "KIVI — int8/int4 KV cache with greedy-lossless decode": K is quantised per
  channel with one (scale, zero) per (batch, head, channel) shared by every
  stored token and recomputed on each append; V per token with one
  (scale, zero) per (batch, head, token) over all channels, computed once at
  append and never changed.
* "Affine quantisation formula": scale = max(1e-5, (max - min)/(qMax - qMin)),
  zero = min, qMin/qMax = -128/127 for int8 and -8/7 for int4; dequantised
  values are (q - qMin)*scale + zero with the fp16 scales cast to fp32 first
  ("The bug class the previous attempt hit", 2).
* "Storage layout": keysQ and valuesQ int8 [B, H, T, D], kScales and kZeros
  fp16 [B, H, D], vScales and vZeros fp16 [B, H, T]; int4 precision is held in
  int8 bytes.
* StreamingLLM "Implementation": after each per-layer append, once the stored
  length exceeds sink + window, the rows between the first `sink` and the last
  `window` are dropped.
* "Caveats": a new token can move a channel's min/max, so the whole K block is
  re-quantised on every append (O(T*D) per step).

Readings:

* Stored bytes are the signed code q = u + qMin (two's complement int8), with
  u = clamp(rint((x - zero)/scale), 0, qMax - qMin) against the stored fp16
  scale and zero: the block format's rounding reading (adding qMin before the
  rounding can flip a half-way tie in fp32).
* The re-quantisation reads the stored K, the only copy the page keeps: every
  stored row is dequantised with the previous (scale, zero) in fp32 (two
  roundings, no FMA), the per-channel min and max run over those values and
  the new rows, and every stored row is coded again against the new metadata.
* Every stored row counts in the K min/max, the sink rows included: the page's
  cache has no fp16 overlay.
* Eviction moves nothing.  Sink position p < n_sink lives in slot p, any other
  position p in slot n_sink + (p - n_sink) mod (capacity - n_sink), and evict
  only raises lo to P - window; the stored set is the page's (the first n_sink
  and the last window rows) without its copy.  The K metadata stays as the
  last append computed it, over the rows stored at that time.

Parity: pinned in tests/test_oracle_kivi_whole.py by the page's printed byte
figures ("Cache-bytes table", "Smoke test — bare minimum"), exact on-grid
reconstruction kept through later appends, the rounding bound of a
re-quantisation, the signed code range, and the stored set after eviction.
"""

import numpy as np

from . import kivi
from .numerics import as_input, canon0, f32

Q_MIN = {8: -128, 4: -8}


class WholeConfig:
    """Shape of the whole-T cache: n_layers, batch, n_kv_heads, n_q_heads, head_dim, bits (8 or 4),
    n_sink (first-N sinks), window (0: never evict), capacity (row slots per stream, sinks included),
    in_dtype ('f16' | 'f32')."""

    def __init__(self, n_layers, batch, n_kv_heads, n_q_heads, head_dim, bits=8, n_sink=0, window=0, capacity=0,
                 in_dtype="f16"):
        assert bits in (8, 4)
        assert n_q_heads % n_kv_heads == 0
        self.n_layers, self.batch, self.n_kv_heads, self.n_q_heads = n_layers, batch, n_kv_heads, n_q_heads
        self.head_dim, self.bits, self.n_sink, self.window, self.in_dtype = head_dim, bits, n_sink, window, in_dtype
        self.capacity = capacity if capacity > 0 else default_capacity(n_sink, window)
        assert self.capacity > n_sink

    @property
    def gqa(self):
        return self.n_q_heads // self.n_kv_heads


def default_capacity(n_sink, window):
    """Slots for the sinks, the window and one 32-row chunk beyond it, rounded up to 32."""
    assert window > 0, "a cache that never evicts needs an explicit capacity"
    return 32 * ((n_sink + window + 32 + 31) // 32)


def stored_positions(P, lo, n_sink):
    """Positions the cache holds: the first min(n_sink, P) and [max(lo, n_sink), P)."""
    return list(range(min(n_sink, P))) + list(range(max(lo, n_sink), P))


class WholeCache:
    """State machine of the whole-T cache for every layer: codes, metadata, (P, lo)."""

    def __init__(self, cfg):
        self.cfg = cfg
        c = cfg
        S = (c.n_layers, c.batch, c.n_kv_heads)
        self.kq = np.zeros(S + (c.capacity, c.head_dim), np.int8)
        self.vq = np.zeros(S + (c.capacity, c.head_dim), np.int8)
        self.ks = np.zeros(S + (c.head_dim,), np.uint16)
        self.kz = np.zeros(S + (c.head_dim,), np.uint16)
        self.vs = np.zeros(S + (c.capacity,), np.uint16)
        self.vz = np.zeros(S + (c.capacity,), np.uint16)
        self.P = [0] * c.n_layers
        self.lo = [0] * c.n_layers

    def slot(self, p):
        ns = self.cfg.n_sink
        return p if p < ns else ns + (p - ns) % (self.cfg.capacity - ns)

    def stored(self, layer):
        return stored_positions(self.P[layer], self.lo[layer], self.cfg.n_sink)

    def fits(self, layer, n):
        """The rows held between this append and the next evict fit the ring slots."""
        c, P = self.cfg, self.P[layer]
        if P + n <= c.n_sink:
            return True
        return P + n - max(self.lo[layer], c.n_sink) <= c.capacity - c.n_sink

    def _k_values(self, layer, b, h, positions):
        u = self.kq[layer, b, h][[self.slot(p) for p in positions]].astype(np.int16) - Q_MIN[self.cfg.bits]
        return kivi.affine_dequant32(u, self.ks[layer, b, h], self.kz[layer, b, h])

    def _v_values(self, layer, b, h, positions):
        sl = [self.slot(p) for p in positions]
        u = self.vq[layer, b, h][sl].astype(np.int16) - Q_MIN[self.cfg.bits]
        return kivi.affine_dequant32(u, self.vs[layer, b, h][sl][:, None], self.vz[layer, b, h][sl][:, None])

    def append(self, layer, k, v):
        """k, v: [B, H, n, D] as handed over (fp16 or fp32).  Re-quantises K over every stored row plus
        the new ones, quantises the new V rows, stores the new rows."""
        c = self.cfg
        k = as_input(k, c.in_dtype)
        v = as_input(v, c.in_dtype)
        n = k.shape[2]
        assert n >= 1 and self.fits(layer, n), "the append would overwrite a stored row (evict first)"
        P = self.P[layer]
        old = self.stored(layer)
        new = list(range(P, P + n))
        qmin = Q_MIN[c.bits]
        for b in range(c.batch):
            for h in range(c.n_kv_heads):
                x_old = self._k_values(layer, b, h, old) if old else np.zeros((0, c.head_dim), np.float32)
                x = np.concatenate([x_old, f32(k[b, h])], axis=0)
                mn, mx = canon0(x.min(axis=0)), canon0(x.max(axis=0))
                s16, z16 = kivi.affine_meta(mn, mx, c.bits)
                u = kivi.affine_codes(x, s16, z16, c.bits).astype(np.int16)
                self.kq[layer, b, h][[self.slot(p) for p in old + new]] = (u + qmin).astype(np.int8)
                self.ks[layer, b, h], self.kz[layer, b, h] = s16, z16
                xv = f32(v[b, h])
                vs16, vz16 = kivi.affine_meta(canon0(xv.min(axis=1)), canon0(xv.max(axis=1)), c.bits)
                uv = kivi.affine_codes(xv, vs16[:, None], vz16[:, None], c.bits).astype(np.int16)
                sl = [self.slot(p) for p in new]
                self.vq[layer, b, h][sl] = (uv + qmin).astype(np.int8)
                self.vs[layer, b, h][sl], self.vz[layer, b, h][sl] = vs16, vz16
        self.P[layer] = P + n

    def evict(self, layer):
        if self.cfg.window > 0:
            self.lo[layer] = max(self.lo[layer], self.P[layer] - self.cfg.window)

    def values(self, layer, b, h, which, positions=None):
        """fp32 dequantised rows of `positions` (default: every stored row), [len, D]."""
        positions = self.stored(layer) if positions is None else list(positions)
        return (self._k_values if which == "k" else self._v_values)(layer, b, h, positions)

    def decode_attention(self, layer, q, scale=None):
        """fp64 softmax attention of q [B, Hq, D] over every stored row; returns [B, Hq, D]."""
        c = self.cfg
        alpha = 1.0 / np.sqrt(float(c.head_dim)) if not scale else float(np.float32(scale))
        q64 = np.asarray(q).astype(np.float64)
        out = np.zeros((c.batch, c.n_q_heads, c.head_dim))
        pos = self.stored(layer)
        for b in range(c.batch):
            for g in range(c.n_kv_heads):
                kh = self.values(layer, b, g, "k", pos).astype(np.float64)
                vh = self.values(layer, b, g, "v", pos).astype(np.float64)
                for j in range(g * c.gqa, (g + 1) * c.gqa):
                    s = alpha * (kh @ q64[b, j])
                    w = np.exp(s - s.max())
                    out[b, j] = (w @ vh) / w.sum()
        return out


def stored_bytes(cfg, n_rows, packed_int4=False):
    """Bytes of one layer holding n_rows rows per (b, head), by the page's storage layout: keysQ and
    valuesQ one byte per element (half a byte when int4 is packed), kScales and kZeros fp16 per
    channel, vScales and vZeros fp16 per row."""
    per_elem = 0.5 if packed_int4 else 1.0
    codes = 2 * n_rows * cfg.head_dim * per_elem
    meta = 2 * 2 * cfg.head_dim + 2 * 2 * n_rows
    return int(cfg.batch * cfg.n_kv_heads * (codes + meta))


def dense_bytes(cfg, n_rows, elem_bytes):
    """Bytes of one layer of an unquantised K/V cache of n_rows rows (elem_bytes 2: bf16, 4: fp32)."""
    return cfg.batch * cfg.n_kv_heads * 2 * n_rows * cfg.head_dim * elem_bytes


