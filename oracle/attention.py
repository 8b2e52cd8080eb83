"""Dequantization, single-query decode attention and causal prefill attention references (test
infrastructure only).

Dequantization follows the StreamingLLM + KIVI page ("Affine quantisation
formula"; "The bug class the previous attempt hit": scales cast to fp32, K and
V dequantized before attention), the q2k page (fp16 overlay reads exact over
the quantized bulk) and the TurboQuant spec page ("Step 2": centroid lookup,
then the inverse rotation).

Attention has a plain definition, written out here in fp64:
o = sum_p softmax_p(alpha * q . k_p) v_p over the valid positions p, with the
keys and values dequantized exactly (fp64 products of the stored fp16/fp32
metadata, no intermediate rounding).  Readings: alpha = 1/sqrt(D)
unless given; query head j reads KV head j // (Hq/Hkv).

``dequant16`` is the materialisation the library's kvq_dequant returns:
the fp32 formulas above rounded once to fp16.

Parity: pinned by brute force on hand-sized caches (one token gives o = v;
equal keys give the mean of V; two tokens give a sigmoid weight) and by the
rotated-domain identity q . R^T k = (R q) . k in tests/test_oracle_attention.py;
the cache-level dequantization (``stream_values``, both paths) by on-grid rows
of every format appended across blocks, sinks, an evicting window and a
wrapping ring, which must come back exactly (KIVI, q2k V), on their planted
level times the block's fp16 RMS (q2k K) or as |c[u]| times the row
(TurboQuant, fp64 inverse) in tests/test_oracle_cache_grid.py.
"""

import numpy as np

from . import kivi, q2k, rope, turboquant
from .cache import G, quantize_stream
from .numerics import from_f16_bits, to_f16_bits


def _bulk_values(cfg, qs, which, positions, tq, exact):
    """Dequantized bulk values of ``positions`` ([m, D]): fp64 if exact else fp32."""
    pos = np.asarray(positions, dtype=np.int64)
    blk, row = pos // G, pos % G
    if which == "k":
        u = qs["k_codes"][blk, row]
        if cfg.fmt == "kivi":
            s, z = qs["k_scale"][blk], qs["k_zero"][blk]
            if exact:
                return u.astype(np.float64) * from_f16_bits(s).astype(np.float64) + from_f16_bits(z).astype(np.float64)
            return kivi.affine_dequant32(u, s, z)
        if cfg.fmt == "q2k":
            r = qs["k_rms"][blk]
            if exact:
                return q2k.LEVELS[u.astype(np.intp)].astype(np.float64) * from_f16_bits(r).astype(np.float64)
            return q2k.k_dequant32(u, r)
        n = qs["k_norm"][blk, row]
        # the inverse rotation over the padded width, then the caller's head_dim channels
        return (turboquant.dequant64 if exact else turboquant.dequant32)(u, n, tq.kc, tq.signs)[:, :cfg.head_dim]
    u = qs["v_codes"][blk, row]
    D = u.shape[1]
    if cfg.fmt == "kivi":
        s = np.repeat(qs["v_scale"][blk, row], 32, axis=1)
        z = np.repeat(qs["v_zero"][blk, row], 32, axis=1)
        if exact:
            return u.astype(np.float64) * from_f16_bits(s).astype(np.float64) + from_f16_bits(z).astype(np.float64)
        return kivi.affine_dequant32(u, s, z)
    if cfg.fmt == "q2k":
        s = np.repeat(qs["v_scale"][blk, row], 32, axis=1)
        if exact:
            return (u.astype(np.float64) - 8.0) * from_f16_bits(s).astype(np.float64)
        return q2k.v_dequant32(u, s)
    n = qs["v_norm"][blk, row]
    assert D == cfg.store_dim
    return (turboquant.dequant64 if exact else turboquant.dequant32)(u, n, tq.vc, tq.signs)[:, :cfg.head_dim]


def stream_values(model, layer, b, h, which, positions, exact=True):
    """Values the cache returns for ``positions`` of stream (layer, b, h), read priority applied.

    exact=True: fp64 exact dequantization (attention reference).
    exact=False: fp32 formulas (then rounded to fp16 by ``dequant16``).
    """
    cfg = model.cfg
    P = model.P[layer]
    src = model.valid(layer, b)
    X = (model.K if which == "k" else model.V)[layer][b, h]
    out = np.zeros((len(positions), cfg.head_dim), dtype=np.float64 if exact else np.float32)
    bulk_idx = [i for i, p in enumerate(positions) if src[p] == "bulk"]
    for i, p in enumerate(positions):
        if src[p] != "bulk":
            v16 = from_f16_bits(to_f16_bits(X[p]))
            out[i] = v16
    if bulk_idx:
        qs = quantize_stream(cfg, model.K[layer][b, h], model.V[layer][b, h],
                             [p for p, _ in model.sink_list(layer, b)], P, model.tq)
        out[bulk_idx] = _bulk_values(cfg, qs, which, [positions[i] for i in bulk_idx], model.tq, exact)
    return out


def dequant16(model, layer, b, h, which, positions):
    """fp16 bit patterns of the materialised values (what kvq_dequant returns)."""
    return to_f16_bits(stream_values(model, layer, b, h, which, positions, exact=False))


def decode_attention(model, layer, q, scale=None, batches=None, heads=None):
    """Reference single-query decode attention.

    q: [B, Hq, D] (fp16 or fp32 array as handed to the library).
    Returns fp64 [len(batches), len(heads), D].
    """
    cfg = model.cfg
    D, r = cfg.head_dim, cfg.gqa
    alpha = 1.0 / np.sqrt(float(D)) if not scale else float(np.float32(scale))
    batches = range(cfg.batch) if batches is None else batches
    heads = range(cfg.n_q_heads) if heads is None else heads
    q64 = np.asarray(q).astype(np.float64)
    out = np.zeros((len(batches), len(heads), D), dtype=np.float64)
    for bi, b in enumerate(batches):
        pos = sorted(model.valid(layer, b).keys())
        cache = {}
        for hi, j in enumerate(heads):
            g = j // r
            if g not in cache:
                kk = stream_values(model, layer, b, g, "k", pos)
                if cfg.rope:  # keys turned by their index in the compressed cache
                    kk = rope.rotate(kk, np.arange(len(pos)), cfg.rope_base)
                cache[g] = (kk, stream_values(model, layer, b, g, "v", pos))
            kh, vh = cache[g]
            qv = q64[b, j]
            if cfg.rope:  # the query sits at the last index (its own row is the last valid one)
                qv = rope.rotate(qv, rope.index_of(pos, model.P[layer] - 1), cfg.rope_base)
            s = alpha * (kh @ qv)
            s = s - s.max()
            w = np.exp(s)
            out[bi, hi] = (w @ vh) / w.sum()
    return out


def prefill_attention(model, layer, q, scale=None, batches=None, heads=None, queries=None):
    """Reference multi-query attention of a prefill chunk over the cache, causal.

    q: [B, Hq, n, D] are the queries of the last n appended positions P-n .. P-1.  Query i attends
    the valid positions p (the cache as it stands: sinks, window, bulk, read priority applied) with
    p <= P - n + i; a query with no such position yields zeros.  Readings: the valid set
    is the cache after the chunk's append and eviction; alpha and the GQA mapping are the decode
    ones.  Returns fp64 [len(batches), len(heads), len(queries), D].
    """
    cfg = model.cfg
    D, r = cfg.head_dim, cfg.gqa
    P = model.P[layer]
    q64 = np.asarray(q).astype(np.float64)
    n = q64.shape[2]
    assert 1 <= n <= P, "the queries are the last n appended positions"
    alpha = 1.0 / np.sqrt(float(D)) if not scale else float(np.float32(scale))
    batches = range(cfg.batch) if batches is None else batches
    heads = range(cfg.n_q_heads) if heads is None else heads
    queries = range(n) if queries is None else queries
    out = np.zeros((len(batches), len(heads), len(queries), D), dtype=np.float64)
    for bi, b in enumerate(batches):
        pos = np.array(sorted(model.valid(layer, b).keys()), dtype=np.int64)
        cache = {}
        for hi, j in enumerate(heads):
            g = j // r
            if g not in cache:
                kk = stream_values(model, layer, b, g, "k", list(pos))
                if cfg.rope:
                    kk = rope.rotate(kk, np.arange(len(pos)), cfg.rope_base)
                cache[g] = (kk, stream_values(model, layer, b, g, "v", list(pos)))
            kh, vh = cache[g]
            for qi, i in enumerate(queries):
                sel = pos <= P - n + i
                if not sel.any():
                    continue
                qv = q64[b, j, i]
                if cfg.rope:  # the query's index: valid positions before its own
                    qv = rope.rotate(qv, rope.index_of(pos, P - n + i), cfg.rope_base)
                out[bi, hi, qi] = softmax_attention(qv, kh[sel], vh[sel], alpha)
    return out


def softmax_attention(q, k, v, alpha):
    """Plain fp64 attention of one query over explicit K [T, D], V [T, D]."""
    s = alpha * (np.asarray(k, np.float64) @ np.asarray(q, np.float64))
    s = s - s.max()
    w = np.exp(s)
    return (w @ np.asarray(v, np.float64)) / w.sum()
