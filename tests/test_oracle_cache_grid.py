"""Cache-level round trip of on-grid inputs through the oracle's cache model.

Rows whose values lie exactly on the quantization grid of their own group are appended through
``CacheModel`` (chunks crossing 32-token blocks, sinks inside blocks, an evicting window, a ring that
wraps several times); every valid position must then come back from ``stream_values`` (fp64 and
fp32 paths) and from the stored bytes of its ring slot, decoded here by a reader written from the
storage format in include/kvq.h (not the oracle's unpackers).  A position routed to another block,
slot, metadata entry or read source fails.

* KIVI (StreamingLLM + KIVI page, "Affine quantisation formula"): every K (block, channel) and V
  (row, 32-channel group) takes values z + u*2^-6 with u spanning 0 .. 2^b - 1, so the group's
  min/max give scale 2^-6 and zero z exactly and every value reconstructs bit-exactly.
* q2k (q2k page, "Summary"): V values q*s with s = 2^-e and |q| <= 7 reaching 7, reconstructing
  exactly.  K (4-level Lloyd-Max over the block RMS) has no exactly reconstructible grid; each value
  sits on a planted level times 2^-e, and the round trip must return that level times one scale per
  (block, channel), that scale being the fp16 RMS of the block's non-sink rows (checked in fp64 here).
* TurboQuant (TurboQuant spec, "Step 1", "Step 2"): each row is R^T (nu * c[u] / |c[u]|) for planted
  codes u (R built here from scipy's Hadamard matrix and the sign vector), so the stored codes equal u
  and the fp64 reconstruction equals |c[u]| times the row.
"""
import zlib

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import attention, cache, turboquant
from oracle.numerics import from_f16_bits

G = 32
LEVELS4 = np.array([-1.5104176085, -0.4527800346, 0.4527800346, 1.5104176085])  # N(0,1) Lloyd-Max


# --- a reader of the documented storage format -------------------------------------------------
def _word_codes(buf, bits):
    """Codes of little-endian 32-bit words, code k of a word at bit 16*(k%2) + bits*(k//2)."""
    per = 32 // bits
    out = []
    for w in range(len(buf) // 4):
        word = int.from_bytes(bytes(buf[4 * w:4 * w + 4]), "little")
        for k in range(per):
            out.append((word >> (16 * (k % 2) + bits * (k // 2))) & ((1 << bits) - 1))
    return out


def _read_record(rec, fmt, D, kb, vb):
    """(K codes [32][D], V codes [32][D], K meta, V meta) of one block record."""
    kc_bytes, vc_bytes = G * D * kb // 8, G * D * vb // 8
    kseq = _word_codes(rec[:kc_bytes], kb)
    kcodes = np.array(kseq).reshape(G, D)
    vseq = _word_codes(rec[kc_bytes:kc_bytes + vc_bytes], vb)
    per_chunk = D // 2
    vcodes = np.zeros((G, D), np.int64)
    for q in range(64):
        kg, i = q // 16, q % 16
        for k in range(per_chunk):
            mu, e = k // 8, k % 8
            t = 16 * (e // 4) + 4 * kg + e % 4
            vcodes[t, 16 * mu + i] = vseq[q * per_chunk + k]
    meta = rec[kc_bytes + vc_bytes:]
    ng = D // 32
    if fmt == "kivi":
        k16 = np.frombuffer(bytes(meta[:4 * D]), "<u2")
        kmeta = (from_f16_bits(k16[:D]), from_f16_bits(k16[D:]))
        v16 = np.frombuffer(bytes(meta[4 * D:4 * D + 4 * G * ng]), "<u2")
        sc = np.array([[v16[(t // 2) * ng * 2 + g * 2 + t % 2] for g in range(ng)] for t in range(G)])
        ze = np.array([[v16[G * ng + (t // 2) * ng * 2 + g * 2 + t % 2] for g in range(ng)] for t in range(G)])
        vmeta = (from_f16_bits(sc.astype(np.uint16)), from_f16_bits(ze.astype(np.uint16)))
    elif fmt == "q2k":
        kmeta = from_f16_bits(np.frombuffer(bytes(meta[:2 * D]), "<u2"))
        v16 = np.frombuffer(bytes(meta[2 * D:2 * D + 2 * G * ng]), "<u2")
        vmeta = from_f16_bits(np.array([[v16[(t // 2) * ng * 2 + g * 2 + t % 2] for g in range(ng)]
                                        for t in range(G)]).astype(np.uint16))
    else:
        kmeta = np.frombuffer(bytes(meta[:4 * G]), "<f4")
        vmeta = np.frombuffer(bytes(meta[4 * G:8 * G]), "<f4")
    return kcodes, vcodes, kmeta, vmeta


# --- on-grid inputs --------------------------------------------------------------------------------
class GridSource:
    """Draws the rows of every position ahead of time, with the block structure of the whole run."""

    def __init__(self, fmt, bits, H, D, P_total, sinks, seed):
        rng = np.random.default_rng(seed)
        self.K = np.zeros((H, P_total, D), np.float64)
        self.V = np.zeros((H, P_total, D), np.float64)
        self.level = np.zeros((H, P_total, D), np.int64)  # q2k K: planted level; TQ: planted K codes
        self.vcode = np.zeros((H, P_total, D), np.int64)  # TQ: planted V codes
        kb, vb = bits
        nblk = -(-P_total // G)
        for h in range(H):
            for beta in range(nblk):
                rows = [p for p in range(beta * G, min(P_total, beta * G + G)) if p not in sinks]
                for p in range(beta * G, min(P_total, beta * G + G)):
                    self._draw_v(fmt, vb, h, p, rng)
                if fmt == "kivi":
                    L = (1 << kb) - 1
                    z = rng.integers(-128, 128, size=D) / 64.0
                    u = rng.integers(0, L + 1, size=(len(rows), D))
                    if len(rows) >= 2:
                        u[0], u[1] = 0, L
                    self.K[h, rows] = z + u / 64.0
                elif fmt == "q2k":
                    e = int(rng.integers(-3, 3))
                    lv = rng.choice(4, size=(len(rows), D), p=[0.2, 0.3, 0.3, 0.2])
                    if rows:
                        lv[0] = rng.choice([0, 3], size=D)  # an outer level first: keeps the inner codes inside
                    self.level[h, rows] = lv
                    self.K[h, rows] = np.float16(LEVELS4[lv] * 2.0 ** e)
            for p in sinks:
                if p < P_total:
                    self.K[h, p] = (rng.standard_normal(D) * 25.0).astype(np.float16)

    def _draw_v(self, fmt, vb, h, p, rng):
        D = self.V.shape[2]
        if fmt == "kivi":
            L = (1 << vb) - 1
            for g in range(D // 32):
                z = rng.integers(-128, 128) / 64.0
                u = rng.integers(0, L + 1, size=32)
                u[0], u[1] = 0, L
                self.V[h, p, 32 * g:32 * g + 32] = z + u / 64.0
        elif fmt == "q2k":
            for g in range(D // 32):
                e = int(rng.integers(-4, 2))
                q = rng.integers(-7, 8, size=32)
                q[int(rng.integers(32))] = 7 * (1 if rng.integers(2) else -1)
                self.V[h, p, 32 * g:32 * g + 32] = q * 2.0 ** e


def _tq_rows(codes_pool, cen, signs, nu, rng, D):
    """One row R^T (nu * c[u] / |c[u]|) with |c[u]| within 1 % of 1 (planted codes u)."""
    Hd = hadamard(D).astype(np.float64)
    while True:
        u = rng.choice(len(cen), size=D, p=codes_pool)
        c = cen[u].astype(np.float64)
        n = np.sqrt((c * c).sum())
        if abs(n - 1.0) < 0.01:
            break
    y = nu * c / n
    x = signs.astype(np.float64) * (Hd @ y) / np.sqrt(D)  # R^T y with R = H diag(signs) / sqrt(D)
    return u, x, n


@pytest.mark.parametrize("fmt,kb,vb,sink_mode", [("kivi", 2, 2, "first_n"), ("kivi", 4, 8, "topk"),
                                                 ("kivi", 8, 4, "first_n"), ("q2k", 2, 4, "topk"),
                                                 ("q2k", 2, 4, "first_n"), ("tq", 4, 2, "first_n")])
def test_on_grid_rows_round_trip_through_the_cache(fmt, kb, vb, sink_mode):
    H, D, W, R = 2, 32 if fmt != "tq" else 64, 70, 9
    chunks = [45, 1, 26, 1, 1, 25, 20, 3, 26, 1, 17, 26, 5, 24, 2, 26, 26, 9, 26, 13, 1, 26]
    P_total = sum(chunks)
    n_sink = 3 if sink_mode == "first_n" else 2
    planted = (0, 1, 2) if sink_mode == "first_n" else (7, 40)
    in_dtype = "f32" if fmt == "tq" else "f16"
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=H, n_q_heads=H, head_dim=D, fmt=fmt, k_bits=kb,
                       v_bits=vb, sink_mode=sink_mode, n_sink=n_sink, window=W, residual=R,
                       capacity=cache.default_capacity(W), in_dtype=in_dtype, seed=11)
    src = GridSource(fmt, (kb, vb), H, D, P_total, set(planted), seed=zlib.crc32(f"{fmt}{kb}{vb}{sink_mode}".encode()))
    if fmt == "tq":
        rng = np.random.default_rng(5)
        signs = turboquant.signs(cfg.seed, D)
        kbnd, kcen = turboquant.codebook(D, kb)
        vbnd, vcen = turboquant.codebook(D, vb)
        pk = np.diff(np.concatenate([[0.0], _beta_cdf(kbnd, D), [1.0]]))
        pv = np.diff(np.concatenate([[0.0], _beta_cdf(vbnd, D), [1.0]]))
        knorm = np.zeros((H, P_total))
        vnorm = np.zeros((H, P_total))
        for h in range(H):
            for p in range(P_total):
                if p in planted:
                    src.K[h, p] = rng.standard_normal(D) * 3
                    src.V[h, p] = rng.standard_normal(D)
                    continue
                src.level[h, p], src.K[h, p], knorm[h, p] = _tq_rows(pk, kcen, signs, 2.0, rng, D)
                src.vcode[h, p], src.V[h, p], vnorm[h, p] = _tq_rows(pv, vcen, signs, 0.5, rng, D)
    dt = np.float32 if in_dtype == "f32" else np.float16
    Kin = src.K.astype(dt)
    Vin = src.V.astype(dt)
    assert np.array_equal(Kin.astype(np.float64), src.K) or fmt == "tq"
    m = cache.CacheModel(cfg)
    P = 0
    _, _, rec_bytes = cache.layout.record_sections(fmt, D, kb, vb)
    for n in chunks:
        k = Kin[None, :, P:P + n]
        v = Vin[None, :, P:P + n]
        m.select(0, k)
        m.append(0, k, v)
        m.evict(0)
        P += n
        if sink_mode == "topk":
            assert sorted(p for p, _ in m.sink_list(0, 0)) == [p for p in planted if p < P]
        srcmap = m.valid(0, 0)
        pos = sorted(srcmap)
        for h in range(H):
            img = m.image(0, 0, h)["bulk"]
            x64k = Kin[h, pos].astype(np.float64)
            x64v = Vin[h, pos].astype(np.float64)
            for exact in (True, False):
                gk = attention.stream_values(m, 0, 0, h, "k", pos, exact=exact).astype(np.float64)
                gv = attention.stream_values(m, 0, 0, h, "v", pos, exact=exact).astype(np.float64)
                over = [i for i, p in enumerate(pos) if srcmap[p] != "bulk"]
                bulk = [i for i, p in enumerate(pos) if srcmap[p] == "bulk"]
                # fp16 overlay (sinks, window) reads the input rounded once to fp16
                assert np.array_equal(gk[over], Kin[h, [pos[i] for i in over]].astype(np.float16).astype(np.float64))
                assert np.array_equal(gv[over], Vin[h, [pos[i] for i in over]].astype(np.float16).astype(np.float64))
                if fmt == "kivi":
                    assert np.array_equal(gk[bulk], x64k[bulk]) and np.array_equal(gv[bulk], x64v[bulk])
                elif fmt == "q2k":
                    assert np.array_equal(gv[bulk], x64v[bulk])
                    _check_q2k_k(src, h, [pos[i] for i in bulk], gk[bulk], planted, P, m.sink_list(0, 0))
                elif exact:
                    bp = [pos[i] for i in bulk]
                    want_k = x64k[bulk] * knorm[h, bp][:, None]
                    want_v = x64v[bulk] * vnorm[h, bp][:, None]
                    assert np.abs(gk[bulk] - want_k).max() <= 2e-6 * np.abs(want_k).max()
                    assert np.abs(gv[bulk] - want_v).max() <= 2e-6 * np.abs(want_v).max()
            # stored bytes of each bulk position's ring slot, read back by the format reader
            for i, p in enumerate(pos):
                if srcmap[p] != "bulk":
                    continue
                kc, vc, km, vm = _read_record(img[(p // G) % cfg.cap_blocks], fmt, D, kb, vb)
                t = p % G
                if fmt == "kivi":
                    assert np.array_equal(kc[t] * km[0] + km[1], Kin[h, p].astype(np.float32))
                    grp = np.repeat(np.arange(D // 32), 32)
                    assert np.array_equal(vc[t] * vm[0][t][grp] + vm[1][t][grp], Vin[h, p].astype(np.float32))
                elif fmt == "q2k":
                    assert np.array_equal(kc[t], src.level[h, p])
                    grp = np.repeat(np.arange(D // 32), 32)
                    assert np.array_equal((vc[t] - 8.0) * vm[t][grp], Vin[h, p].astype(np.float32))
                else:
                    assert np.array_equal(kc[t], src.level[h, p]) and np.array_equal(vc[t], src.vcode[h, p])
                    assert abs(km[t] - 2.0) <= 1e-5 and abs(vm[t] - 0.5) <= 1e-5
    assert P > 2 * cfg.capacity  # the ring wrapped at least twice


def _check_q2k_k(src, h, bulk_pos, got, planted, P, sink_list):
    sinks = {p for p, _ in sink_list}
    by_group = {}
    for p, row in zip(bulk_pos, got):
        by_group.setdefault(p // G, []).append((p, row))
    for beta, items in by_group.items():
        lv = np.array([src.level[h, p] for p, _ in items])
        vals = np.array([row for _, row in items])
        scale = vals / LEVELS4[lv]                               # one scale per (block, channel)
        assert np.allclose(scale, scale[0][None, :], rtol=1e-6, atol=0)
        calib = [p for p in range(beta * G, min(P, beta * G + G)) if p not in sinks]
        x = src.K[h, calib].astype(np.float16).astype(np.float64)
        rms = np.sqrt((x * x).mean(axis=0))
        assert np.all(np.abs(scale[0] - rms) <= 2.0 ** -10 * rms), "scale is not the fp16 RMS of the non-sink rows"


def _beta_cdf(bnd_t, D):
    from scipy.special import betainc
    return betainc(D / 2, D / 2, (np.asarray(bnd_t, np.float64) + 1.0) / 2.0)
