"""Pins of the whole-T KIVI cache oracle (the StreamingLLM + KIVI page's own KIVI cache).

Against the page: the byte figures of "Cache-bytes table" and "Smoke test — bare minimum"
(tests/golden/kivi_whole_bytes.json), the stored set of the StreamingLLM "Implementation" section,
V final at append, and the "Affine quantisation formula" (exact on-grid values, kept exact through
every later re-quantisation; the signed code range; brute-force nearest level; the rounding bound
of a re-quantisation that widens the range).
"""
import json
import os

import numpy as np

from oracle import kivi, kivi_whole as kw
from oracle.numerics import from_f16_bits

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kivi_whole_bytes.json")))


def _near(value, printed, unit):
    """value (bytes) rounds to the printed figure at the printed precision."""
    digits = len(str(printed).split(".")[1]) if "." in str(printed) else 0
    return abs(value / unit - printed) <= 0.5 * 10.0 ** -digits + 1e-12


def _page_model():
    m = GOLD["model"]
    return kw.WholeConfig(1, m["batch"], m["n_kv_heads"], m["n_kv_heads"], m["head_dim"], bits=8, n_sink=4,
                          window=256), m["n_layers"]


def test_cache_bytes_table_rows():
    cfg, L = _page_model()
    for row in GOLD["table"]:
        T = row["stored"]
        assert _near(L * kw.dense_bytes(cfg, T, 2), row["bf16_MB"], 1e6), row
        int8 = L * kw.stored_bytes(cfg, T)
        if "int8_KB" in row:
            assert _near(int8, row["int8_KB"], 1e3), (row, int8)
        else:
            assert _near(int8, row["int8_MB"], 1e6), (row, int8)
        if "int4_packed_MB" in row:
            assert _near(L * kw.stored_bytes(cfg, T, packed_int4=True), row["int4_packed_MB"], 1e6)
    # int4 precision in int8 storage costs exactly the int8 bytes (the table's "stored=int8 bytes" column)
    c4 = kw.WholeConfig(1, 1, 8, 8, 32, bits=4, n_sink=4, window=256)
    assert kw.stored_bytes(c4, 504) == kw.stored_bytes(cfg, 504)


def test_smoke_test_bytes_through_the_state_machine():
    """A 4-token prompt and 100 generated tokens, evicting after every append: 104 stored rows,
    691,200 bytes over 12 layers ("~691 KB at int8"); the printed 2.6 MB is the fp32 size."""
    cfg, L = _page_model()
    c = kw.WholeCache(cfg)
    rng = np.random.default_rng(0)
    s = GOLD["smoke"]
    c.append(0, rng.standard_normal((1, 8, s["prompt_tokens"], 32)), rng.standard_normal((1, 8, 4, 32)))
    c.evict(0)
    for _ in range(s["generated"]):
        c.append(0, rng.standard_normal((1, 8, 1, 32)), rng.standard_normal((1, 8, 1, 32)))
        c.evict(0)
    n = len(c.stored(0))
    assert n == 104
    assert L * kw.stored_bytes(cfg, n) == 691_200
    assert round(L * kw.stored_bytes(cfg, n) / 1e3) == s["int8_KB_approx"]
    assert _near(L * kw.dense_bytes(cfg, n, 4), s["dense_MB"], 1e6)
    assert not _near(L * kw.dense_bytes(cfg, n, 2), s["dense_MB"], 1e6)


def test_stored_set_is_first_sinks_and_last_window():
    """The page drops [sink, len - window) after each append: 4 + 256 = 260 rows after 500 tokens."""
    cfg = kw.WholeConfig(1, 1, 1, 1, 32, bits=8, n_sink=4, window=256)
    c = kw.WholeCache(cfg)
    rng = np.random.default_rng(1)
    for step in range(500):
        c.append(0, rng.standard_normal((1, 1, 1, 32)), rng.standard_normal((1, 1, 1, 32)))
        c.evict(0)
        P = step + 1
        want = list(range(min(4, P))) + list(range(max(4, P - 256), P))
        assert c.stored(0) == want
        slots = [c.slot(p) for p in want]
        assert len(set(slots)) == len(slots) and max(slots) < cfg.capacity
    assert len(c.stored(0)) == 260


def _grid_rows(rng, n, D, z, s, L, extremes):
    u = rng.integers(0, L + 1, size=(n, D))
    if extremes:
        u[0, :], u[1, :] = 0, L
    return (np.float32(z) + u.astype(np.float32) * np.float32(s)).astype(np.float32), u


def test_on_grid_values_stay_exact_through_recomputes():
    """K on one grid per channel (the first chunk holds each channel's 0 and L), V rows on a grid
    with their own extremes: every later append re-quantises the stored K, and every stored value
    must still reconstruct exactly, with codes u + qMin and the grid as metadata."""
    rng = np.random.default_rng(2)
    for bits in (8, 4):
        L = (1 << bits) - 1
        D = 32
        cfg = kw.WholeConfig(1, 1, 1, 1, D, bits=bits, n_sink=2, window=40, in_dtype="f32")
        c = kw.WholeCache(cfg)
        z, s = -0.75, 2.0 ** -5
        vals = {}
        for step, n in enumerate([5, 1, 7, 1, 30, 3, 1, 12]):
            k, uk = _grid_rows(rng, n, D, z, s, L, extremes=step == 0)
            uv = rng.integers(0, L + 1, size=(n, D))
            uv[:, 0], uv[:, 1] = 0, L
            v = (np.float32(0.5) + uv.astype(np.float32) * np.float32(2.0 ** -6)).astype(np.float32)
            P = c.P[0]
            c.append(0, k[None, None], v[None, None])
            for i in range(n):
                vals[P + i] = (k[i], v[i])
            c.evict(0)
            pos = c.stored(0)
            kx, vx = c.values(0, 0, 0, "k", pos), c.values(0, 0, 0, "v", pos)
            assert np.array_equal(kx, np.stack([vals[p][0] for p in pos]))
            assert np.array_equal(vx, np.stack([vals[p][1] for p in pos]))
            assert np.all(from_f16_bits(c.ks[0, 0, 0]) == np.float32(s))
            assert np.all(from_f16_bits(c.kz[0, 0, 0]) == np.float32(z))
            codes = c.kq[0, 0, 0][[c.slot(p) for p in pos]].astype(np.int32)
            want = np.rint((np.stack([vals[p][0] for p in pos]) - np.float32(z)) / np.float32(s)).astype(np.int32)
            assert np.array_equal(codes, want + kw.Q_MIN[bits])


def test_unchanged_metadata_codes_back_to_the_same_code():
    """A re-quantisation whose scale s and zero z equal the stored ones gives every stored code u back
    when |z| <= 2^22 s: fl(fl(u s) + z) - z, divided by s, is within 2^-24 (|z| / s + 3u) of u, below
    1/2.  Every positive fp16 scale at or above fp16(1e-5), zeros of both signs up to the bound (and
    at it), every 8-bit and 4-bit code, through the oracle's own dequantisation and codes."""
    rng = np.random.default_rng(11)
    s_bits = np.arange(0x0001, 0x7C00, dtype=np.uint16)
    s_bits = s_bits[from_f16_bits(s_bits) >= np.float32(np.float16(1e-5))]
    for bits in (8, 4):
        L = (1 << bits) - 1
        u = np.arange(L + 1, dtype=np.int16)
        for chunk in np.array_split(s_bits, 64):
            sv = from_f16_bits(chunk).astype(np.float64)
            bound = np.minimum(4194304.0 * sv, 65504.0)
            # zeros: the bound itself (rounded down into fp16), half of it, random fractions, 0, both signs
            zs = np.stack([bound, 0.5 * bound, rng.random(chunk.size) * bound, np.zeros(chunk.size)], 1)
            zs = np.concatenate([zs, -zs], 1)
            z16 = np.float16(zs).view(np.uint16)
            over = np.abs(from_f16_bits(z16).astype(np.float64)) > 4194304.0 * sv[:, None]
            z16 = np.where(over, np.float16(np.nextafter(np.float16(zs), np.float16(0))).view(np.uint16), z16)
            for j in range(z16.shape[1]):
                x = kivi.affine_dequant32(u[None, :], chunk[:, None], z16[:, j, None])
                back = kivi.affine_codes(x, chunk[:, None], z16[:, j, None], bits)
                assert np.array_equal(back.astype(np.int16), np.broadcast_to(u, back.shape)), (bits, j)


def test_signed_code_range():
    rng = np.random.default_rng(3)
    for bits, lo_, hi_ in ((8, -128, 127), (4, -8, 7)):
        cfg = kw.WholeConfig(1, 1, 2, 2, 64, bits=bits, capacity=256)
        c = kw.WholeCache(cfg)
        c.append(0, rng.standard_normal((1, 2, 100, 64)), rng.standard_normal((1, 2, 100, 64)))
        for arr in (c.kq[0, 0, :, :100], c.vq[0, 0, :, :100]):
            assert arr.min() == lo_ and arr.max() == hi_


def test_codes_are_the_nearest_level_by_brute_force():
    """Codes of a single chunk against every level of the stored grid (ties excepted)."""
    rng = np.random.default_rng(4)
    for bits in (8, 4):
        L = (1 << bits) - 1
        cfg = kw.WholeConfig(1, 1, 1, 1, 32, bits=bits, capacity=64, in_dtype="f32")
        c = kw.WholeCache(cfg)
        k = (rng.standard_normal((20, 32)) * 3).astype(np.float32)
        v = (rng.standard_normal((20, 32)) * 3).astype(np.float32)
        c.append(0, k[None, None], v[None, None])
        s, z = from_f16_bits(c.ks[0, 0, 0]).astype(np.float64), from_f16_bits(c.kz[0, 0, 0]).astype(np.float64)
        for t in range(20):
            for ch in range(32):
                levels = np.arange(L + 1) * s[ch] + z[ch]
                d = np.abs(levels - float(k[t, ch]))
                best = np.flatnonzero(d <= d.min() + 1e-12 * max(1.0, abs(float(k[t, ch]))))
                assert int(c.kq[0, 0, 0, t, ch]) - kw.Q_MIN[bits] in best
            sv, zv = float(from_f16_bits(c.vs[0, 0, 0, t])), float(from_f16_bits(c.vz[0, 0, 0, t]))
            for ch in range(32):
                d = np.abs(np.arange(L + 1) * sv + zv - float(v[t, ch]))
                best = np.flatnonzero(d <= d.min() + 1e-12 * max(1.0, abs(float(v[t, ch]))))
                assert int(c.vq[0, 0, 0, t, ch]) - kw.Q_MIN[bits] in best
        # the per-channel K grid spans the chunk: zero = fp16(min), zero + L*scale >= max up to fp16 rounding
        assert np.all(np.abs(z - k.min(0)) <= 2.0 ** -10 * np.abs(k.min(0)) + 1e-7)


def test_widening_append_moves_stored_values_by_at_most_half_a_step():
    rng = np.random.default_rng(5)
    for bits in (8, 4):
        cfg = kw.WholeConfig(1, 1, 1, 1, 64, bits=bits, capacity=128, in_dtype="f32")
        c = kw.WholeCache(cfg)
        c.append(0, rng.standard_normal((1, 1, 40, 64)).astype(np.float32), rng.standard_normal((1, 1, 40, 64)))
        before = c.values(0, 0, 0, "k")
        vbefore = c.values(0, 0, 0, "v")
        big = (rng.standard_normal((1, 1, 3, 64)) * 5).astype(np.float32)  # widens most channels
        c.append(0, big, rng.standard_normal((1, 1, 3, 64)))
        after = c.values(0, 0, 0, "k")
        s16 = from_f16_bits(c.ks[0, 0, 0]).astype(np.float64)
        z16 = from_f16_bits(c.kz[0, 0, 0]).astype(np.float64)
        L = (1 << bits) - 1
        allx = np.concatenate([before, big[0, 0]], 0).astype(np.float64)
        clamp = np.maximum(0, z16 - allx.min(0)) + np.maximum(0, allx.max(0) - (z16 + L * s16))
        bound = s16 / 2 + clamp + 1e-6 * np.abs(allx).max(0)
        assert np.all(np.abs(after - allx) <= bound[None, :])
        assert np.any(from_f16_bits(c.ks[0, 0, 0]) > 0) and not np.array_equal(after[:40], before)
        # V of the stored rows is final at append
        assert np.array_equal(c.values(0, 0, 0, "v")[:40], vbefore)


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    cfg = kw.WholeConfig(1, 2, 2, 4, 32, bits=8, n_sink=2, window=20, in_dtype="f32")
    c = kw.WholeCache(cfg)
    for n in (9, 1, 30):
        if not c.fits(0, n):
            c.evict(0)
        c.append(0, rng.standard_normal((2, 2, n, 32)), rng.standard_normal((2, 2, n, 32)))
        c.evict(0)
    out = c.decode_attention(0, np.zeros((2, 4, 32), np.float32))
    for b in range(2):
        for j in range(4):
            mean = c.values(0, b, j // 2, "v").astype(np.float64).mean(0)
            assert np.allclose(out[b, j], mean, rtol=0, atol=1e-12)
    one = kw.WholeCache(kw.WholeConfig(1, 1, 1, 1, 32, bits=4, capacity=32, in_dtype="f32"))
    one.append(0, rng.standard_normal((1, 1, 1, 32)), rng.standard_normal((1, 1, 1, 32)))
    o = one.decode_attention(0, rng.standard_normal((1, 1, 32)).astype(np.float32))
    assert np.array_equal(o[0, 0], one.values(0, 0, 0, "v")[0].astype(np.float64))
