"""Pins of the oracle's fp16 conversion, canonical sum of squares and packing."""
import json
import os

import numpy as np
import torch

from oracle import layout
from oracle.numerics import canon0, from_f16_bits, sumsq_canonical, to_f16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_all_patterns_roundtrip():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = from_f16_bits(bits)
    finite = np.isfinite(f)
    assert np.array_equal(to_f16_bits(f[finite]), bits[finite])


def test_f16_rne_against_torch_on_ties_and_random():
    # every midpoint between adjacent finite fp16 values, and +-1 fp32 ulp around it
    pos = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = from_f16_bits(pos).astype(np.float64)
    hi = from_f16_bits(pos + 1).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: midpoints of fp16 neighbours are fp32-representable
    cases = [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))]
    rng = np.random.default_rng(1)
    r = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    r = r[np.isfinite(r) & (np.abs(r) < 65504)]
    cases.append(r)
    for c in cases:
        c = np.concatenate([c, -c])
        ours = to_f16_bits(c)
        ref = torch.from_numpy(c).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ours, ref)
    # ties go to the even mantissa
    assert np.all(to_f16_bits(mid) % 2 == 0)


def test_sumsq_canonical_is_the_butterfly_and_close_to_exact():
    rng = np.random.default_rng(2)
    for d in (2, 4, 32, 64, 128):
        x = rng.standard_normal((50, d)).astype(np.float32) * np.float32(3)
        got = sumsq_canonical(x)
        # the same tree written as the xor butterfly a_l <- a_l + a_{l^off} for every lane
        a = [[np.float32(v[2 * l]) * np.float32(v[2 * l]) + np.float32(v[2 * l + 1]) * np.float32(v[2 * l + 1])
              for l in range(d // 2)] for v in x]
        off = d // 4
        while off >= 1:
            a = [[np.float32(row[l] + row[l ^ off]) for l in range(d // 2)] for row in a]
            off //= 2
        assert np.array_equal(got, np.array([row[0] for row in a], np.float32))
        exact = (x.astype(np.float64) ** 2).sum(axis=1)
        assert np.all(np.abs(got - exact) <= 1e-6 * d * exact)


def test_canon_zero():
    assert to_f16_bits(canon0(np.float32(-0.0))) == 0
    assert np.signbit(np.float32(-0.0)) and not np.signbit(canon0(np.float32(-0.0)))


def test_word_interleaved_packing_worked_example():
    # 4-bit codes 1..8 in one word: even codes in the low half, odd codes in the high half
    b = layout.pack_words(np.arange(1, 9), 4)
    assert list(b) == [0x31, 0x75, 0x42, 0x86]
    # 2-bit: codes k%4 for k = 0..15: low half holds codes 0,2,..,14 = 0,2,0,2,...
    b = layout.pack_words(np.arange(16) % 4, 2)
    low = sum(((2 * k) % 4) << (2 * k) for k in range(8))
    high = sum(((2 * k + 1) % 4) << (2 * k) for k in range(8))
    assert int.from_bytes(bytes(b), "little") == low | (high << 16)
    # 8-bit: codes 10, 11, 12, 13 -> bytes [10, 12, 11, 13]
    assert list(layout.pack_words(np.array([10, 11, 12, 13]), 8)) == [10, 12, 11, 13]


def test_pack_roundtrip_all_values():
    for bits in (2, 4, 8):
        per = 32 // bits
        codes = np.arange(1 << bits).repeat(per)[: ((1 << bits) * per // per) * per]
        codes = np.resize(codes, (7, per * 4))
        assert np.array_equal(layout.unpack_words(layout.pack_words(codes, bits), bits), codes)


def test_v_tile_order_is_a_bijection():
    seen = {(layout.t_of(kg, e)) for kg in range(4) for e in range(8)}
    assert seen == set(range(32))
    rng = np.random.default_rng(3)
    for D in (32, 64, 128):
        for bits in (2, 4, 8):
            codes = rng.integers(0, 1 << bits, size=(3, 32, D)).astype(np.uint8)
            kb = layout.pack_k_rows(codes, bits)
            vb = layout.pack_v_tiles(codes, bits)
            assert kb.shape[-1] == vb.shape[-1] == 32 * D * bits // 8
            assert np.array_equal(layout.unpack_k_rows(kb, D, bits), codes)
            assert np.array_equal(layout.unpack_v_tiles(vb, D, bits), codes)


def test_v_tile_hand_position():
    # channel 17 (mu = 1, i = 1) of token 21 (kg = 1, e = 5: 16*(5//4) + 4*1 + 5%4 = 21), 4-bit, D = 128:
    # chunk 16*1 + 1 = 17 of 32 bytes; sequence index 8*1 + 5 = 13 -> word 1, in-word index 5 -> bit 16 + 4*2
    D, bits = 128, 4
    codes = np.zeros((32, D), np.uint8)
    codes[21, 17] = 0xB
    vb = layout.pack_v_tiles(codes, bits)
    nz = np.flatnonzero(vb)
    assert list(nz) == [17 * 32 + 4 + 3] and vb[nz[0]] == 0x0B  # byte 3 of word 1 holds bits 24..31
    # bits 16+8 .. 16+11 of word 1 = byte 3, low nibble


def test_v_meta_order_hand_position_and_roundtrip():
    # token 5, group 2 of D = 128 (4 groups): pair 2, group 2, second of the pair -> 2*8 + 2*2 + 1 = 21
    meta = np.zeros((32, 4), np.uint16)
    meta[5, 2] = 0xABCD
    flat = layout.pack_v_meta(meta)
    assert list(np.flatnonzero(flat)) == [21] and flat[21] == 0xABCD
    rng = np.random.default_rng(4)
    for ng in (1, 2, 4):
        m = rng.integers(0, 1 << 16, size=(3, 32, ng)).astype(np.uint16)
        f = layout.pack_v_meta(m)
        assert sorted(f.reshape(3, -1)[0].tolist()) == sorted(m[0].reshape(-1).tolist())
        assert np.array_equal(layout.unpack_v_meta(f, ng), m)


def test_record_bytes_per_token():
    # bytes per token per KV head (codes + metadata amortised over the 32-token block)
    assert layout.record_sections("kivi", 128, 2, 2)[2] == 96 * 32
    assert layout.record_sections("kivi", 128, 4, 4)[2] == 160 * 32
    assert layout.record_sections("kivi", 32, 8, 8)[2] == 72 * 32
    assert layout.record_sections("q2k", 128, 2, 4)[2] == 112 * 32
    assert layout.record_sections("tq", 128, 4, 2)[2] == 104 * 32


def test_splitmix64_published_outputs():
    from oracle import turboquant
    g = json.load(open(os.path.join(GOLD, "splitmix64_seed0.json")))
    assert [hex(v) for v in turboquant.splitmix64(g["seed"], 4)] == [hex(int(h, 16)) for h in g["outputs_hex"]]
