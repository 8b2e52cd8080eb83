"""Pins of the ring/eviction geometry, overlay and accounting
(StreamingLLM + KIVI page 'Implementation' and 'Smoke test'; q2k page 'Summary' and 'Gate';
kivi_sink page 'How it works' item 4 and 'Evidence')."""
import json
import os

import numpy as np
import pytest

from oracle import accounting, attention, cache
from oracle.numerics import to_f16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(rng, B, H, n, D, dt=np.float16):
    return rng.standard_normal((B, H, n, D)).astype(dt), rng.standard_normal((B, H, n, D)).astype(dt)


def test_streaming_cap_sink_plus_window():
    g = json.load(open(os.path.join(GOLD, "streaming_llm_cap.json")))
    W, S = g["window"], g["sink"]
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=1, head_dim=32, fmt="kivi", k_bits=8,
                       v_bits=8, sink_mode="first_n", n_sink=S, window=W, capacity=cache.default_capacity(W),
                       in_dtype="f32")
    m = cache.CacheModel(cfg)
    rng = np.random.default_rng(50)
    for step in range(g["tokens_generated"]):
        k, v = _rows(rng, 1, 1, 1, 32, np.float32)
        m.append(0, k, v)
        m.evict(0)
        P = step + 1
        valid = m.valid(0, 0)
        assert len(valid) == min(P, g["stored_cap"])
        if P >= S + W:
            assert sorted(valid) == list(range(S)) + list(range(P - W, P))
    assert cfg.capacity == 320


def test_append_without_evict_hits_capacity():
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=1, head_dim=32, window=64,
                       capacity=cache.default_capacity(64), k_bits=8, v_bits=8)
    m = cache.CacheModel(cfg)
    rng = np.random.default_rng(51)
    with pytest.raises(AssertionError, match="capacity"):
        for _ in range(200):
            m.append(0, *_rows(rng, 1, 1, 1, 32))


@pytest.mark.parametrize("fmt,kb,vb", [("kivi", 2, 2), ("q2k", 2, 4), ("tq", 4, 2)])
def test_partition_and_overlay_exact(fmt, kb, vb):
    rng = np.random.default_rng(52)
    B, H, D = 2, 2, 64
    cfg = cache.Config(n_layers=1, batch=B, n_kv_heads=H, n_q_heads=2 * H, head_dim=D, fmt=fmt, k_bits=kb,
                       v_bits=vb, sink_mode="topk", n_sink=3, window=100, residual=16,
                       capacity=cache.default_capacity(100), seed=5)
    m = cache.CacheModel(cfg)
    for n in [90, 1, 7, 40, 1, 1]:
        k, v = _rows(rng, B, H, n, D)
        m.select(0, k)
        m.append(0, k, v)
        m.evict(0)
        for b in range(B):
            src = m.valid(0, b)
            acc = accounting.account(m, 0, b)
            assert acc["n_sink"] + acc["n_residual"] + acc["n_compressed"] == acc["n_valid"] == len(src)
            assert acc["current_length"] == m.P[0]
            # sets are disjoint and cover the valid set exactly
            sink = {p for p, s in src.items() if s == "sink"}
            win = {p for p, s in src.items() if s == "window"}
            bulk = {p for p, s in src.items() if s == "bulk"}
            assert sink | win | bulk == set(src) and not (sink & win or sink & bulk or win & bulk)
            assert sink == {p for p, _ in m.sink_list(0, b)}
            # overlay reads exact fp16 over the quantized bulk
            over = sorted(sink | win)
            for h in range(H):
                got = attention.dequant16(m, 0, b, h, "k", over)
                want = to_f16_bits(m.K[0][b, h, over])
                assert np.array_equal(got, want)


def test_chunking_invariance_with_static_sinks():
    rng = np.random.default_rng(53)
    B, H, D, T = 1, 2, 64, 300
    k, v = _rows(rng, B, H, T, D)
    cfg = cache.Config(n_layers=1, batch=B, n_kv_heads=H, n_q_heads=H, head_dim=D, fmt="kivi", k_bits=4,
                       v_bits=4, sink_mode="first_n", n_sink=4, residual=8, capacity=320)
    a = cache.CacheModel(cfg)
    a.append(0, k, v)
    b = cache.CacheModel(cfg)
    for lo, hi in [(0, 5), (5, 33), (33, 64), (64, 250), (250, 251), (251, 300)]:
        b.append(0, k[:, :, lo:hi], v[:, :, lo:hi])
    for h in range(H):
        ia, ib = a.image(0, 0, h), b.image(0, 0, h)
        for key in ia:
            assert np.array_equal(ia[key], ib[key])


def test_complete_blocks_freeze_and_ring_keeps_latest():
    rng = np.random.default_rng(54)
    D = 32
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=1, head_dim=D, fmt="kivi", k_bits=8,
                       v_bits=8, window=64, capacity=cache.default_capacity(64))
    m = cache.CacheModel(cfg)
    m.append(0, *_rows(rng, 1, 1, 40, D))
    m.evict(0)
    first = m.image(0, 0, 0)["bulk"][0].copy()
    m.append(0, *_rows(rng, 1, 1, 20, D))
    m.evict(0)
    assert np.array_equal(m.image(0, 0, 0)["bulk"][0], first)  # block 0 complete: frozen
    for _ in range(4):
        m.append(0, *_rows(rng, 1, 1, 16, D))
        m.evict(0)
    P = m.P[0]
    assert P == 124 and m.lo[0] == 60 and cfg.cap_blocks == 4
    # block 3 (rows 96..123) sits in slot 3 and block 2 in slot 2; slot 0 holds block 0 until block 4 arrives
    qs = cache.quantize_stream(cfg, m.K[0][0, 0], m.V[0][0, 0], [], P)
    recs = cache.block_records(cfg, qs)
    img = m.image(0, 0, 0)["bulk"]
    assert np.array_equal(img[3], recs[3]) and np.array_equal(img[0], recs[0])


def test_tq_accounting_bytes():
    rng = np.random.default_rng(55)
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=16, n_q_heads=16, head_dim=128, fmt="tq", k_bits=4,
                       v_bits=2, capacity=64)
    m = cache.CacheModel(cfg)
    m.append(0, *_rows(rng, 1, 16, 10, 128))
    acc = accounting.account(m, 0, 0)
    assert acc["compressed_bytes"] == 10 * (1024 + 512 + 16 * 8)
