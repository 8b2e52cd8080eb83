"""Pins of sink selection (kivi_sink page: 'How it works', 'Fidelity to the paper', 'Evidence')."""
import json
import os

import numpy as np

from oracle import cache, kivi, sinks

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_score_is_mean_key_norm():
    rng = np.random.default_rng(40)
    k = rng.standard_normal((8, 50, 128)).astype(np.float32)
    s = sinks.token_scores(k)
    ref = np.linalg.norm(k.astype(np.float64), axis=2).mean(0)
    assert np.allclose(s, ref, rtol=2e-6)


def test_single_call_equals_brute_force_topk_with_position_tiebreak():
    rng = np.random.default_rng(41)
    sc = rng.integers(0, 6, size=40).astype(np.float32)  # many ties
    C = sinks.topk_commit([], range(100, 140), sc, 7)
    brute = sorted(range(40), key=lambda i: (-sc[i], i))[:7]
    assert [p for p, _ in C] == [100 + i for i in brute]


def test_rows_one_per_call_fill_in_arrival_order_and_are_never_restored():
    C = []
    for p, s in enumerate([1.0, 5.0, 2.0, 9.0, 100.0]):
        C = sinks.topk_commit(C, [p], [s], 3)
    assert [p for p, _ in C] == [0, 1, 2]  # a full set is permanent: later high-norm rows stay quantized


def test_committed_count_is_min_of_n_sink_and_rows_seen():
    # |C'| = |C| + min(n_sink - |C|, new rows in the merged top-k) and the merged top-k holds at least
    # min(n_sink, |C| + n) - |C| new rows, so |C| = min(n_sink, P) after every call: the set is full
    # (and every later call a no-op) exactly once n_sink rows have arrived
    rng = np.random.default_rng(43)
    for trial in range(200):
        K = int(rng.integers(1, 17))
        C, P = [], 0
        for _ in range(int(rng.integers(1, 8))):
            n = int(rng.integers(1, 9))
            sc = rng.integers(0, 4, size=n).astype(np.float32)  # ties with the committed scores too
            C = sinks.topk_commit(C, range(P, P + n), sc, K)
            P += n
            assert len(C) == min(K, P), (trial, K, P, len(C))


def test_displaced_row_rule():
    # C = {a}; a later call with 10 stronger rows commits 4 of them (in rank order) and C is full
    C = sinks.topk_commit([], [0], [1.0], 5)
    C = sinks.topk_commit(C, range(1, 11), np.arange(10, 0, -1, dtype=np.float32) + 10, 5)
    assert [p for p, _ in C] == [0, 1, 2, 3, 4]


def test_planted_sinks_recovered_and_key_mse_improves():
    g = json.load(open(os.path.join(GOLD, "kivi_sink_planted.json")))
    rng = np.random.default_rng(42)
    B, H, T, D = 2, 4, 1024, 64
    k = rng.standard_normal((B, H, T, D)).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    planted = [sorted(rng.choice(np.arange(40, T), g["n_sink_tokens"], replace=False)) for _ in range(B)]
    for b in range(B):
        k[b, :, planted[b]] = (k[b, :, planted[b]].astype(np.float32) * g["planted_magnitude"]).astype(np.float16)
    base = dict(n_layers=1, batch=B, n_kv_heads=H, n_q_heads=H, head_dim=D, fmt="kivi",
                k_bits=g["bit_width_inlier"], v_bits=g["bit_width_inlier"], residual=0, capacity=T)
    models = {}
    for mode, ns in [("none", 0), ("topk", g["n_sink_tokens"]), ("first_n", g["n_sink_tokens"])]:
        m = cache.CacheModel(cache.Config(sink_mode=mode, n_sink=ns, **base))
        m.select(0, k)
        m.append(0, k, v)
        models[mode] = m
    for b in range(B):
        got = sorted(p for p, _ in models["topk"].C[0][b])
        assert got == [int(p) for p in planted[b]]
    from oracle import attention
    pos = list(range(T))
    err = {}
    for mode, m in models.items():
        e = 0.0
        for b in range(B):
            for h in range(H):
                kh = attention.stream_values(m, 0, b, h, "k", pos)
                e += ((kh - k[b, h].astype(np.float64)) ** 2).sum()
        err[mode] = e
    # sink protection lowers key MSE; dynamic selection beats first-N when sinks are not at the front
    assert err["topk"] < err["none"] and err["topk"] < err["first_n"]


def test_zero_sinks_reproduce_plain_kivi_bytes():
    rng = np.random.default_rng(43)
    B, H, T, D = 1, 2, 200, 64
    k = rng.standard_normal((B, H, T, D)).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    cfg = cache.Config(n_layers=1, batch=B, n_kv_heads=H, n_q_heads=H, head_dim=D, fmt="kivi", k_bits=2,
                       v_bits=2, sink_mode="topk", n_sink=0, capacity=256)
    m = cache.CacheModel(cfg)
    m.select(0, k)
    m.append(0, k, v)
    img = m.image(0, 0, 1)
    # plain KIVI written without any sink machinery: per-block K, per-token V
    x = k[0, 1].astype(np.float32)
    for blk in range(7):
        rows = x[32 * blk: 32 * blk + 32]
        n = rows.shape[0]
        pad = np.zeros((32, D), np.float32)
        pad[:n] = rows
        codes, s16, z16 = kivi.quantize_k_block(pad, np.arange(32) < n, 2)
        from oracle import layout
        assert np.array_equal(img["bulk"][blk, :32 * D * 2 // 8], layout.pack_k_rows(codes, 2))
        off, size, _ = layout.record_sections("kivi", D, 2, 2)
        km = img["bulk"][blk, off["k_meta"]:off["k_meta"] + size["k_meta"]].view("<u2")
        assert np.array_equal(km[:D], s16) and np.array_equal(km[D:], z16)
