"""The plain-C99 oracle (oracle/c) against the numpy oracle: the same call sequences give the same
stored bytes, committed sinks, byte accounting and values bit for bit, the same format tables bit for
bit, and decode attention equal to fp64 rounding (the two sum in different orders), RoPE on read included.  Together with the
pins of the numpy oracle (tests/test_oracle_*.py) this pins the C oracle."""
import numpy as np
import pytest

from oracle import attention, cache, q2k, turboquant
from oracle import accounting
from oracle import c_model


def test_fp16_conversion_matches_ieee_round_to_nearest_even():
    allf16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allf16 = allf16[np.isfinite(allf16)].astype(np.float32)
    rng = np.random.default_rng(1)
    rnd = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s for s in (1e-6, 1e-3, 1.0, 1e3, 6e4)])
    # midpoints between adjacent fp16 values (ties) and values just beside them, subnormals included
    lo = np.arange(0, 0x7bff, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = np.arange(1, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    beside = np.concatenate([np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))])
    edge = np.array([65504, 65519.996, 65520, 1e6, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001, 2.0 ** -26, 1e-30,
                     0.0], np.float32)
    for x in (allf16, rnd, mid, beside, edge, -rnd, -mid, -edge):
        assert np.array_equal(c_model.f32_to_f16(x), x.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("d", [32, 64, 96, 128, 160])
def test_tables_equal_the_numpy_oracle(d):
    for bits in (2, 3, 4):
        nb, nc = turboquant.codebook(d, bits)
        cb, cc = c_model.tq_codebook(d, bits)
        assert np.array_equal(cb.view(np.uint32), nb.view(np.uint32)), (d, bits)
        assert np.array_equal(cc.view(np.uint32), nc.view(np.uint32)), (d, bits)
    for seed in (0, 7, 0x5EED0004):
        assert np.array_equal(c_model.tq_signs(seed, d), turboquant.signs(seed, d))
    th, lv = c_model.q2k_grid()
    assert np.array_equal(th.view(np.uint32), q2k.THETA.view(np.uint32))
    assert np.array_equal(lv.view(np.uint32), q2k.LEVELS.view(np.uint32))


CASES = {
    "kivi2_topk_window": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                              v_bits=2, sink_mode="topk", n_sink=3, window=100, residual=16),
    "kivi48_first_n_f32": dict(n_layers=2, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="kivi", k_bits=4,
                               v_bits=8, sink_mode="first_n", n_sink=4, residual=5, in_dtype="f32"),
    "kivi8_plain_d32": dict(n_layers=1, batch=2, n_kv_heads=1, n_q_heads=3, head_dim=32, fmt="kivi", k_bits=8,
                            v_bits=8, window=64),
    "q2k_topk": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="q2k", k_bits=2, v_bits=4,
                     sink_mode="topk", n_sink=5, residual=32),
    "q2k_first_n_window_f32": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=2, head_dim=32, fmt="q2k", k_bits=2,
                                   v_bits=4, sink_mode="first_n", n_sink=4, window=50, residual=8, in_dtype="f32"),
    "tq_k4v2": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=4, v_bits=2,
                    sink_mode="first_n", n_sink=2, seed=0x5EED0004),
    "tq_k3v2_dense_topk_window": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq",
                                      k_bits=3, v_bits=2, sink_mode="topk", n_sink=2, window=80, residual=8,
                                      tq_dense3=True, seed=5),
    "tq_k3v3_d32": dict(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=2, head_dim=32, fmt="tq", k_bits=3, v_bits=3,
                        seed=9, in_dtype="f32"),
    "tq_k4v2_d96_window": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=96, fmt="tq", k_bits=4,
                               v_bits=2, sink_mode="first_n", n_sink=2, window=70, residual=8, seed=31),
    "tq_k4v4_d160_f32": dict(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=2, head_dim=160, fmt="tq", k_bits=4,
                             v_bits=4, residual=4, in_dtype="f32", seed=32),
    "kivi4_first_n_res40_window": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="kivi",
                                       k_bits=4, v_bits=4, sink_mode="first_n", n_sink=4, window=90, residual=40),
    "kivi2_topk_window_rope": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi",
                                   k_bits=2, v_bits=2, sink_mode="topk", n_sink=3, window=100, residual=16,
                                   rope=True),
    "q2k_first_n_rope_base": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="q2k", k_bits=2,
                                  v_bits=4, sink_mode="first_n", n_sink=4, residual=8, rope=True,
                                  rope_base=500000.0),
}
SCHEDULE = [70, 1, 1, 33, 1, 20, 2, 31, 1, 17, 1]


@pytest.mark.parametrize("name", list(CASES))
def test_replay_equals_the_numpy_oracle(name):
    kw = dict(CASES[name])
    W = kw.get("window", 0)
    cap = cache.default_capacity(W) + 64 if W else 256
    cfg = cache.Config(capacity=cap, **kw)
    npm = cache.CacheModel(cfg)
    cm = c_model.CModel(cfg)
    rng = np.random.default_rng(len(name))
    dt = np.float32 if kw.get("in_dtype") == "f32" else np.float16
    B, H, D, L = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.n_layers
    mult = np.exp(rng.standard_normal((H, D)))  # channel outliers
    for step, n in enumerate(SCHEDULE):
        for layer in range(L):
            k = (rng.standard_normal((B, H, n, D)) * mult[None, :, None, :])
            if step == 0:
                k[:, :, [5, 40]] *= 25.0  # high-norm rows for the top-k sinks
            k = k.astype(dt)
            v = rng.standard_normal((B, H, n, D)).astype(dt)
            for mdl in (npm, cm):
                mdl.select(layer, k)
                mdl.append(layer, k, v)
                mdl.evict(layer)
            P, lo = cm.state(layer)
            assert (P, lo) == (npm.P[layer], npm.lo[layer])
            pos, sc, cnt = cm.sink_state(layer)
            npos, nsc, ncnt = npm.sink_state(layer)
            assert np.array_equal(pos, npos) and np.array_equal(cnt, ncnt)
            assert np.array_equal(sc.view(np.uint32), nsc.view(np.uint32))
            for b in range(B):
                assert cm.account(layer, b) == accounting.account(npm, layer, b)
                for h in range(H):
                    ci, ni = cm.image(layer, b, h), npm.image(layer, b, h)
                    for key in ("bulk", "win_k", "win_v", "sink_k", "sink_v"):
                        assert np.array_equal(ci[key], ni[key]), (step, layer, b, h, key)
        if step in (0, 3, 7, len(SCHEDULE) - 1):
            for layer in range(L):
                for b in range(B):
                    pos = sorted(npm.valid(layer, b))
                    for h in range(H):
                        for which in ("k", "v"):
                            v64, v16 = cm.values(layer, b, h, which, pos)
                            assert np.array_equal(v64, attention.stream_values(npm, layer, b, h, which, pos))
                            assert np.array_equal(v16, attention.dequant16(npm, layer, b, h, which, pos))
                q = rng.standard_normal((B, cfg.n_q_heads, D)).astype(dt)
                ref = attention.decode_attention(npm, layer, q)
                for threads in (1, 3):
                    got = cm.decode_attention(layer, q, threads=threads)
                    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_capacity_and_order_errors():
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=1, head_dim=32, sink_mode="topk", n_sink=2,
                       capacity=64)
    cm = c_model.CModel(cfg)
    k = np.zeros((1, 1, 10, 32), np.float16)
    with pytest.raises(AssertionError, match="select"):
        cm.append(0, k, k)
    cm.select(0, k)
    cm.append(0, k, k)
    big = np.zeros((1, 1, 60, 32), np.float16)
    cm.select(0, big)
    with pytest.raises(AssertionError, match="capacity"):
        cm.append(0, big, big)
