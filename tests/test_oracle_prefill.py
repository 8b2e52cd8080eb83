"""Pins of the fp64 causal prefill-attention reference (multi-query attention over the cache)."""
import numpy as np

from oracle import attention, cache


def _model(fmt="kivi", kb=2, vb=2, D=32, H=2, Hq=4, residual=0, n_sink=0, sink_mode="none", window=0, cap=256):
    cfg = cache.Config(n_layers=1, batch=2, n_kv_heads=H, n_q_heads=Hq, head_dim=D, fmt=fmt, k_bits=kb, v_bits=vb,
                       residual=residual, capacity=cap, n_sink=n_sink, sink_mode=sink_mode, window=window)
    return cfg, cache.CacheModel(cfg)


def _push(m, rng, n, D, H=2):
    k = rng.standard_normal((2, H, n, D)).astype(np.float16)
    v = rng.standard_normal((2, H, n, D)).astype(np.float16)
    m.select(0, k)
    m.append(0, k, v)
    m.evict(0)
    return k, v


def test_one_query_is_decode_attention():
    rng = np.random.default_rng(90)
    cfg, m = _model(residual=8, n_sink=3, sink_mode="topk")
    _push(m, rng, 70, 32)
    q = rng.standard_normal((2, 4, 1, 32)).astype(np.float16)
    a = attention.prefill_attention(m, 0, q)[:, :, 0]
    b = attention.decode_attention(m, 0, q[:, :, 0])
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_last_query_of_a_chunk_sees_everything_valid():
    rng = np.random.default_rng(91)
    cfg, m = _model(fmt="q2k", kb=2, vb=4, D=64, residual=16)
    _push(m, rng, 45, 64)
    _push(m, rng, 50, 64)
    q = rng.standard_normal((2, 4, 50, 64)).astype(np.float16)
    a = attention.prefill_attention(m, 0, q, queries=[49])[:, :, 0]
    b = attention.decode_attention(m, 0, q[:, :, 49])
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_zero_query_is_the_causal_mean_of_values():
    # q = 0: every valid score is 0, so query i averages the values of the valid positions <= its own
    rng = np.random.default_rng(92)
    cfg, m = _model(kb=4, vb=4, residual=4, n_sink=2, sink_mode="first_n", window=48, cap=128)
    for n in (40, 30, 33):
        _push(m, rng, n, 32)
    P, n = m.P[0], 33
    q = np.zeros((2, 4, n, 32), dtype=np.float16)
    o = attention.prefill_attention(m, 0, q)
    for b in range(2):
        valid = sorted(m.valid(0, b).keys())
        for j in range(4):
            vh = attention.stream_values(m, 0, b, j // 2, "v", valid)
            for i in (0, 7, n - 1):
                sel = [t for t, p in enumerate(valid) if p <= P - n + i]
                assert np.allclose(o[b, j, i], vh[sel].mean(0), rtol=0, atol=1e-13)


def test_rows_after_a_query_do_not_reach_it():
    # rows read exact from the fp16 window: changing the last rows of the chunk leaves earlier queries
    rng = np.random.default_rng(93)
    outs = []
    for variant in range(2):
        r2 = np.random.default_rng(94)
        cfg, m = _model(residual=64, cap=128)
        k = r2.standard_normal((2, 2, 40, 32)).astype(np.float16)
        v = r2.standard_normal((2, 2, 40, 32)).astype(np.float16)
        if variant:
            k[:, :, 30:] = rng.standard_normal((2, 2, 10, 32)).astype(np.float16)
            v[:, :, 30:] = rng.standard_normal((2, 2, 10, 32)).astype(np.float16)
        m.append(0, k, v)
        q = np.random.default_rng(95).standard_normal((2, 4, 40, 32)).astype(np.float16)
        outs.append(attention.prefill_attention(m, 0, q))
    assert np.array_equal(outs[0][:, :, :30], outs[1][:, :, :30])
    assert not np.allclose(outs[0][:, :, 30:], outs[1][:, :, 30:])


def test_query_without_valid_position_gives_zeros():
    # window 32 with no sinks: after 100 rows, positions below 68 are evicted, so a query whose
    # position precedes every valid one has nothing to attend
    rng = np.random.default_rng(96)
    cfg, m = _model(window=32, cap=160)
    _push(m, rng, 60, 32)
    _push(m, rng, 40, 32)
    lo = min(m.valid(0, 0).keys())
    q = rng.standard_normal((2, 4, 40, 32)).astype(np.float16)
    o = attention.prefill_attention(m, 0, q)
    P = m.P[0]
    first_ok = lo - (P - 40)
    assert first_ok > 0 and np.all(o[:, :, :first_ok] == 0) and np.all(np.abs(o[:, :, first_ok:]).sum(-1) > 0)
