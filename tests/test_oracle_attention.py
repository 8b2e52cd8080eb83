"""Pins of the fp64 decode-attention reference (plain softmax attention over dequantized K, V)."""
import numpy as np
from scipy.special import softmax

from oracle import attention, cache


def _model(fmt="kivi", kb=8, vb=8, T=1, D=32, H=1, Hq=1, residual=0, seed=0):
    cfg = cache.Config(n_layers=1, batch=1, n_kv_heads=H, n_q_heads=Hq, head_dim=D, fmt=fmt, k_bits=kb, v_bits=vb,
                       residual=residual, capacity=64, seed=seed)
    return cfg, cache.CacheModel(cfg)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(60)
    cfg, m = _model()
    k = rng.standard_normal((1, 1, 1, 32)).astype(np.float16)
    v = rng.standard_normal((1, 1, 1, 32)).astype(np.float16)
    m.append(0, k, v)
    q = rng.standard_normal((1, 1, 32)).astype(np.float16)
    o = attention.decode_attention(m, 0, q)[0, 0]
    assert np.array_equal(o, attention.stream_values(m, 0, 0, 0, "v", [0])[0])


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(61)
    cfg, m = _model(T=20)
    k = np.repeat(rng.standard_normal((1, 1, 1, 32)).astype(np.float16), 20, axis=2)
    v = rng.standard_normal((1, 1, 20, 32)).astype(np.float16)
    m.append(0, k, v)
    q = rng.standard_normal((1, 1, 32)).astype(np.float16)
    o = attention.decode_attention(m, 0, q)[0, 0]
    vh = attention.stream_values(m, 0, 0, 0, "v", list(range(20)))
    assert np.allclose(o, vh.mean(0), rtol=0, atol=1e-12)


def test_two_tokens_sigmoid_weight():
    rng = np.random.default_rng(62)
    cfg, m = _model(residual=2)  # both rows read exact from the fp16 window
    k = rng.standard_normal((1, 1, 2, 32)).astype(np.float16)
    v = rng.standard_normal((1, 1, 2, 32)).astype(np.float16)
    m.append(0, k, v)
    q = rng.standard_normal((1, 1, 32)).astype(np.float16)
    o = attention.decode_attention(m, 0, q)[0, 0]
    k64, v64, q64 = (a.astype(np.float64) for a in (k[0, 0], v[0, 0], q[0, 0]))
    w = 1.0 / (1.0 + np.exp(-(q64 @ (k64[0] - k64[1])) / np.sqrt(32)))
    assert np.allclose(o, w * v64[0] + (1 - w) * v64[1], rtol=0, atol=1e-12)


def test_gqa_mapping_and_library_softmax():
    rng = np.random.default_rng(63)
    cfg, m = _model(fmt="q2k", kb=2, vb=4, D=64, H=2, Hq=8)
    k = rng.standard_normal((1, 2, 50, 64)).astype(np.float16)
    v = rng.standard_normal((1, 2, 50, 64)).astype(np.float16)
    m.append(0, k, v)
    q = rng.standard_normal((1, 8, 64)).astype(np.float16)
    o = attention.decode_attention(m, 0, q)
    for j in range(8):
        g = j // 4
        kh = attention.stream_values(m, 0, 0, g, "k", list(range(50)))
        vh = attention.stream_values(m, 0, 0, g, "v", list(range(50)))
        w = softmax(kh @ q[0, j].astype(np.float64) / 8.0)
        assert np.allclose(o[0, j], w @ vh, rtol=1e-12, atol=1e-12)
