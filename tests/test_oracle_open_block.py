"""Pin of the open-block reading (oracle.cache.Config.defers_open_block): block formats with fp16 input and
an fp16 window of at least one block quantize a block once, when its last row arrives; until then its
record is zero bytes.  Against the re-quantize-on-every-append rule (the same cache with a window of 16
rows): every ring slot holds the same bytes at every step except the open block's, which is zero here and
the partial quantization there, and once a block completes both rules store the same record.  The values
the cache serves never come from an open block's record when the window covers the block (the window
rows are served first), so decode attention and dequantized values do not depend on the rule."""
import numpy as np
import pytest

from oracle import attention, cache

G = cache.G
SCHEDULE = [45, 1, 1, 17, 1, 31, 1, 1, 64, 3, 1]


@pytest.mark.parametrize("fmt,kb,vb", [("kivi", 2, 2), ("kivi", 4, 8), ("q2k", 2, 4)])
def test_open_block_is_zero_until_complete(fmt, kb, vb):
    kw = dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt=fmt, k_bits=kb, v_bits=vb,
              sink_mode="topk", n_sink=3, window=150, capacity=cache.default_capacity(150) + 96)
    defer = cache.CacheModel(cache.Config(residual=32, **kw))
    eager = cache.CacheModel(cache.Config(residual=16, **kw))
    assert defer.cfg.defers_open_block and not eager.cfg.defers_open_block
    assert not cache.Config(residual=32, in_dtype="f32", **kw).defers_open_block
    rng = np.random.default_rng(3)
    completed = 0
    for n in SCHEDULE:
        k = (rng.standard_normal((1, 2, n, 64)) * np.exp(rng.standard_normal(64))).astype(np.float16)
        v = rng.standard_normal((1, 2, n, 64)).astype(np.float16)
        for m in (defer, eager):
            m.select(0, k)
            m.append(0, k, v)
            m.evict(0)
        P = defer.P[0]
        open_slot = ((P - 1) // G) % defer.cfg.cap_blocks if P % G else -1
        for h in range(2):
            a, b = defer.image(0, 0, h)["bulk"], eager.image(0, 0, h)["bulk"]
            for slot in range(a.shape[0]):
                if slot == open_slot:
                    assert not a[slot].any() and b[slot].any()
                else:
                    assert np.array_equal(a[slot], b[slot]), (P, h, slot)
        completed += P % G == 0
        # every valid position of the open block is served from the window
        lo = defer.lo[0]
        for p in range(max(lo, P - P % G), P):
            assert p >= P - defer.cfg.residual
    assert completed >= 2


def test_values_do_not_depend_on_the_rule():
    kw = dict(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=2, head_dim=32, fmt="kivi", k_bits=2, v_bits=2,
              residual=32, capacity=256)
    m = cache.CacheModel(cache.Config(**kw))
    rng = np.random.default_rng(5)
    for n in (40, 1, 7):
        k = rng.standard_normal((1, 1, n, 32)).astype(np.float16)
        m.append(0, k, k)
    P = m.P[0]
    pos = list(range(P))
    vals = attention.stream_values(m, 0, 0, 0, "k", pos)
    k_all = np.concatenate([m.K[0][0, 0, :P]], axis=0)
    # the open block's rows (and the rest of the window) come back exactly as handed over
    assert np.array_equal(vals[P - 32:], k_all[P - 32:].astype(np.float64))
