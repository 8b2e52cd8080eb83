"""Pins of the byte accounting (kivi_sink page, "How it works" item 4: sink bytes and residual fp16
bytes tracked separately, no double counting; StreamingLLM + KIVI page, "Caveats": the generation
counter reported next to the stored count).

Every expected figure below is counted by hand from the positions each case leaves valid, written
out in the comment above it; none is computed by a formula shared with ``oracle.accounting``.
Per-row and per-block byte sizes come from the storage format (include/kvq.h):

  KIVI b bits, D channels: K codes D*b/8 and V codes D*b/8 per row, V scale + zero 2*2*(D/32)
  per row, K scale + zero 2*2*D per 32-token block that still holds a compressed row.
  q2k, D channels: K codes D/4, V codes D/2, V scale 2*(D/32) per row; K RMS 2*D per block.
  TurboQuant K4/V2, D channels: K codes D/2, V codes D/4, K norm + V norm 8 per row.
"""
import numpy as np
import pytest

from oracle import accounting, cache


def _model(**kw):
    base = dict(n_layers=1, batch=1, n_q_heads=kw.get("n_kv_heads", 1))
    base.update(kw)
    return cache.CacheModel(cache.Config(**base))


def _feed(m, chunks, seed, planted=()):
    """Append fp16 N(0,1) chunks (keys of absolute positions in `planted` scaled 25x), evicting after each."""
    rng = np.random.default_rng(seed)
    cfg = m.cfg
    for n in chunks:
        P = m.P[0]
        k = rng.standard_normal((1, cfg.n_kv_heads, n, cfg.head_dim))
        v = rng.standard_normal((1, cfg.n_kv_heads, n, cfg.head_dim))
        for p in planted:
            if P <= p < P + n:
                k[:, :, p - P] *= 25.0
        k, v = k.astype(np.float16), v.astype(np.float16)
        m.select(0, k)
        m.append(0, k, v)
        m.evict(0)


def _check(m, want):
    got = accounting.account(m, 0, 0)
    assert got == want


def test_kivi2_first_n_partially_evicted_blocks():
    # P = 100, W = 40 -> lo = 60.  Valid: sinks {0, 1} + [60, 100) = 42 positions.
    # Window R = 8: [92, 100).  Bulk: [60, 92) = 32 rows in block 1 (60..63) and block 2 (64..91).
    # Block 0 holds only the two sinks among valid rows: no K metadata for it.
    # Per head: codes 32*(8+8) = 512, V meta 32*4 = 128, K meta 2 blocks * 128 = 256 -> 896; 2 heads: 1792.
    # Sinks 2 rows * 2 heads * 32 * 2 B * (K and V) = 512.  Window 8 * 2 * 32 * 4 = 2048.
    m = _model(n_kv_heads=2, head_dim=32, fmt="kivi", k_bits=2, v_bits=2, sink_mode="first_n", n_sink=2,
               window=40, residual=8, capacity=cache.default_capacity(40))
    _feed(m, [10] * 10, 1)
    assert (m.P[0], m.lo[0]) == (100, 60)
    _check(m, {"n_valid": 42, "n_compressed": 32, "n_sink": 2, "n_residual": 8, "current_length": 100,
               "compressed_bytes": 1792, "sink_fp16_bytes": 512, "residual_fp16_bytes": 2048})


def test_kivi4_topk_sinks_inside_blocks():
    # One 100-row chunk with keys at 5 and 70 planted 25x: the top-2 sinks are {5, 70}.
    # W = 40 -> lo = 60.  Valid: {5} + [60, 100) = 41 positions (70 lies inside the window range).
    # Sources: 5 and 70 sink; [92, 100) window (8); bulk [60, 92) minus {70} = 31 rows in blocks 1, 2.
    # Per head: codes 31*(16+16) = 992, V meta 31*4 = 124, K meta 2 * 128 = 256 -> 1372; 2 heads: 2744.
    # Sinks 2 * 2 * 32 * 4 = 512.  Window 8 * 2 * 32 * 4 = 2048.
    m = _model(n_kv_heads=2, head_dim=32, fmt="kivi", k_bits=4, v_bits=4, sink_mode="topk", n_sink=2,
               window=40, residual=8, capacity=160)
    _feed(m, [100], 2, planted=(5, 70))
    assert sorted(p for p, _ in m.sink_list(0, 0)) == [5, 70]
    _check(m, {"n_valid": 41, "n_compressed": 31, "n_sink": 2, "n_residual": 8, "current_length": 100,
               "compressed_bytes": 2744, "sink_fp16_bytes": 512, "residual_fp16_bytes": 2048})


def test_kivi2_block_whose_valid_rows_are_all_sinks():
    # 16 first-N sinks, W = 8, R = 0, P = 64 -> lo = 56.  Valid: [0, 16) + [56, 64) = 24.
    # Block 0's valid rows are all sinks (16..31 evicted): no K metadata.  Bulk: [56, 64) = 8 rows of
    # block 1.  Codes 8*(8+8) = 128, V meta 8*4 = 32, K meta 1 * 128 -> 288.  Sinks 16 * 32 * 4 = 2048.
    m = _model(n_kv_heads=1, head_dim=32, fmt="kivi", k_bits=2, v_bits=2, sink_mode="first_n", n_sink=16,
               window=8, residual=0, capacity=cache.default_capacity(8))
    _feed(m, [20, 12, 8, 8, 8, 8], 3)
    assert (m.P[0], m.lo[0]) == (64, 56)
    _check(m, {"n_valid": 24, "n_compressed": 8, "n_sink": 16, "n_residual": 0, "current_length": 64,
               "compressed_bytes": 288, "sink_fp16_bytes": 2048, "residual_fp16_bytes": 0})


def test_q2k_no_eviction():
    # W = 0, P = 70: valid [0, 70).  Sinks 0..3, window R = 16: [54, 70); bulk [4, 54) = 50 rows in
    # blocks 0 and 1.  Per head: codes 50*(8+16) = 1200, V scales 50*2 = 100, K RMS 2 * 64 = 128 -> 1428;
    # 2 heads: 2856.  Sinks 4 * 2 * 32 * 4 = 1024.  Window 16 * 2 * 32 * 4 = 4096.
    m = _model(n_kv_heads=2, head_dim=32, fmt="q2k", k_bits=2, v_bits=4, sink_mode="first_n", n_sink=4,
               residual=16, capacity=96)
    _feed(m, [33, 37], 4)
    _check(m, {"n_valid": 70, "n_compressed": 50, "n_sink": 4, "n_residual": 16, "current_length": 70,
               "compressed_bytes": 2856, "sink_fp16_bytes": 1024, "residual_fp16_bytes": 4096})


def test_kivi8_window_covers_every_valid_row():
    # No sinks, W = 8, R = 16, P = 50 -> lo = 42: valid [42, 50), all of it in the fp16 window
    # ([max(P - R, lo), P) = [42, 50)).  Nothing compressed, no block metadata.
    # Window 8 * 1 * 64 * 4 = 2048.
    m = _model(n_kv_heads=1, head_dim=64, fmt="kivi", k_bits=8, v_bits=8, window=8, residual=16,
               capacity=cache.default_capacity(8))
    _feed(m, [20, 10, 10, 10], 5)
    _check(m, {"n_valid": 8, "n_compressed": 0, "n_sink": 0, "n_residual": 8, "current_length": 50,
               "compressed_bytes": 0, "sink_fp16_bytes": 0, "residual_fp16_bytes": 2048})


def test_turboquant_after_eviction():
    # TurboQuant K4/V2, D = 128, first-N 2, W = 40, R = 8, P = 100: bulk [60, 92) = 32 rows.
    # Per row 64 + 32 codes + 8 norm bytes = 104 -> 3328.  Sinks 2 * 128 * 4 = 1024.  Window 8 * 512 = 4096.
    m = _model(n_kv_heads=1, head_dim=128, fmt="tq", k_bits=4, v_bits=2, sink_mode="first_n", n_sink=2,
               window=40, residual=8, capacity=cache.default_capacity(40), seed=3)
    _feed(m, [25, 25, 25, 25], 6)
    _check(m, {"n_valid": 42, "n_compressed": 32, "n_sink": 2, "n_residual": 8, "current_length": 100,
               "compressed_bytes": 3328, "sink_fp16_bytes": 1024, "residual_fp16_bytes": 4096})


@pytest.mark.parametrize("case", range(3))
def test_counts_match_enumeration_after_every_call(case):
    """The three counts partition the valid set as enumerated position by position."""
    kw = [dict(fmt="kivi", k_bits=2, v_bits=2, sink_mode="topk", n_sink=3, window=50, residual=12),
          dict(fmt="q2k", k_bits=2, v_bits=4, sink_mode="first_n", n_sink=4, window=33, residual=40),
          dict(fmt="kivi", k_bits=8, v_bits=4, sink_mode="none", n_sink=0, window=0, residual=5)][case]
    cap = cache.default_capacity(kw["window"]) + 96 if kw["window"] else 512
    m = _model(n_kv_heads=1, head_dim=32, capacity=cap, **kw)
    rng = np.random.default_rng(10 + case)
    for n in [1, 31, 2, 40, 1, 1, 64, 3]:
        _feed(m, [n], int(rng.integers(1 << 30)))
        P, lo = m.P[0], m.lo[0]
        sinks = {p for p, _ in m.sink_list(0, 0)}
        valid = sinks | set(range(lo, P))
        window = {p for p in range(max(P - kw["residual"], lo), P)} - sinks
        bulk = valid - sinks - window
        acc = accounting.account(m, 0, 0)
        assert (acc["n_valid"], acc["n_sink"], acc["n_residual"], acc["n_compressed"]) == \
            (len(valid), len(sinks), len(window), len(bulk))
