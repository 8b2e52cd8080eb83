"""GPU parity: the HIP library against the oracle on seeded inputs, element by element.

Bar: stored bytes (codes, packed words, metadata, fp16 overlay, sink
positions and scores) bit-exact; dequantized fp16 within 1 ulp; decode
attention max over (b, j) of ||o - o_ref||_inf / ||o_ref||_inf <= 1e-3.
Sizes span several 32-token blocks, ragged tails, ring wrap-around and the
open-block re-quantization.
"""
import numpy as np
import pytest
import torch

from harness import TOL_ATTN, Pair, stable_seed

pytestmark = pytest.mark.gpu

CASES = {
    "kivi2_topk_res16": dict(n_layers=2, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                             v_bits=2, sink_mode="topk", n_sink=3, residual=16, capacity=512),
    "kivi8_f32_firstn_ring": dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="kivi",
                                  k_bits=8, v_bits=8, sink_mode="first_n", n_sink=4, window=64, in_dtype="f32"),
    "kivi4_firstn_win_res": dict(n_layers=1, batch=3, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="kivi", k_bits=4,
                                 v_bits=4, sink_mode="first_n", n_sink=4, window=96, residual=8),
    "kivi24_nosink": dict(n_layers=1, batch=2, n_kv_heads=1, n_q_heads=16, head_dim=128, fmt="kivi", k_bits=2,
                          v_bits=4, residual=0, capacity=384),
    "q2k_firstn_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="q2k", k_bits=2,
                           v_bits=4, sink_mode="first_n", n_sink=4, residual=24, capacity=512),
    "tq42": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=4, v_bits=2,
                 capacity=512, seed=0x5EED0004),
    "tq24_topk_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq", k_bits=2,
                          v_bits=4, sink_mode="topk", n_sink=2, window=128, residual=8, seed=77),
    "fast_kivi4_r8_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="kivi", k_bits=4,
                              v_bits=4, sink_mode="first_n", n_sink=4, window=160, residual=16),
    "fast_kivi8_r2_topk": dict(n_layers=1, batch=2, n_kv_heads=3, n_q_heads=6, head_dim=128, fmt="kivi", k_bits=8,
                               v_bits=8, sink_mode="topk", n_sink=5, residual=0, capacity=512),
    "fast_kivi2_r1_win": dict(n_layers=1, batch=1, n_kv_heads=4, n_q_heads=4, head_dim=128, fmt="kivi", k_bits=2,
                              v_bits=2, window=96, residual=0),
    "fast_kivi2_topk_res200": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi",
                                   k_bits=2, v_bits=2, sink_mode="topk", n_sink=4, residual=200, capacity=512),
    "fast_q2k_r8_topk": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="q2k", k_bits=2,
                             v_bits=4, sink_mode="topk", n_sink=4, residual=40, capacity=512),
    "fast_tq42_r8_topk_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="tq", k_bits=4,
                                  v_bits=2, sink_mode="topk", n_sink=3, residual=40, capacity=512, seed=11),
    "fast_tq42_r1_win": dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=128, fmt="tq", k_bits=4,
                             v_bits=2, sink_mode="first_n", n_sink=4, window=96, residual=8, seed=12),
    "kivi28_d32_topk_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=32, fmt="kivi", k_bits=2,
                                v_bits=8, sink_mode="topk", n_sink=3, residual=8, capacity=512),
    "kivi84_d64_firstn_win": dict(n_layers=1, batch=2, n_kv_heads=3, n_q_heads=3, head_dim=64, fmt="kivi", k_bits=8,
                                  v_bits=4, sink_mode="first_n", n_sink=4, window=128, residual=4),
    "fast_tq42_r2_ring_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=128, fmt="tq", k_bits=4,
                                  v_bits=2, window=160, residual=16, seed=13),
    # 3-bit TurboQuant codes (two per byte, one bit unused): K3/V2 on the matrix-core path, the head_dim
    # 64 and 32 cases on the generic one
    "fast_tq32_r4_topk_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=3,
                                  v_bits=2, sink_mode="topk", n_sink=3, residual=24, capacity=512, seed=14),
    "tq43_d64_firstn_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq", k_bits=4,
                                v_bits=3, sink_mode="first_n", n_sink=2, window=128, residual=8, seed=15),
    "tq33_d32_f32": dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="tq", k_bits=3, v_bits=3,
                         capacity=512, in_dtype="f32", seed=16),
    # the dense 8-in-3 stream (codes straddle words; V chunks are not word-aligned at head_dim 32); dense
    # 3-bit K at a stored width of 128 runs on the matrix-core path
    "tq32_dense_r4_topk_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=3,
                                   v_bits=2, sink_mode="topk", n_sink=3, residual=24, capacity=512, seed=17,
                                   tq_dense3=True),
    "tq43_dense_d64_firstn_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq", k_bits=4,
                                      v_bits=3, sink_mode="first_n", n_sink=2, window=128, residual=8, seed=18,
                                      tq_dense3=True),
    "tq33_dense_d32_f32": dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="tq", k_bits=3,
                               v_bits=3, capacity=512, in_dtype="f32", seed=19, tq_dense3=True),
    # head_dim 96: rows zero-padded to 128 for the Walsh-Hadamard rotation, every rotated coordinate
    # coded, Beta(48, 48) codebooks; K4/V2 on the matrix-core path, the others on the generic one
    "fast_tq42_d96_r4_firstn_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=96, fmt="tq",
                                        k_bits=4, v_bits=2, sink_mode="first_n", n_sink=3, residual=24,
                                        capacity=512, seed=20),
    "tq44_d96_f32_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=96, fmt="tq", k_bits=4,
                             v_bits=4, sink_mode="first_n", n_sink=2, window=128, residual=8, in_dtype="f32",
                             seed=21),
    "tq32_dense_d96": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=6, head_dim=96, fmt="tq", k_bits=3,
                           v_bits=2, capacity=512, seed=22, tq_dense3=True),
    # head_dim 160: rows zero-padded to 256 (lanes hold four channels; the last transform stage pairs
    # channel c with c + 128 in the lane), Beta(80, 80) codebooks, generic decode
    "tq42_d160_r4_firstn_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=160, fmt="tq",
                                    k_bits=4, v_bits=2, sink_mode="first_n", n_sink=3, residual=24,
                                    capacity=512, seed=25),
    "tq33_dense_d160_f32_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=160, fmt="tq",
                                    k_bits=3, v_bits=3, sink_mode="first_n", n_sink=2, window=128, residual=8,
                                    in_dtype="f32", seed=26, tq_dense3=True),
    "tq34_d160_r3": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=6, head_dim=160, fmt="tq", k_bits=3,
                         v_bits=4, capacity=512, seed=27),
    # 3- and 4-bit V codes in 4-bit slots on the matrix-core path (V centroids from an LDS table)
    "fast_tq43_r4_topk_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=4,
                                  v_bits=3, sink_mode="topk", n_sink=3, residual=24, capacity=512, seed=28),
    "fast_tq44_r2_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=128, fmt="tq", k_bits=4,
                             v_bits=4, sink_mode="first_n", n_sink=4, window=160, residual=16, seed=29),
    "fast_tq34_r8_res": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="tq", k_bits=3,
                             v_bits=4, residual=40, capacity=512, seed=30),
    "fast_tq43_d96_r1": dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=96, fmt="tq", k_bits=4,
                             v_bits=3, sink_mode="first_n", n_sink=2, capacity=512, seed=31),
    # dense 3-bit K (three words per lane and row chunk) with 4-bit V slots, on the matrix-core path
    "fast_tq34_dense_r4_win": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=3,
                                   v_bits=4, sink_mode="first_n", n_sink=3, window=128, residual=16, seed=32,
                                   tq_dense3=True),
    # dense 3-bit V (six words per lane's chunk) on the matrix-core path
    "fast_tq33_dense_r2_topk": dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=128, fmt="tq", k_bits=3,
                                    v_bits=3, sink_mode="topk", n_sink=2, residual=8, capacity=512, seed=33,
                                    tq_dense3=True),
    "fast_tq43_dense_r8_win": dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="tq", k_bits=4,
                                   v_bits=3, sink_mode="first_n", n_sink=4, window=160, residual=24, seed=34,
                                   tq_dense3=True),
}

SCHEDULE = [70, 1, 1, 33, 1, 100, 2, 31, 1]


def _log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_parity_sequence(name):
    kw = CASES[name]
    pair = Pair(data_seed=stable_seed(name), **kw)
    rng = np.random.default_rng(5)
    layers = range(kw["n_layers"])
    D = kw["head_dim"]
    worst_attn = 0.0
    sched = SCHEDULE if not kw.get("window") else SCHEDULE + [32, 5, 27, 1, 30, 2, 31, 1, 32, 32, 7]
    for step, n in enumerate(sched):
        if kw.get("window"):
            # a windowed ring admits an append only up to the slot of the oldest live block
            cap_b, P, lo = pair.gpu.layout.cap_blocks, pair.model.P[0], pair.model.lo[0]
            n = max(1, min(n, 32 * (cap_b + lo // 32) - P))
        for layer in layers:
            mult = None
            if kw["fmt"] != "tq":
                mult = torch.from_numpy(6.0 ** rng.random((kw["n_kv_heads"], D))).cuda()
            planted = None
            if kw.get("sink_mode") == "topk" and step == 0:
                planted = [(b, [int(x) for x in rng.choice(n, 2, replace=False)]) for b in range(kw["batch"])]
            _log(f"[{name}] step {step} layer {layer} append n={n}")
            pair.push(layer, n, k_mult=mult, planted=planted)
            pair.compare_bytes(layer)
            err, _ = pair.compare_attention(layer)
            worst_attn = max(worst_attn, err)
            assert err <= TOL_ATTN, f"attention rel err {err:.3e} at step {step}"
    for layer in layers:
        for which in (0, 1):
            ulp = pair.compare_dequant(layer, which)
            assert ulp <= 1, f"dequant differs by {ulp} ulp"
    _log(f"[{name}] worst attention rel err {worst_attn:.3e}")


def test_attention_deterministic_and_scale():
    kw = CASES["kivi2_topk_res16"]
    pair = Pair(data_seed=3, **kw)
    pair.push(0, 300)
    q = pair.query()
    _, o1 = pair.attention(0, q)
    _, o2 = pair.attention(0, q)
    assert torch.equal(o1, o2)
    err, _ = pair.compare_attention(0, q, scale=0.05)
    assert err <= TOL_ATTN


def test_error_paths_are_host_checked():
    from quantized_kv_cache_kivi_amd import kvq
    kw = CASES["kivi2_topk_res16"]
    pair = Pair(data_seed=4, **kw)
    k, v = pair.rows(10)
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvq_append(0, k, v)  # TOPK append without select
    assert e.value.status == -4
    pair.select(0, k)
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvq_append(0, k[:, :, :5].contiguous(), v[:, :, :5].contiguous())  # different chunk
    assert e.value.status == -4
    pair.append(0, k, v)
    out = torch.empty((2, 2, 4, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvq_dequant(0, 0, 8, 4, out)  # past P
    assert e.value.status == -2
    ring = Pair(data_seed=4, **CASES["kivi8_f32_firstn_ring"])
    with pytest.raises(kvq.KvqError) as e:
        for _ in range(12):
            ring.push(0, 16, evict=False)  # never evicting fills the ring
    assert e.value.status == -3
    empty = Pair(data_seed=4, **CASES["tq42"])
    with pytest.raises(kvq.KvqError) as e:
        empty.attention(0)
    assert e.value.status == -2


def test_account_matches_oracle():
    from oracle import accounting
    kw = CASES["kivi4_firstn_win_res"]
    pair = Pair(data_seed=6, **kw)
    for n in (50, 1, 77, 3):
        pair.push(0, n)
    got = pair.gpu.kvq_account(0)
    ref = {k: 0 for k in got}
    for b in range(kw["batch"]):
        a = accounting.account(pair.model, 0, b)
        for k in ref:
            ref[k] += a[k] if k != "current_length" else 0
    ref["current_length"] = pair.model.P[0]
    assert got == ref
