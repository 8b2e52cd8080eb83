"""GPU parity of causal prefill attention (kvq_prefill_attn) against the oracle, through the C ABI.

Bar: for every (b, query head, query) row, ||o - o_ref||_inf / ||o_ref||_inf <= 1e-3 (the decode
attention bar); rows whose query has no valid position are zeros on both sides, exactly.  Cases
cover GQA ratios 1, 2, 3 (padding columns), 4 and 8, head_dim 32, 64 and 128 (and TurboQuant's padded
96 and 160), KIVI widths, q2k and
TurboQuant (every K/V width pair: rotated queries, rotated fp16 rows, outputs rotated back), top-k
and first-n sinks, the fp16 window, an evicting ring (early queries whose own rows are gone),
several query tiles per stream and a chunk that starts inside an open block.
"""
import numpy as np
import pytest
import torch

from harness import TOL_ATTN, Pair, stable_seed
from oracle import attention as oattn
from quantized_kv_cache_kivi_amd import synth

pytestmark = pytest.mark.gpu

CASES = {
    "kivi2_r4_topk_res16": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                                 v_bits=2, sink_mode="topk", n_sink=3, residual=16, capacity=1024), [70, 100, 1, 33]),
    "q2k_r8_firstn_res40": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="q2k", k_bits=2,
                                 v_bits=4, sink_mode="first_n", n_sink=4, residual=40, capacity=1024), [200, 64, 7]),
    # q2k runs 8 waves of one column tile: at head_dim 32 a staging thread holds one channel pair
    "q2k_r2_d32_ring": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=32, fmt="q2k", k_bits=2,
                             v_bits=4, sink_mode="first_n", n_sink=2, window=64, residual=8), [60, 20, 33]),
    "q2k_r3_d64_topk": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=6, head_dim=64, fmt="q2k", k_bits=2,
                             v_bits=4, sink_mode="topk", n_sink=3, residual=16, capacity=1024), [90, 33]),
    "kivi4_r2_d64_ring": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="kivi", k_bits=4,
                               v_bits=4, sink_mode="first_n", n_sink=2, window=32, residual=8), [60, 20, 33]),
    "kivi2_r4_ring_nosink": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                                  v_bits=2, window=32, residual=4), [50, 30]),
    "kivi8_r1_d32": (dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="kivi", k_bits=8, v_bits=8,
                          residual=0, capacity=1024), [300, 45]),
    "kivi24_r3_topk": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=6, head_dim=128, fmt="kivi", k_bits=2,
                            v_bits=4, sink_mode="topk", n_sink=5, residual=0, capacity=1024), [90, 250]),
    "tq42_r4_topk_res16": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=4,
                                v_bits=2, sink_mode="topk", n_sink=3, residual=16, capacity=1024), [70, 100, 1, 33]),
    "tq22_r2_d64_ring": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq", k_bits=2,
                              v_bits=2, sink_mode="first_n", n_sink=2, window=32, residual=8), [60, 20, 33]),
    "tq44_r1_d32": (dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="tq", k_bits=4, v_bits=4,
                         residual=0, capacity=1024), [150, 45]),
    "tq32_r4_topk": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=3, v_bits=2,
                          sink_mode="topk", n_sink=3, residual=16, capacity=1024), [70, 33]),
    "tq43_r2_d64": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq", k_bits=4, v_bits=3,
                         residual=8, capacity=1024), [90, 20]),
    "tq33_dense_r2_d64": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="tq", k_bits=3,
                               v_bits=3, sink_mode="first_n", n_sink=2, residual=8, capacity=1024, tq_dense3=True),
                          [90, 20]),
    "tq32_dense_r4_d32": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=8, head_dim=32, fmt="tq", k_bits=3,
                               v_bits=2, residual=0, capacity=1024, tq_dense3=True), [70, 33]),
    "tq24_r8_firstn": (dict(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=8, head_dim=128, fmt="tq", k_bits=2,
                            v_bits=4, sink_mode="first_n", n_sink=4, residual=40, capacity=1024), [200, 7]),
    # fp32 input: queries staged through LDS as fp16 hi + lo
    "kivi2_r4_topk_f32": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                               v_bits=2, sink_mode="topk", n_sink=3, residual=16, capacity=1024, in_dtype="f32"),
                          [70, 300, 1, 33]),
    "kivi8_r1_d32_f32_ring": (dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="kivi", k_bits=8,
                                   v_bits=8, sink_mode="first_n", n_sink=2, window=64, residual=8, in_dtype="f32"),
                              [60, 20, 33]),
    "q2k_r2_d64_f32": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="q2k", k_bits=2,
                            v_bits=4, residual=40, capacity=1024, in_dtype="f32"), [100, 7]),
    "tq42_r4_f32": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=4, v_bits=2,
                         sink_mode="first_n", n_sink=2, residual=16, capacity=1024, in_dtype="f32"), [90, 20]),
    # head_dim 96: queries and outputs of 96 channels, rows padded to 128 for the rotation
    "tq42_r4_d96": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=96, fmt="tq", k_bits=4, v_bits=2,
                         sink_mode="first_n", n_sink=2, residual=16, capacity=1024, seed=23), [70, 33]),
    "tq44_r2_d96_f32_ring": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=96, fmt="tq", k_bits=4,
                                  v_bits=4, window=64, residual=8, in_dtype="f32", seed=24), [60, 20, 33]),
    # head_dim 160: queries and outputs of 160 channels, rows padded to 256 (sixteen 16-channel tiles)
    "tq42_r4_d160": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=160, fmt="tq", k_bits=4,
                          v_bits=2, sink_mode="first_n", n_sink=2, residual=16, capacity=1024, seed=28), [70, 33]),
    "tq33_dense_r2_d160_f32_ring": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=160, fmt="tq",
                                         k_bits=3, v_bits=3, window=64, residual=8, in_dtype="f32", seed=29,
                                         tq_dense3=True), [60, 20, 33]),
}


def _log(*a):
    print(*a, flush=True)


def _check(pair, n, seed):
    c = pair.ocfg
    q = synth.normal((c.batch, c.n_q_heads, n, c.head_dim), pair.seed, 70_000 + seed, "cuda")
    q = (q.float() if c.in_dtype == "f32" else q.half()).contiguous()
    out = torch.full((c.batch, c.n_q_heads, n, c.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    pair.gpu.kvq_prefill_attn(0, q, out)
    torch.cuda.synchronize()
    ref = oattn.prefill_attention(pair.model, 0, q.cpu().numpy())
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), "non-finite outputs"
    den = np.abs(ref).max(axis=-1)
    empty = den == 0
    assert np.array_equal(got[empty], ref[empty]), "queries without valid positions must give zeros"
    err = np.abs(got - ref).max(axis=-1)[~empty] / den[~empty]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL_ATTN, f"prefill attention rel err {worst:.3e}"
    return worst, int(empty.sum())


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(name):
    kw, chunks = CASES[name]
    pair = Pair(data_seed=stable_seed(name), **kw)
    rng = np.random.default_rng(7)
    worst = 0.0
    for step, n in enumerate(chunks):
        mult = torch.from_numpy(6.0 ** rng.random((kw["n_kv_heads"], kw["head_dim"]))).cuda()
        planted = None
        if kw.get("sink_mode") == "topk" and step == 0:
            planted = [(b, [int(x) for x in rng.choice(n, 2, replace=False)]) for b in range(kw["batch"])]
        pair.push(0, n, k_mult=mult, planted=planted)
        err, nempty = _check(pair, n, step)
        worst = max(worst, err)
        _log(f"[{name}] chunk {step} n={n} P={pair.model.P[0]}: rel err {err:.2e}, empty queries {nempty}")
    _log(f"[{name}] worst {worst:.3e}")


def test_prefill_rejects_bad_calls():
    from quantized_kv_cache_kivi_amd import kvq
    kw, _ = CASES["kivi2_r4_topk_res16"]
    pair = Pair(data_seed=3, **kw)
    pair.push(0, 40)
    c = pair.ocfg
    q = torch.zeros((c.batch, c.n_q_heads, 41, c.head_dim), dtype=torch.float16, device="cuda")
    out = torch.zeros((c.batch, c.n_q_heads, 41, c.head_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvq_prefill_attn(0, q, out)  # more queries than appended positions
    assert e.value.status == -2
    buf = torch.zeros(c.batch * c.n_q_heads * 10 * c.head_dim + 1, dtype=torch.float16, device="cuda")
    qmis = buf[1:].view(c.batch, c.n_q_heads, 10, c.head_dim)  # 2-byte aligned only
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvq_prefill_attn(0, qmis, out[:, :, :10].contiguous())
    assert e.value.status == -1
