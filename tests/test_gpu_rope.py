"""GPU parity of RoPE on read (kvq_config.rope = 1) against the oracle, through the C ABI.

Keys and queries are handed over before RoPE; decode attention (head_dim 128 fp16 KIVI with equal
widths: the matrix-core decode kernel, keys dequantized and turned in registers, the query turned
per row tile; q2k and other head_dims: the prefill kernel split over row blocks; fp32: the generic
split kernel) and prefill attention (matrix-core kernel, staged keys turned in LDS, queries as
fp16 hi + lo pairs) turn them by their index in the compressed cache.  Bar: max
over (b, query head[, query]) of ||o - o_ref||_inf / ||o_ref||_inf <= 1e-3.  Cases: KIVI-2, KIVI-4,
KIVI-8 and q2k; head_dim 32, 64, 128; GQA 1, 2, 4, 8; top-k and first-N sinks; an evicting window
(indices re-packed after eviction) and no eviction (indices = positions); fp16 and fp32 input;
a RoPE base other than the default; chunks below and above 256 rows (one and two column tiles per
wave in the prefill kernel).  Storage is unchanged by the flag (bytes compared once).
"""
import numpy as np
import pytest
import torch

from harness import TOL_ATTN, Pair, stable_seed
from oracle import attention as oattn
from quantized_kv_cache_kivi_amd import synth

pytestmark = pytest.mark.gpu

CASES = {
    "kivi2_d128_r4_topk_win96_res16": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi",
                                            k_bits=2, v_bits=2, sink_mode="topk", n_sink=3, window=96, residual=16,
                                            rope=True), [70] + [1] * 6 + [50, 1, 1]),
    "q2k_d128_r8_firstn_res40": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="q2k",
                                      k_bits=2, v_bits=4, sink_mode="first_n", n_sink=4, residual=40, capacity=512,
                                      rope=True), [200, 1, 33]),
    "kivi4_d64_r2_f32_firstn_win40": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="kivi",
                                           k_bits=4, v_bits=4, sink_mode="first_n", n_sink=2, window=40, residual=8,
                                           in_dtype="f32", rope=True, rope_base=500000.0), [60, 20, 1, 1, 1]),
    "kivi8_d32_r1_plain_positions": (dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, fmt="kivi",
                                          k_bits=8, v_bits=8, capacity=512, rope=True), [300, 1, 45]),
    # the matrix-core decode kernel (head_dim 128, fp16, KIVI with equal widths): several blocks per
    # wave, evicting windows, both sink modes, GQA 1 / 2 / 8
    "kivi4_d128_r2_firstn_win200_res24": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=128,
                                               fmt="kivi", k_bits=4, v_bits=4, sink_mode="first_n", n_sink=4,
                                               window=200, residual=24, capacity=384, rope=True), [230, 1, 70, 1, 1]),
    "kivi8_d128_r8_topk_res8": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=16, head_dim=128, fmt="kivi",
                                     k_bits=8, v_bits=8, sink_mode="topk", n_sink=6, residual=8, capacity=1024,
                                     rope=True), [500, 1, 33]),
    "kivi2_d128_r1_long_plain": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=2, head_dim=128, fmt="kivi",
                                      k_bits=2, v_bits=2, residual=0, capacity=2560, rope=True,
                                      rope_base=500000.0), [2200, 1, 64]),
}


def _log(*a):
    print(*a, flush=True)


def _prefill_err(pair, n, tag):
    c = pair.ocfg
    q = synth.normal((c.batch, c.n_q_heads, n, c.head_dim), pair.seed, 71_000 + tag, "cuda").to(pair.tdtype).contiguous()
    out = torch.full((c.batch, c.n_q_heads, n, c.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    pair.gpu.kvq_prefill_attn(0, q, out)
    torch.cuda.synchronize()
    ref = oattn.prefill_attention(pair.model, 0, q.cpu().numpy())
    got = out.cpu().numpy().astype(np.float64)
    den = np.abs(ref).max(axis=-1)
    empty = den == 0
    assert np.isfinite(got).all()
    assert np.array_equal(got[empty], ref[empty])
    err = np.abs(got - ref).max(axis=-1)[~empty] / den[~empty]
    return float(err.max()) if err.size else 0.0


@pytest.mark.parametrize("name", list(CASES))
def test_rope_decode_and_prefill(name):
    kw, chunks = CASES[name]
    pair = Pair(data_seed=stable_seed(name), **kw)
    worst_d = worst_p = 0.0
    for step, n in enumerate(chunks):
        pair.push(0, n)
        err, _ = pair.compare_attention(0)
        worst_d = max(worst_d, err)
        worst_p = max(worst_p, _prefill_err(pair, n, step))
        if step == 0:
            assert pair.compare_bytes(0) > 0
        _log(f"[{name}] step {step} n={n} P={pair.model.P[0]}: decode {err:.2e}, prefill worst {worst_p:.2e}")
    assert worst_d <= TOL_ATTN and worst_p <= TOL_ATTN
    _log(f"[{name}] worst decode {worst_d:.3e}, prefill {worst_p:.3e}")


def test_rope_rejected_with_turboquant():
    from quantized_kv_cache_kivi_amd import kvq
    cfg = kvq.make_config(1, 1, 2, 4, 128, "tq", 4, 2, capacity=64, rope=True)
    assert kvq.config_check(cfg) == -1 and "rope" in kvq.last_error()
