"""kvq_decode_step (select + append of one row + evict + decode attention in one call) against the four
separate calls, through the C ABI: on the same inputs, two GPU caches, one driven by the separate calls
and one by kvq_decode_step, end every step with bit-identical outputs and bit-identical stored bytes
(bulk records, staging rows, fp16 window, sink pool and sink state), and the separate-call cache stays
equal to the oracle (stored bytes bit-exact, attention within 1e-3).  The schedules cross block
boundaries (steps that open a block, which the fused launch handles, and steps that complete one, which
run as separate launches), start from an empty cache in top-k mode (rows committed as sinks run as
separate launches), and cover KIVI-2/4, q2k, RoPE on read, and configurations that never fuse
(TurboQuant, also at head_dim 160; a window shorter than a block, fp32 input)."""
import numpy as np
import pytest
import torch

from harness import TOL_ATTN, Pair, stable_seed

pytestmark = pytest.mark.gpu

CASES = {
    "kivi2_topk5_res32_win96": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi",
                                     k_bits=2, v_bits=2, sink_mode="topk", n_sink=5, window=96, residual=32),
                                70, 70),
    "q2k_firstn4_res128": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="q2k", k_bits=2,
                                v_bits=4, sink_mode="first_n", n_sink=4, residual=128, capacity=512), 150, 40),
    "kivi4_res40_win150_rope": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=128, fmt="kivi",
                                     k_bits=4, v_bits=4, window=150, residual=40, rope=True), 3, 70),
    "kivi2_topk3_from_empty": (dict(n_layers=1, batch=2, n_kv_heads=1, n_q_heads=4, head_dim=128, fmt="kivi",
                                    k_bits=2, v_bits=2, sink_mode="topk", n_sink=3, residual=32, capacity=256),
                               0, 45),
    "tq42_res32_never_fused": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq",
                                    k_bits=4, v_bits=2, residual=32, capacity=256, seed=3), 40, 35),
    "kivi2_res16_never_fused": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi",
                                     k_bits=2, v_bits=2, sink_mode="first_n", n_sink=2, window=64, residual=16),
                                50, 35),
    "kivi2_f32_never_fused": (dict(n_layers=1, batch=1, n_kv_heads=1, n_q_heads=2, head_dim=64, fmt="kivi", k_bits=2,
                                   v_bits=2, residual=32, capacity=256, in_dtype="f32"), 20, 35),
    "tq33_d160_never_fused": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=160, fmt="tq", k_bits=3,
                                   v_bits=3, sink_mode="first_n", n_sink=2, window=96, residual=16, seed=5,
                                   tq_dense3=True), 40, 35),
}


def _regions(pair, cache):
    keep = pair.gpu
    pair.gpu = cache
    try:
        return pair.gpu_regions(0)
    finally:
        pair.gpu = keep


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_equals_separate_calls(name):
    from quantized_kv_cache_kivi_amd import kvq
    kw, n0, steps = CASES[name]
    pair = Pair(data_seed=stable_seed(name), **kw)
    fused = kvq.Cache(pair.cfg)
    c = pair.ocfg
    if n0:
        k, v = pair.rows(n0)
        for g in (pair, None):
            if g is None:
                if c.sink_mode == "topk":
                    fused.kvq_select_sinks(0, k)
                fused.kvq_append(0, k, v)
                fused.kvq_evict(0)
            else:
                pair.select(0, k)
                pair.append(0, k, v)
                pair.evict(0)
    worst = 0.0
    out_f = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
    for i in range(steps):
        k, v = pair.rows(1)
        q = pair.query(tag=i)
        pair.select(0, k)
        pair.append(0, k, v)
        pair.evict(0)
        _, out_s = pair.attention(0, q)
        fused.kvq_decode_step(0, k, v, q, out_f)
        torch.cuda.synchronize()
        assert torch.equal(out_s, out_f), f"step {i}: outputs differ"
        assert fused.kvq_get_state(0) == pair.gpu.kvq_get_state(0)
        a, b = _regions(pair, pair.gpu), _regions(pair, fused)
        for key in a:
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), f"step {i}: {key} differs"
        if i % 8 == 7 or i == steps - 1:
            pair.compare_bytes(0)
            err, _ = pair.compare_attention(0, q)
            worst = max(worst, err)
    assert worst <= TOL_ATTN
    print(f"[{name}] {steps} steps equal; worst attention error {worst:.2e}", flush=True)
