"""kvq_decode_attn_nomalloc (the decode entry point for callers that cannot allocate device memory)
against kvq_decode_attn on the same caches: identical kernels and split policy, so the outputs must
be bit-identical.  Two calls in a row on one GPU, the second on a smaller cache, so the second reuses
the static workspace the first left behind; configurations whose partials exceed the static
workspace are refused before any launch."""
import pytest
import torch

from harness import Pair, stable_seed

CASES = {
    # (config, prefill rows, decode steps): the second case of each pair is the smaller input
    "kivi2_fast_gqa4": (dict(n_layers=1, batch=4, n_kv_heads=4, n_q_heads=16, head_dim=128, fmt="kivi", k_bits=2,
                             v_bits=2, sink_mode="topk", n_sink=5, residual=32, capacity=2048), 1500),
    "kivi2_fast_small": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                              v_bits=2, sink_mode="topk", n_sink=5, residual=32, capacity=256), 90),
    "q2k_fast": (dict(n_layers=1, batch=3, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="q2k", k_bits=2, v_bits=4,
                      sink_mode="first_n", n_sink=4, residual=64, capacity=1024), 700),
    "kivi4_generic_d64": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=4, head_dim=64, fmt="kivi", k_bits=4,
                               v_bits=4, sink_mode="first_n", n_sink=4, window=200, residual=16), 300),
    "tq_k4v2": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="tq", k_bits=4, v_bits=2,
                     capacity=1024, seed=7), 600),
    "rope_kivi2": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, fmt="kivi", k_bits=2,
                        v_bits=2, sink_mode="first_n", n_sink=4, residual=16, capacity=1024, rope=True), 500),
}
PAIRS = [(big, "kivi2_fast_small") for big in ("kivi2_fast_gqa4", "q2k_fast", "kivi4_generic_d64", "tq_k4v2",
                                                "rope_kivi2")]


def _filled(name):
    kw, n = CASES[name]
    pair = Pair(data_seed=stable_seed(name), **kw)
    step = 48 if kw.get("window") else n  # a windowed ring is evicted every 48 rows
    for m in [min(step, n - i) for i in range(0, n, step)] + [1]:
        pair.push(0, m, evict=bool(kw.get("window")))
    return pair


@pytest.mark.gpu
@pytest.mark.parametrize("first,second", PAIRS)
def test_nomalloc_matches_workspace_entry(first, second):
    for name in (first, second):
        print(f"[no-alloc] case {name}", flush=True)
        pair = _filled(name)
        q = pair.query()
        c = pair.ocfg
        ref = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
        got = torch.full_like(ref, float("nan"))
        pair.gpu.kvq_decode_attn(0, q, ref)
        pair.gpu.kvq_decode_attn_nomalloc(0, q, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{name}: no-alloc output differs from kvq_decode_attn"


@pytest.mark.gpu
def test_nomalloc_refuses_partials_beyond_the_static_workspace():
    from quantized_kv_cache_kivi_amd import kvq
    # 4096 streams x (1 bulk split + 4 fp16-row groups of 64) x 4 heads x 130 floats = 42.6 MB > 32 MiB
    cfg = kvq.make_config(1, 512, 8, 32, 128, "kivi", 2, 2, residual=256, capacity=512)
    cache = kvq.Cache(cfg)
    k = torch.zeros((512, 8, 300, 128), dtype=torch.float16, device="cuda")
    cache.kvq_select_sinks(0, k)
    cache.kvq_append(0, k, k)
    q = torch.zeros((512, 32, 128), dtype=torch.float16, device="cuda")
    out = torch.empty((512, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as ei:
        cache.kvq_decode_attn_nomalloc(0, q, out)
    assert ei.value.status == -3 and "workspace" in str(ei.value)
    cache.kvq_decode_attn(0, q, out)  # the caller-workspace entry point still serves it
    torch.cuda.synchronize()
