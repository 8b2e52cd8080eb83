"""Benchmark of the quantized KV cache decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the hot path for one decode token of one layer:
kvq_select_sinks -> kvq_append (1 row) -> kvq_evict -> kvq_decode_attn, on
seeded synthetic inputs already resident in HBM.  The default workload is the
KIVI 2-bit cache with dynamic sinks: 1 layer, batch 8, 8 KV heads, 32 query
heads, head_dim 128, fp16 K/V with channel outliers (RMS spread up to 6x) and
5 planted 25x sink rows per batch element, a 4096-token prefill, 5 top-k key-
norm sinks, an fp16 window of 32, int2 K and V in 32-token groups.

Cold cache: the cache is replicated enough times to exceed the 256 MB
Infinity Cache, and consecutive steps use different replicas, so each
decode-attention call streams its cache from HBM.  A warm-cache figure (one
replica) is reported separately.

value = algorithmic decode-attention bytes per step / wall time per step
(whole step: select + append + evict + attention).  The roofline object is the
decode-attention kernel alone: the same algorithmic bytes / its average
duration from HIP timing events (recorded without the system-scope fence) on its
stream.  Algorithmic bytes = packed codes and
metadata of the valid quantized tokens + fp16 sink and window rows + q + out.
"""

import argparse
import json
import math
import os
import sys
import time

METRIC = "decode-attn HBM GB/s (% of peak) + context tokens/s over quantized KV cache"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak

CONFIGS = {
    1: dict(name="tiny-streaming-int8", kw=dict(n_layers=12, batch=1, n_kv_heads=8, n_q_heads=8, head_dim=32,
                                                fmt="kivi", k_bits=8, v_bits=8, sink_mode="first_n", n_sink=4,
                                                window=256, residual=0, in_dtype="f32"),
            prefill=0, desc="12 layers, batch 1, 8 heads, d=32, fp32 K/V, int8 K/V, sink 4, window 256, "
                            "decode from empty"),
    2: dict(name="kivi2-dynamic-sinks", kw=dict(n_layers=1, batch=8, n_kv_heads=8, n_q_heads=32, head_dim=128,
                                                fmt="kivi", k_bits=2, v_bits=2, sink_mode="topk", n_sink=5,
                                                residual=32),
            prefill=4096, desc="1 layer, batch 8, 8 KV / 32 q heads, d=128, fp16 K/V, int2 K/V group 32, "
                               "5 top-k key-norm sinks (planted 25x), fp16 window 32, T=4096 prefill"),
    3: dict(name="q2k", kw=dict(n_layers=1, batch=16, n_kv_heads=8, n_q_heads=32, head_dim=128, fmt="q2k",
                                k_bits=2, v_bits=4, sink_mode="first_n", n_sink=4, residual=128),
            prefill=32768, desc="1 layer, batch 16, 8 KV / 32 q heads, d=128, fp16 K/V, K 2-bit Lloyd-Max over "
                                "block RMS (channel spread log-U[5.8, 74.9]), V 4-bit, 4 sinks, fp16 window 128, "
                                "T=32768"),
    4: dict(name="turboquant-k4v2", kw=dict(n_layers=1, batch=8, n_kv_heads=8, n_q_heads=32, head_dim=128,
                                            fmt="tq", k_bits=4, v_bits=2, seed=0x5EED0004),
            prefill=16384, desc="1 layer, batch 8, 8 KV / 32 q heads, d=128, fp16 AR(1) rho=0.8 K/V, "
                                "TurboQuant K4/V2, T=16384"),
    5: dict(name="long-streaming-int4", kw=dict(n_layers=1, batch=64, n_kv_heads=8, n_q_heads=32, head_dim=128,
                                                fmt="kivi", k_bits=4, v_bits=4, sink_mode="first_n", n_sink=4,
                                                window=65536, residual=128),
            prefill=65540, desc="1 layer, batch 64, 8 KV / 32 q heads, d=128, fp16 K/V, int4 K/V, sink 4, "
                                "window 65536, fp16 window 128, full 65540-token cache"),
}
SEEDS = {1: 0x5EED0001, 2: 0x5EED0002, 3: 0x5EED0003, 4: 0x5EED0004, 5: 0x5EED0005}


class HipTimer:
    """A pair of HIP timing events recorded without the system-scope fence (hipEventDisableSystemFence):
    a default event writes back and invalidates the caches when it is recorded, which adds several
    microseconds inside every bracket around a short call.  The elapsed time is read only after a device
    synchronisation, so the fence is not needed for it."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    _hip = None

    @classmethod
    def runtime(cls):
        if cls._hip is None:
            import ctypes
            # the HIP runtime this process already uses (torch's); libkvq resolves to the same one
            paths = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
            cls._hip = ctypes.CDLL(paths[0] if paths else "libamdhip64.so")
            cls._hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
            cls._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            cls._hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            cls._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        return cls._hip

    def __init__(self):
        import ctypes
        self.ct = ctypes
        hip = self.runtime()
        self.ev = [ctypes.c_void_p(), ctypes.c_void_p()]
        for e in self.ev:
            if hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, i, stream):
        if self.runtime().hipEventRecord(self.ev[i], self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self):
        t = self.ct.c_float()
        if self.runtime().hipEventElapsedTime(self.ct.byref(t), self.ev[0], self.ev[1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def __del__(self):
        for e in getattr(self, "ev", []):
            if e:
                self.runtime().hipEventDestroy(e)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_rows(cfgno, kw, n, seed, tag, device, kmult=None, planted=None):
    import torch
    from quantized_kv_cache_kivi_amd import synth
    B, H, D = kw["batch"], kw["n_kv_heads"], kw["head_dim"]
    shape = (B, H, n, D)
    if cfgno == 4:
        k = synth.ar1(shape, 0.8, seed, tag, device)
        v = synth.ar1(shape, 0.8, seed, tag + 1, device)
    else:
        k = synth.normal(shape, seed, tag, device)
        v = synth.normal(shape, seed, tag + 1, device)
    if kmult is not None:
        k = k * kmult[None, :, None, :]
    if planted is not None:
        for b, pos in enumerate(planted):
            k[b, :, pos, :] *= 25.0
    dt = torch.float32 if kw.get("in_dtype") == "f32" else torch.float16
    return k.to(dt).contiguous(), v.to(dt).contiguous()


def key_multipliers(cfgno, kw, seed, device):
    from quantized_kv_cache_kivi_amd import synth
    H, D = kw["n_kv_heads"], kw["head_dim"]
    if cfgno in (2, 5):
        return synth.channel_multipliers(H, D, 6.0, seed, 7, device)
    if cfgno == 3:
        return synth.q2k_multipliers(H, D, seed, 7, device)
    return None


def prefill_bytes(kw, P, n):
    """Bytes one sink-selection call and one append call of n rows at position P must move.

    Selection reads the K rows.  Append reads K and V and the staged rows of an open first block,
    and writes the packed codes and V metadata of the new rows, the K metadata of every touched
    block, the fp16 window rows among the new rows and the staged rows of an open last block
    (sink rows, at most n_sink per batch element, are not counted)."""
    D, H, B = kw["head_dim"], kw["n_kv_heads"], kw["batch"]
    R = kw.get("residual", 0)
    fmt, kb, vb = kw.get("fmt", "kivi"), kw.get("k_bits", 2), kw.get("v_bits", 2)
    esz = 4 if kw.get("in_dtype") == "f32" else 2
    kmeta_blk, vmeta_tok = {"kivi": (4 * D, 4 * (D // 32)), "q2k": (2 * D, 2 * (D // 32))}.get(fmt, (0, 8))
    S = B * H
    sel = S * n * D * esz if kw.get("sink_mode") == "topk" and kw.get("n_sink", 0) > 0 else 0
    nblk = (P + n - 1) // 32 - P // 32 + 1
    staged_in = (P % 32) * D * esz if fmt != "tq" else 0
    staged_out = ((P + n) % 32) * D * esz if fmt != "tq" else 0
    app = S * (2 * n * D * esz + staged_in + n * (D * (kb + vb) // 8 + vmeta_tok) + nblk * kmeta_blk
               + min(n, R) * 2 * D * 2 + staged_out)
    return sel, app


def prefill_attention_flops(kw, P, lo, n, sinks_per_b):
    """Algorithmic FLOPs of one causal prefill-attention call: 4*D per (query head, query, attended
    row), the attended rows of query i being the valid positions (sinks, [lo, P)) up to P-n+i."""
    D, Hq = kw["head_dim"], kw["n_q_heads"]
    total = 0
    for b in range(kw["batch"]):
        early = sorted(p for p in sinks_per_b[b] if p < lo)
        for i in range(n):
            pos = P - n + i
            total += max(0, pos - lo + 1) + sum(1 for p in early if p <= pos)
    return 4 * D * Hq * total


def prefill_attention_figure(kw, cache, P, sinks_per_b, seed, dev, stream, max_flops=5e13):
    """kvq_prefill_attn of the queries of the last min(4096, P) positions on one replica right after
    its prefill: median of three calls (HIP timing events) against the fp16 matrix-core peak."""
    import torch
    from quantized_kv_cache_kivi_amd import synth
    if P == 0:
        return None
    n = min(4096, P)
    _, lo = cache.kvq_get_state(0)
    flops = prefill_attention_flops(kw, P, lo, n, sinks_per_b)
    if flops > max_flops:
        return {"skipped": f"{flops / 1e12:.0f} TFLOP per call exceeds the bench budget"}
    qdt = torch.float32 if kw.get("in_dtype") == "f32" else torch.float16
    q = synth.normal((kw["batch"], kw["n_q_heads"], n, kw["head_dim"]), seed, 60_000, dev).to(qdt).contiguous()
    out = torch.empty((kw["batch"], kw["n_q_heads"], n, kw["head_dim"]), dtype=torch.float32, device=dev)
    cache.kvq_prefill_attn(0, q, out)
    ts = []
    for _ in range(3):
        e = HipTimer()
        e.record(0, stream)
        cache.kvq_prefill_attn(0, q, out)
        e.record(1, stream)
        torch.cuda.synchronize()
        ts.append(e.ms())
    t = sorted(ts)[1]
    achieved = flops / (t * 1e-3) / 1e12
    return {"queries": n, "P": P, "us": t * 1e3, "TFLOP_per_call": flops / 1e12,
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / MFMA_F16_PEAK_TFLOPS},
            "note": "algorithmic FLOPs (4*D per query head, query and attended row); the kernel issues 2.5x "
                    "that on the matrix cores (K and V, weights as fp16 hi + lo pairs; 3x for TurboQuant, "
                    "whose rotated queries are hi + lo pairs too)"}


def whole_decode_bytes(wk, n_stored, esz):
    """Algorithmic bytes of one whole-T decode-attention call: every stored row's K and V codes and its
    V scale and zero, the K scales and zeros, q and out."""
    S, D, r = wk["batch"] * wk["n_kv_heads"], wk["head_dim"], wk["n_q_heads"] // wk["n_kv_heads"]
    return S * (n_stored * (2 * D + 4) + 4 * D + r * D * esz + r * D * 4)


def whole_append_bytes(wk, n_old, n, esz):
    """Algorithmic bytes of one whole-T append of n rows over n_old stored rows: the stored K codes read
    once (every channel's new extremes come from them: the page's O(T*D) recompute), the new K and V
    rows read, their codes and V metadata written, the K metadata read and written.  Stored codes are
    written back only in the channel groups whose scale or zero changed (a few per append in steady
    state; their bytes are data-dependent and not counted)."""
    S, D = wk["batch"] * wk["n_kv_heads"], wk["head_dim"]
    return S * (n_old * D + n * D + 2 * n * D * esz + n * (D + 4) + 8 * D)


def whole_figure(dev, stream, with_oracle=False):
    """The StreamingLLM + KIVI page's own KIVI cache (K scales over the whole stored T), two workloads:
    the page's model shape (12 layers, 8 heads, d=32, int8, sink 4 + window 256, fp32 K/V, a 4-token
    prompt then 500 decode steps of append + evict + attention per layer), and one layer at batch 8,
    8 KV / 32 q heads, d=128, int8, T=4096 for the kernels' bandwidth."""
    import torch
    from quantized_kv_cache_kivi_amd import kvq, synth
    res = {}
    med = lambda v: sorted(v)[len(v) // 2]
    # the page's model: every step is 12 x (append 1 row, evict, decode attention)
    pk = dict(n_layers=12, batch=1, n_kv_heads=8, n_q_heads=8, head_dim=32, bits=8, n_sink=4, window=256,
              in_dtype="f32")
    c = kvq.WholeCache(kvq.make_whole_config(**pk))
    seed = 0x5EED0006
    shp = lambda n: (1, 8, n, 32)
    k0, v0 = synth.normal(shp(4), seed, 1, dev).float(), synth.normal(shp(4), seed, 2, dev).float()
    steps = 500
    ks = synth.normal((steps,) + shp(1), seed, 3, dev).float()
    vs = synth.normal((steps,) + shp(1), seed, 4, dev).float()
    qs = synth.normal((steps, 1, 8, 32), seed, 5, dev).float()
    out = torch.empty((1, 8, 32), dtype=torch.float32, device=dev)
    for layer in range(12):
        c.kvqw_append(layer, k0.contiguous(), v0.contiguous())
        c.kvqw_evict(layer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for layer in range(12):
            c.kvqw_append(layer, ks[i], vs[i])
            c.kvqw_evict(layer)
            c.kvqw_decode_attn(layer, qs[i], out)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    stored = c.kvqw_account(0)["n_stored"]
    ev_a, ev_d = [HipTimer() for _ in range(24)], [HipTimer() for _ in range(24)]
    for j in range(24):
        ev_a[j].record(0, stream)
        c.kvqw_append(0, ks[j], vs[j])
        ev_a[j].record(1, stream)
        c.kvqw_evict(0)
        ev_d[j].record(0, stream)
        c.kvqw_decode_attn(0, qs[j], out)
        ev_d[j].record(1, stream)
    torch.cuda.synchronize()
    ta, td = med([e.ms() for e in ev_a[4:]]) * 1e3, med([e.ms() for e in ev_d[4:]]) * 1e3
    res["page_model"] = {
        "workload": "12 layers, batch 1, 8 heads, d=32, int8, sink 4, window 256, fp32 K/V, 4-token prompt + "
                    f"{steps} decode steps (append 1 row + evict + decode attention per layer)",
        "tokens_per_s": steps / el, "us_per_step": el / steps * 1e6, "stored_rows": stored,
        "append_us": ta, "decode_attn_us": td,
        "cache_bytes_12_layers": 12 * c.kvqw_account(0)["code_bytes"] + 12 * c.kvqw_account(0)["meta_bytes"],
        "note": "launch-bound: 2 kernel launches per layer and step (append, decode attention; evict is host-side) over 8 x 260 rows of 68 bytes"}
    if with_oracle:  # the oracle on one layer of the same model, steady state (260 stored rows), 1 thread
        from threadpoolctl import threadpool_limits

        from oracle import kivi_whole as okw
        with threadpool_limits(limits=1):
            om = okw.WholeCache(okw.WholeConfig(1, 1, 8, 8, 32, bits=8, n_sink=4, window=256, in_dtype="f32"))
            om.append(0, k0.cpu().numpy(), v0.cpu().numpy())
            om.evict(0)
            kc, vc, qc = ks.cpu().numpy(), vs.cpu().numpy(), qs.cpu().numpy()
            for i in range(260):
                om.append(0, kc[i], vc[i])
                om.evict(0)
            t0 = time.perf_counter()
            n_or = 0
            for i in range(260, steps):
                om.append(0, kc[i], vc[i])
                om.evict(0)
                om.decode_attention(0, qc[i])
                n_or += 1
                if time.perf_counter() - t0 > 10.0:
                    break
            t_or = time.perf_counter() - t0
        res["page_model"]["cpu_baseline"] = {
            "value": n_or / t_or / 12, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_or} decode steps of one layer at 260 stored rows (append + evict + attention), "
                      "scaled to the 12 layers of a step"}
    del c
    # bandwidth workload
    wk = dict(n_layers=1, batch=8, n_kv_heads=8, n_q_heads=32, head_dim=128, bits=8, n_sink=0, window=0,
              capacity=4096 + 64, in_dtype="f16")
    c = kvq.WholeCache(kvq.make_whole_config(**wk))
    T = 4096
    k = synth.normal((8, 8, T, 128), seed, 6, dev) * synth.channel_multipliers(8, 128, 6.0, seed, 7, dev)[None, :, None, :]
    v = synth.normal((8, 8, T, 128), seed, 8, dev)
    c.kvqw_append(0, k.half().contiguous(), v.half().contiguous())
    del k, v
    n_steps = 24
    sk = [synth.normal((8, 8, 1, 128), seed, 100 + i, dev).half().contiguous() for i in range(n_steps)]
    sv = [synth.normal((8, 8, 1, 128), seed, 200 + i, dev).half().contiguous() for i in range(n_steps)]
    q = synth.normal((8, 32, 128), seed, 300, dev).half().contiguous()
    out = torch.empty((8, 32, 128), dtype=torch.float32, device=dev)
    ev_a, ev_d = [HipTimer() for _ in range(n_steps)], [HipTimer() for _ in range(n_steps)]
    for j in range(n_steps):
        ev_a[j].record(0, stream)
        c.kvqw_append(0, sk[j], sv[j])
        ev_a[j].record(1, stream)
        ev_d[j].record(0, stream)
        c.kvqw_decode_attn(0, q, out)
        ev_d[j].record(1, stream)
    torch.cuda.synchronize()
    ta, td = med([e.ms() for e in ev_a[4:]]), med([e.ms() for e in ev_d[4:]])
    n_mid = T + n_steps // 2
    ba, bd = whole_append_bytes(wk, n_mid, 1, 2), whole_decode_bytes(wk, n_mid + 1, 2)
    res["bandwidth"] = {
        "workload": "1 layer, batch 8, 8 KV / 32 q heads, d=128, int8, fp16 K/V with 6x channel spread, T=4096 "
                    "(+1 row per step), no eviction",
        "decode_attn": {"us": td * 1e3, "bytes": bd, "GBps": bd / (td * 1e-3) / 1e9,
                        "roofline": {"bound": "hbm", "achieved": bd / (td * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                                     "unit": "GB/s", "frac": bd / (td * 1e-3) / 1e9 / HBM_PEAK_GBPS}},
        "append": {"us": ta * 1e3, "bytes": ba, "GBps": ba / (ta * 1e-3) / 1e9,
                   "roofline": {"bound": "hbm", "achieved": ba / (ta * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                                "unit": "GB/s", "frac": ba / (ta * 1e-3) / 1e9 / HBM_PEAK_GBPS},
                   "note": "one row appended re-derives every K channel's scale and zero from all 4096 stored "
                           "rows (one read of the stored K codes) and re-codes the stored rows of the channel "
                           "groups whose scale or zero changed (the others code to the same bytes and are kept)"},
        "note": "median of 20 calls, HIP timing events"}
    return res


def rope_figure(cfgno, kw, pre_k, pre_v, sinks_per_b, seed, dev, stream):
    """The same workload with RoPE on read (keys and queries turned by their index in the compressed
    cache): one replica, its prefill, then decode attention (generic split kernel) and prefill
    attention of the last 4096 queries, medians of HIP timing events."""
    import torch
    from quantized_kv_cache_kivi_amd import kvq, synth
    if pre_k is None or kw.get("fmt") == "tq":
        return None
    rk = dict(kw, rope=True)
    c = kvq.Cache(kvq.make_config(**rk))
    T0 = pre_k.shape[2]
    for s0 in range(0, T0, 4096):
        k = pre_k[:, :, s0:s0 + 4096].contiguous()
        v = pre_v[:, :, s0:s0 + 4096].contiguous()
        c.kvq_select_sinks(0, k)
        c.kvq_append(0, k, v)
        c.kvq_evict(0)
    dt = torch.float32 if kw.get("in_dtype") == "f32" else torch.float16
    q = synth.normal((kw["batch"], kw["n_q_heads"], kw["head_dim"]), seed, 61_000, dev).to(dt).contiguous()
    out = torch.empty((kw["batch"], kw["n_q_heads"], kw["head_dim"]), dtype=torch.float32, device=dev)
    evs = [HipTimer() for _ in range(20)]
    for e in evs:
        e.record(0, stream)
        c.kvq_decode_attn(0, q, out)
        e.record(1, stream)
    torch.cuda.synchronize()
    t = sorted(e.ms() for e in evs[4:])[8]
    P, lo = c.kvq_get_state(0)
    nb, _ = algorithmic_bytes(kw, P, lo, sinks_per_b)
    res = {"decode_attn": {"us": t * 1e3, "bytes": nb, "GBps": nb / (t * 1e-3) / 1e9,
                           "roofline": {"bound": "hbm", "achieved": nb / (t * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                                        "unit": "GB/s", "frac": nb / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS},
                           "note": "matrix-core decode kernel (one launch): keys dequantized in fp32 and turned "
                                   "by their row in the 16-token tile, the query turned per tile by the position "
                                   "difference; fp16 window and sink rows turned by index difference"}}
    pa = prefill_attention_figure(kw, c, T0, sinks_per_b, seed, dev, stream)
    if pa is not None:
        pa["note"] = "matrix-core kernel; staged keys turned in LDS, queries as fp16 hi + lo (3 score products)"
    res["prefill_attn"] = pa
    return res


def decode_figure(cfgno, dev, stream, ncalls=40, kw_extra=None, label=None):
    """Decode attention of one workload on its full-size cache, cold: the cache is replicated until the
    replicas exceed 1 GB and consecutive calls read different replicas.  Reports the call's duration (HIP
    events on its stream, median), algorithmic GB/s and the fraction of the 8 TB/s peak, and next to it a
    plain streaming read (kvq_stream_read) of the same number of bytes from the same replicas: the
    bandwidth this GPU delivers to a read of that size, and the decode call's fraction of it.  Windowed
    workloads also time the per-step append (1 row) + evict."""
    import torch
    from quantized_kv_cache_kivi_amd import kvq, synth
    C = CONFIGS[cfgno]
    kw = dict(C["kw"], **(kw_extra or {}))
    seed, T0 = SEEDS[cfgno], C["prefill"]
    if kw.get("window", 0) == 0:
        kw["capacity"] = 32 * math.ceil((T0 + 32 + 64) / 32)
    cfg = kvq.make_config(**kw)
    per_rep = kvq.required_bytes(cfg)
    nrep = max(1, min(64, math.ceil(1.0e9 / max(per_rep, 1))))
    kmult = key_multipliers(cfgno, kw, seed, dev)
    planted = synth.planted_positions(kw["batch"], kw["n_sink"], T0, seed, 11) \
        if kw.get("sink_mode") == "topk" else None
    chunk = 4096
    chunks = []
    for i, s0 in enumerate(range(0, T0, chunk)):
        n = min(chunk, T0 - s0)
        pl = None if planted is None else [[p - s0 for p in row if s0 <= p < s0 + n] for row in planted]
        chunks.append(make_rows(cfgno, kw, n, seed, 100 + 7 * i, dev, kmult, pl))
    reps = []
    for _ in range(nrep):
        c = kvq.Cache(cfg)
        for k, v in chunks:
            c.kvq_select_sinks(0, k)
            c.kvq_append(0, k, v)
            c.kvq_evict(0)
        reps.append(c)
    del chunks
    torch.cuda.synchronize()
    sinks_per_b = [[] for _ in range(kw["batch"])]
    if kw.get("n_sink", 0) > 0:
        pos = reps[0].region(0, "sink_pos", kw["batch"] * kw["n_sink"] * 4).cpu().view(torch.int32)
        sinks_per_b = [[int(p) for p in row if p >= 0] for row in pos.reshape(kw["batch"], -1).tolist()]
    dt = torch.float32 if kw.get("in_dtype") == "f32" else torch.float16
    q = synth.normal((kw["batch"], kw["n_q_heads"], kw["head_dim"]), seed, 50_000, dev).to(dt).contiguous()
    out = torch.empty((kw["batch"], kw["n_q_heads"], kw["head_dim"]), dtype=torch.float32, device=dev)
    P, lo = reps[0].kvq_get_state(0)
    nbytes, nctx = algorithmic_bytes(kw, P, lo, sinks_per_b)

    def timed(fn, n):
        for i in range(5):
            fn(i)
        evs = [HipTimer() for _ in range(n)]
        for i in range(n):
            evs[i].record(0, stream)
            fn(5 + i)
            evs[i].record(1, stream)
        torch.cuda.synchronize()
        t = sorted(e.ms() * 1e3 for e in evs)
        return t[len(t) // 2], sum(t) / len(t)

    dec_med, dec_mean = timed(lambda i: reps[i % nrep].kvq_decode_attn(0, q, out), ncalls)
    rd_bytes = (min(nbytes, per_rep) // 16) * 16
    word = torch.zeros(4, dtype=torch.int32, device=dev)
    rd_med, rd_mean = timed(lambda i: kvq.kvq_stream_read(reps[i % nrep].buf, rd_bytes, word), ncalls)
    gbps = nbytes / dec_med / 1e3
    read_gbps = rd_bytes / rd_med / 1e3
    tr = load_traffic(cfgno)
    fig = {"workload": f"{C['name']}: {C['desc']}" + (f" ({label})" if label else ""), "P": P, "lo": lo,
           "cache_replicas": nrep,
           "bytes_per_call": nbytes, "us_per_call": dec_med, "us_per_call_mean": dec_mean, "GBps": gbps,
           "frac_of_peak": gbps / HBM_PEAK_GBPS, "context_tokens_per_s": nctx / (dec_med * 1e-6),
           "stream_read": {"bytes": rd_bytes, "us": rd_med, "GBps": read_gbps, "frac_of_peak": read_gbps / HBM_PEAK_GBPS},
           "frac_of_stream_read": gbps / read_gbps,
           "traffic_bytes_per_call": tr["bytes_per_call"] if tr and not kw_extra else None}
    if kw.get("window", 0) > 0:  # per-step append of one row + evict, on the one replica it advances
        steps = [make_rows(cfgno, kw, 1, seed, 10_000 + 3 * i, dev, kmult) for i in range(ncalls + 5)]
        c = reps[0]

        def app(i):
            k, v = steps[i]
            c.kvq_select_sinks(0, k)
            c.kvq_append(0, k, v)
            c.kvq_evict(0)

        a_med, a_mean = timed(app, ncalls)
        fig["append_evict_us"] = a_med
    del reps
    torch.cuda.empty_cache()
    return fig


def algorithmic_bytes(kw, P, lo, sinks_per_b):
    """Bytes one decode-attention call must move (valid tokens only)."""
    D, H, Hq, B = kw["head_dim"], kw["n_kv_heads"], kw["n_q_heads"], kw["batch"]
    R = kw.get("residual", 0)
    fmt, kb, vb = kw.get("fmt", "kivi"), kw.get("k_bits", 2), kw.get("v_bits", 2)
    if fmt == "tq" and not kw.get("tq_dense3"):  # 3-bit TurboQuant codes sit in 4-bit slots
        kb, vb = (4 if kb == 3 else kb), (4 if vb == 3 else vb)
    if fmt == "kivi":
        kmeta_blk, vmeta_tok = 4 * D, 4 * (D // 32)
    elif fmt == "q2k":
        kmeta_blk, vmeta_tok = 2 * D, 2 * (D // 32)
    else:
        kmeta_blk, vmeta_tok = 0, 8
    wlo = max(lo, P - R)
    total = 0
    n_ctx = 0
    for b in range(B):
        C = {p for p in sinks_per_b[b] if 0 <= p < P}
        c_bulk = sorted(p for p in C if lo <= p < wlo)
        n_fp = len(C) + (P - wlo) - sum(1 for p in C if p >= wlo)
        n_bulk = (wlo - lo) - len(c_bulk)
        nblk = (wlo - 1) // 32 - lo // 32 + 1 if wlo > lo else 0
        for blk in {p // 32 for p in c_bulk}:  # a block whose bulk rows are all sinks holds no compressed row
            a, z = max(lo, 32 * blk), min(wlo, 32 * blk + 32)
            if (z - a) == sum(1 for p in c_bulk if a <= p < z):
                nblk -= 1
        total += H * (n_bulk * (D * (kb + vb) // 8 + vmeta_tok) + nblk * kmeta_blk + n_fp * 2 * D * 2)
        n_ctx += (P - lo) + sum(1 for p in C if p < lo)
    esz = 4 if kw.get("in_dtype") == "f32" else 2
    total += B * Hq * D * esz + B * Hq * D * 4
    return total, n_ctx


def host_threads():
    """Threads the C oracle runs on: this process's CPU affinity, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(cfgno, kw, prefill_k, prefill_v, steps_kv, q, sink_mode_topk, budget_s=20.0):
    """The plain-C oracle as it stands (oracle/c: fp64 decode attention over the cache it dequantizes from
    its own stored rows), timed on the host on a bounded sample of the same workload, on every host core
    this process may use (OpenMP over the streams) and on one thread."""
    import numpy as np

    from oracle import cache as ocache
    from oracle import c_model
    ocfg = ocache.Config(**{**kw, "capacity": ocache.default_capacity(kw.get("window", 0),
                                                                      prefill_k.shape[2] + 64 + len(steps_kv))})
    threads = host_threads()
    t0 = time.perf_counter()
    m = c_model.CModel(ocfg)
    k0, v0 = prefill_k.cpu().numpy(), prefill_v.cpu().numpy()
    for s0 in range(0, k0.shape[2], 4096):
        kc, vc = k0[:, :, s0:s0 + 4096], v0[:, :, s0:s0 + 4096]
        m.select(0, kc)
        m.append(0, kc, vc)
        m.evict(0)
    t_prefill = time.perf_counter() - t0
    calls, t_n, t_1, nbytes, nbytes1 = 0, 0.0, 0.0, 0, 0
    for (k, v), qq in zip(steps_kv, q):
        kk, vv = k.cpu().numpy(), v.cpu().numpy()
        m.select(0, kk)
        m.append(0, kk, vv)
        m.evict(0)
        qn = qq.cpu().numpy()
        P, lo = m.state(0)
        pos, _, cnt = m.sink_state(0)
        sinks = [[int(p) for p in row[:c] if p >= 0] for row, c in zip(pos, cnt)]
        b_ = algorithmic_bytes(kw, P, lo, sinks)[0]
        t1 = time.perf_counter()
        m.decode_attention(0, qn, threads=threads)
        t_n += time.perf_counter() - t1
        nbytes += b_
        if calls < 2:  # the same call on one thread (first two steps)
            t1 = time.perf_counter()
            m.decode_attention(0, qn, threads=1)
            t_1 += time.perf_counter() - t1
            nbytes1 += b_
        calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    res = {"value": nbytes / t_n / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "one_thread": {"value": nbytes1 / t_1 / 1e9, "unit": "GB/s", "cores": 1},
           "sample": f"the whole workload ({kw['batch']} x {kw['n_kv_heads']} streams, {kw['n_q_heads']} query "
                     f"heads): the plain-C oracle replays the {prefill_k.shape[2]}-row prefill ({t_prefill:.1f} s) "
                     f"and {calls} decode steps; value = algorithmic decode-attention bytes / oracle decode-"
                     f"attention time (fp64 over the cache it dequantizes from its stored rows; OpenMP over the "
                     f"streams on {threads} threads; one_thread: the first two calls again on one thread)"}
    extra = {}
    # rows beyond the decode hot path keep the numpy oracle: causal prefill attention and RoPE on read
    if prefill_k.shape[2] > 0:
        import torch
        from threadpoolctl import threadpool_limits

        from oracle import attention as oattn
        from quantized_kv_cache_kivi_amd import synth
        sub = dict(kw)
        sub["batch"] = 1
        with threadpool_limits(limits=1):
            mn = ocache.CacheModel(ocache.Config(**{**sub, "capacity": ocfg.capacity}), reserve=prefill_k.shape[2] + 64)
            kb, vb = k0[:1], v0[:1]
            for s0 in range(0, kb.shape[2], 4096):
                mn.select(0, kb[:, :, s0:s0 + 4096])
                mn.append(0, kb[:, :, s0:s0 + 4096], vb[:, :, s0:s0 + 4096])
                mn.evict(0)
            P, lo = mn.P[0], mn.lo[0]
            nq = 8
            heads = list(range(0, kw["n_q_heads"], kw["n_q_heads"] // kw["n_kv_heads"]))
            qdt = torch.float32 if kw.get("in_dtype") == "f32" else torch.float16
            qp = synth.normal((1, kw["n_q_heads"], nq, kw["head_dim"]), 7, 62_000).to(qdt).numpy()
            t1 = time.perf_counter()
            oattn.prefill_attention(mn, 0, qp, heads=heads)
            tp = time.perf_counter() - t1
            early = [p for p, _ in mn.sink_list(0, 0) if p < lo]
            rows = sum(max(0, P - nq + i - lo + 1) + sum(1 for p in early if p <= P - nq + i) for i in range(nq))
            flops = 4 * kw["head_dim"] * len(heads) * rows
            extra["prefill_attn"] = {"value": flops / tp / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                                     "sample": f"batch element 0, {len(heads)} query heads (one per KV head), the "
                                               f"last {nq} of {P} positions as queries; algorithmic FLOPs / oracle "
                                               f"time (numpy oracle, fp64, 1 BLAS thread)"}
            if kw.get("fmt") != "tq":  # the same cache read with RoPE on read
                mr = ocache.CacheModel(mn.cfg.with_(rope=True), reserve=P)
                for s0 in range(0, kb.shape[2], 4096):
                    mr.select(0, kb[:, :, s0:s0 + 4096])
                    mr.append(0, kb[:, :, s0:s0 + 4096], vb[:, :, s0:s0 + 4096])
                    mr.evict(0)
                qd = qp[:, :, -1]
                t1 = time.perf_counter()
                oattn.decode_attention(mr, 0, qd)
                td = time.perf_counter() - t1
                nb_r = algorithmic_bytes(sub, mr.P[0], mr.lo[0], [[p for p, _ in mr.sink_list(0, 0)]])[0]
                extra["rope_decode_attn"] = {"value": nb_r / td / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                                             "sample": f"batch element 0 after the {mr.P[0]}-row prefill, every "
                                                       f"query head, one decode call with RoPE on read (numpy "
                                                       f"oracle, fp64, 1 BLAS thread)"}
    res["rows"] = extra
    return res


DECODE_SOURCES = ["decode_fast.hip", "decode.hip", "decode_shared.h", "device_common.h", "kvq_internal.h",
                  "kvq_api.cpp"]
DECODE_KERNELS = ("k_decode_fast", "k_merge_parts", "k_decode", "k_merge_heads", "k_decode_merge")
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read and 1 GiB written per launch


def decode_fingerprint():
    """sha256 of the sources that decide what the decode-attention kernels read and write."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_kv_cache_kivi_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(cfgno):
    return os.path.join(PROFILES, f"decode_traffic_{CONFIGS[cfgno]['name']}.json")


def load_traffic(cfgno):
    """HBM bytes per decode-attention call from hardware counters, if taken on the current kernels."""
    try:
        with open(traffic_file(cfgno)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("fingerprint") == decode_fingerprint() else None


def copy_calibration():
    """A plain copy of known size (1 GiB read, 1 GiB written per launch) for the FETCH_SIZE /
    WRITE_SIZE counter calibration."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 4 copies of {COPY_BYTES} bytes")


def _pmc_per_dispatch(d, counter, match):
    """Mean per dispatch of `counter` (summed over its instances) for kernels whose name contains any
    of `match`, per kernel base name, from a rocprofv3 --pmc output directory."""
    import collections
    import csv
    import glob
    per = collections.defaultdict(float)
    names = {}
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            if r["Counter_Name"] != counter or not any(m in r["Kernel_Name"] for m in match):
                continue
            key = r["Dispatch_Id"]
            per[key] += float(r["Counter_Value"])
            names[key] = next(m for m in match if m in r["Kernel_Name"])
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    return {k: sum(v) / len(v) for k, v in out.items()}, {k: len(v) for k, v in out.items()}


def summarize_pmc(cfgno, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, cmds):
    """Decode-attention HBM bytes per call from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by what the counter reads for the 1 GiB calibration copy; writes the JSON the bench
    reads and a short markdown summary under profiles/."""
    fk, nf = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", DECODE_KERNELS)
    wk, nw = _pmc_per_dispatch(write_dir, "WRITE_SIZE", DECODE_KERNELS)
    cf, _ = _pmc_per_dispatch(copy_fetch_dir, "FETCH_SIZE", ("copy", "elementwise"))
    cw, _ = _pmc_per_dispatch(copy_write_dir, "WRITE_SIZE", ("copy", "elementwise"))
    f_read = COPY_BYTES / (max(cf.values()) * 1024.0)
    f_write = COPY_BYTES / (max(cw.values()) * 1024.0)
    per_kernel = {k: {"fetch_kib": fk.get(k, 0.0), "write_kib": wk.get(k, 0.0), "dispatches": nf.get(k, 0)}
                  for k in sorted(set(fk) | set(wk))}
    traffic = sum(v["fetch_kib"] * 1024.0 * f_read + v["write_kib"] * 1024.0 * f_write for v in per_kernel.values())
    t = {"workload": CONFIGS[cfgno]["name"], "fingerprint": decode_fingerprint(), "bytes_per_call": traffic,
         "read_factor": f_read, "write_factor": f_write, "copy_fetch_kib": max(cf.values()),
         "copy_write_kib": max(cw.values()), "per_kernel": per_kernel, "commands": cmds}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(cfgno), "w") as f:
        json.dump(t, f, indent=1)
    lines = [f"# HBM traffic of one decode-attention call: {CONFIGS[cfgno]['name']}", "",
             f"Workload: {CONFIGS[cfgno]['desc']}.", "", "Commands (MI355X, ROCm 7.2):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", "| kernel | FETCH_SIZE KiB / dispatch | WRITE_SIZE KiB / dispatch | dispatches |", "|---|---|---|---|"]
    for k, v in per_kernel.items():
        lines.append(f"| {k} | {v['fetch_kib']:.1f} | {v['write_kib']:.1f} | {v['dispatches']} |")
    lines += ["", f"Calibration copy of {COPY_BYTES} bytes: FETCH_SIZE {max(cf.values()):.1f} KiB, WRITE_SIZE "
              f"{max(cw.values()):.1f} KiB; read factor {f_read:.4f}, write factor {f_write:.4f}.", "",
              f"HBM bytes per decode-attention call: {traffic / 1e6:.2f} MB (source fingerprint "
              f"{t['fingerprint']}).", ""]
    with open(os.path.join(PROFILES, f"decode_traffic_{CONFIGS[cfgno]['name']}.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({"traffic_bytes_per_call": traffic, "per_kernel": per_kernel}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=sorted(CONFIGS))
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas (0: enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-figures", action="store_true",
                    help="skip the whole-T cache and RoPE-on-read figures (profiling runs of the other kernels)")
    ap.add_argument("--pmc-run", action="store_true",
                    help="run the warmup and timed steps without timing or output (for rocprofv3 --pmc passes)")
    ap.add_argument("--copy-calibration", action="store_true", help="run the 1 GiB calibration copy and exit")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc outputs into profiles/decode_traffic_<workload>.{json,md}")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help="commands recorded with --summarize-pmc")
    ap.add_argument("--by-config", default="2,3,4,5",
                    help="workloads whose full-size decode attention is timed beside the headline ('' for none)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.config, *args.summarize_pmc, args.pmc_commands)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every stream of the cache is "
              "independent; sharding batch or KV heads across GPUs needs no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_kv_cache_kivi_amd import kvq, synth

    dev = "cuda"
    C = CONFIGS[args.config]
    kw = dict(C["kw"])
    seed = SEEDS[args.config]
    T0 = C["prefill"]
    # timed steps: kvq_decode_step without events (value), with events (the kernel's duration), then the
    # same steps as separate calls
    total_steps = 3 * args.steps + args.warmup
    # capacity: prefill + every step's row on one replica, rounded to blocks (windowed configs use the default ring)
    if kw.get("window", 0) == 0:
        kw["capacity"] = 32 * math.ceil((T0 + total_steps + 32) / 32)
    cfg = kvq.make_config(**kw)
    per_rep = kvq.required_bytes(cfg)
    L = kw["n_layers"]
    if args.replicas:
        nrep = args.replicas
    else:
        call_bytes_guess = max(per_rep // L, 1)
        nrep = max(1, min(64, math.ceil(1.0e9 / call_bytes_guess)))
        nrep = min(nrep, max(1, int(200e9 // per_rep)))
    log(f"[bench] config {args.config} ({C['name']}): {nrep} replicas x {per_rep / 1e6:.1f} MB")

    kmult = key_multipliers(args.config, kw, seed, dev)
    planted = None
    if kw.get("sink_mode") == "topk":
        planted = synth.planted_positions(kw["batch"], kw["n_sink"], T0, seed, 11)
    reps = []
    pre_k = pre_v = None
    if T0 > 0:
        pre_k, pre_v = make_rows(args.config, kw, T0, seed, 100, dev, kmult, planted)
    pstream = torch.cuda.current_stream().cuda_stream
    pre_t = []  # (P, n, select timer, append timer) of every prefill chunk
    for r in range(nrep):
        c = kvq.Cache(cfg)
        for layer in range(L):
            if T0 > 0:
                chunk = 4096
                for s0 in range(0, T0, chunk):
                    k = pre_k[:, :, s0:s0 + chunk].contiguous()
                    v = pre_v[:, :, s0:s0 + chunk].contiguous()
                    ts, ta = HipTimer(), HipTimer()
                    ts.record(0, pstream)
                    c.kvq_select_sinks(layer, k)
                    ts.record(1, pstream)
                    ta.record(0, pstream)
                    c.kvq_append(layer, k, v)
                    ta.record(1, pstream)
                    c.kvq_evict(layer)
                    pre_t.append((s0, k.shape[2], ts, ta))
        reps.append(c)
    torch.cuda.synchronize()
    prefill = None
    if pre_t:
        full = [(prefill_bytes(kw, P_, n_), ts.ms(), ta.ms()) for P_, n_, ts, ta in pre_t if n_ == min(4096, T0)]
        sel_us = sorted(x[1] * 1e3 for x in full)
        app_us = sorted(x[2] * 1e3 for x in full)
        b_sel, b_app = full[0][0]
        med = lambda v: v[len(v) // 2]
        prefill = {"chunk_rows": min(4096, T0), "calls": len(full),
                   "select_us": med(sel_us), "select_GBps": b_sel / med(sel_us) / 1e3 if b_sel else None,
                   "append_us": med(app_us), "append_GBps": b_app / med(app_us) / 1e3,
                   "note": "median over the full-size prefill chunks of every replica, HIP timing events around "
                           "each call; bytes from bench.prefill_bytes (select: K read; append: K+V read, codes, "
                           "metadata, fp16 rows written)"}
        del pre_t
    sinks_per_b = [[] for _ in range(kw["batch"])]
    if kw.get("n_sink", 0) > 0:
        n = kw["batch"] * kw["n_sink"]
        pos = reps[0].region(0, "sink_pos", n * 4).cpu().view(torch.int32).reshape(kw["batch"], kw["n_sink"])
        sinks_per_b = [[int(p) for p in row if p >= 0] for row in pos.tolist()]
    log(f"[bench] prefill done; sinks of b=0: {sinks_per_b[0]}")
    prefill_attn = prefill_attention_figure(kw, reps[0], T0, sinks_per_b, seed, dev, pstream) \
        if not args.pmc_run else None
    extras = not (args.pmc_run or args.no_extra_figures)
    kivi_whole = whole_figure(dev, pstream, with_oracle=not args.no_cpu_baseline) if extras else None
    rope_on_read = rope_figure(args.config, kw, pre_k, pre_v, sinks_per_b, seed, dev, pstream) if extras else None

    # per-step inputs, resident on the GPU before timing
    step_kv = [make_rows(args.config, kw, 1, seed, 10_000 + 3 * i, dev, kmult) for i in range(total_steps)]
    dt = torch.float32 if kw.get("in_dtype") == "f32" else torch.float16
    qs = [synth.normal((kw["batch"], kw["n_q_heads"], kw["head_dim"]), seed, 50_000 + i, dev).to(dt).contiguous()
          for i in range(total_steps)]
    out = torch.empty((kw["batch"], kw["n_q_heads"], kw["head_dim"]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def step(i, ev=None, fused=True):
        """One decode step of every layer: kvq_decode_step (select_sinks + append of one row + evict +
        decode_attn; one launch when the row opens or extends a block), or the four calls separately.
        The events bracket the decode step (fused) or the decode-attention call (separate)."""
        c = reps[i % nrep]
        k, v = step_kv[i]
        for layer in range(L):
            if fused:
                if ev is not None:
                    ev.record(0, stream)
                c.kvq_decode_step(layer, k, v, qs[i], out)
                if ev is not None:
                    ev.record(1, stream)
                continue
            c.kvq_select_sinks(layer, k)
            c.kvq_append(layer, k, v)
            c.kvq_evict(layer)
            if ev is not None:
                ev.record(0, stream)
            c.kvq_decode_attn(layer, qs[i], out)
            if ev is not None:
                ev.record(1, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.pmc_run:
        for j in range(args.steps):
            step(args.warmup + j)
        torch.cuda.synchronize()
        log(f"[bench] pmc run: {args.warmup + args.steps} steps")
        return
    # exact (P, lo) each timed call sees: prefill, plus one row per earlier step on the same replica
    rows_on = [0] * nrep
    for i in range(args.warmup):
        rows_on[i % nrep] += 1
    W = kw.get("window", 0)

    def timed(j0, fused, events=True):
        evs = [HipTimer() for _ in range(args.steps)] if events else [None] * args.steps
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(args.steps):
            step(j0 + j, evs[j], fused)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        nb, nc = 0, 0
        for j in range(args.steps):
            r = (j0 + j) % nrep
            rows_on[r] += 1
            P = T0 + rows_on[r]
            lo = max(0, P - W) if W > 0 else 0
            b_, n_ = algorithmic_bytes(kw, P, lo, sinks_per_b)
            nb += b_ * L
            nc += n_ * L
        ev_ms = sum(e.ms() for e in evs) / args.steps if events else None
        return elapsed * 1e3 / args.steps, ev_ms, nb / args.steps, nc / args.steps

    # the whole-step rate without instrumentation: an event pair around every call adds ~4 us of GPU
    # time per step, so the call durations come from a second pass over the following steps
    ms_step, _, bytes_per_step, ctx_per_step = timed(args.warmup, True, events=False)
    _, kern_ms, ev_bytes, ev_ctx = timed(args.warmup + args.steps, True)
    calls_per_step = L
    achieved = ev_bytes / calls_per_step / (kern_ms / calls_per_step * 1e-3) / 1e9
    sep_ms, sep_kern_ms, sep_bytes, _ = timed(args.warmup + 2 * args.steps, False)
    separate = {"ms_per_step": sep_ms, "value": sep_bytes / (sep_ms * 1e-3) / 1e9,
                "decode_attn_us_per_call": sep_kern_ms * 1e3 / calls_per_step,
                "decode_attn_GBps": sep_bytes / calls_per_step / (sep_kern_ms / calls_per_step * 1e-3) / 1e9,
                "note": "the same steps as four calls per layer (select_sinks, append, evict, decode_attn), "
                        "timed after the kvq_decode_step steps; events around the decode_attn call"}

    # warm cache: one replica, decode-attention only
    warm = None
    if nrep > 1:
        wev = [HipTimer() for _ in range(50)]
        for i in range(50):
            wev[i].record(0, stream)
            reps[0].kvq_decode_attn(0, qs[0], out)
            wev[i].record(1, stream)
        torch.cuda.synchronize()
        wms = sum(e.ms() for e in wev[10:]) / 40
        P, lo = reps[0].kvq_get_state(0)
        wb, _ = algorithmic_bytes(kw, P, lo, sinks_per_b)
        warm = {"decode_attn_us": wms * 1e3, "GBps": wb / (wms * 1e-3) / 1e9,
                "note": "same cache re-read back to back (served partly from the Infinity Cache)"}

    tr = load_traffic(args.config)
    traffic = tr["bytes_per_call"] if tr else None  # HBM bytes per decode-attention call (counters)
    res = {
        "metric": METRIC,
        "value": bytes_per_step / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{C['name']}: {C['desc']}", "steps_are": "kvq_decode_step per layer: select_sinks "
                   "+ append(1 row) + evict + decode_attn (one launch when the row opens or extends a block, "
                   "separate launches when it completes one or becomes a sink)", "cache_replicas": nrep,
                   "parallelism": "1 GPU"},
        "context_tokens_per_s": ctx_per_step / (ms_step * 1e-3),
        "decode_attn": {"us_per_call": kern_ms * 1e3 / calls_per_step, "GBps": achieved,
                        "context_tokens_per_s": ev_ctx / (kern_ms * 1e-3),
                        "bytes_per_call": ev_bytes / calls_per_step,
                        "note": "HIP events around each kvq_decode_step call (the appended row's copies "
                                "included), over the steps after the value's steps"},
        "separate_calls": separate,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "warm_cache": warm,
        "prefill": prefill,
        "prefill_attn": prefill_attn,
        "kivi_whole": kivi_whole,
        "rope_on_read": rope_on_read,
    }
    by_cfg = [int(x) for x in args.by_config.split(",") if x.strip()]
    if by_cfg:
        del reps
        torch.cuda.empty_cache()
        res["decode_attn_by_config"] = {}
        for cn in by_cfg:
            log(f"[bench] decode attention of config {cn} at full size")
            res["decode_attn_by_config"][str(cn)] = decode_figure(cn, dev, stream)
        if extras and 4 in by_cfg:
            # the other TurboQuant widths and packings at config 4's shape (same inputs and cache size)
            res["turboquant_widths"] = {}
            for name, ex in (("k3v2", dict(k_bits=3, v_bits=2)), ("k3v2_dense3", dict(k_bits=3, v_bits=2, tq_dense3=True)),
                             ("k4v3", dict(k_bits=4, v_bits=3)), ("k4v4", dict(k_bits=4, v_bits=4)),
                             ("k3v3_dense3", dict(k_bits=3, v_bits=3, tq_dense3=True))):
                log(f"[bench] decode attention of TurboQuant {name} at config 4's shape")
                res["turboquant_widths"][name] = decode_figure(4, dev, stream, ncalls=20, kw_extra=ex,
                                                               label=f"TurboQuant {name}")
    if not args.no_cpu_baseline:
        try:
            n_cpu = min(args.steps, 16)
            res["cpu_baseline"] = cpu_baseline(args.config, kw, pre_k if pre_k is not None else
                                               step_kv[0][0][:, :, :0], pre_v if pre_v is not None else
                                               step_kv[0][1][:, :, :0], step_kv[:n_cpu], qs[:n_cpu],
                                               kw.get("sink_mode") == "topk")
            rows = res["cpu_baseline"].pop("rows", {})
            if res.get("prefill_attn") and "prefill_attn" in rows:
                res["prefill_attn"]["cpu_baseline"] = rows["prefill_attn"]
            if res.get("rope_on_read") and "rope_decode_attn" in rows:
                res["rope_on_read"]["decode_attn"]["cpu_baseline"] = rows["rope_decode_attn"]
        except Exception as e:  # the baseline is a report, never a reason to lose the GPU line
            res["cpu_baseline"] = {"value": None, "unit": "GB/s", "cores": 1, "kind": "oracle",
                                   "sample": f"failed: {e!r}"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
