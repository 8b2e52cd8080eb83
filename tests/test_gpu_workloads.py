"""GPU parity at the full sizes of the five benchmark workloads, through the C ABI, in the launch
configuration bench.py times (same library entry points, same shapes, same split policy).

The GPU cache holds every batch element; the oracle replays the same calls for sampled batch
elements (the first, one in the middle and the last) on exactly the rows the library received, so
each comparison is element by element on those streams.  The large workloads (q2k, TurboQuant, the
long int4 stream) replay on the plain-C oracle (oracle/c, bit-exact with the numpy oracle), which
makes their full decode schedules affordable; the others on the numpy oracle:

* stored bytes of every sampled stream (packed codes, metadata, fp16 window, sink pool), sink
  positions / scores / count: bit-exact;
* decode attention of the sampled batch elements (also with RoPE on read at the KIVI-2 and int4
  sizes): max over heads of ||o - o_ref||_inf / ||o_ref||_inf <= 1e-3;
* kvq_dequant of sampled positions: within 1 fp16 ulp.

Workload recipes (seeded, synthetic) follow bench.CONFIGS: the tiny 12-layer StreamingLLM + KIVI
int8 decode from empty, KIVI-2 with planted 25x sinks, q2k at T = 32768, TurboQuant K4/V2 at
T = 16384 and the long int4 stream with W = 65536.  Prefill rows are drawn per 4096-row chunk.
"""
import numpy as np
import pytest
import torch

import bench
from harness import TOL_ATTN, rel_attn_err
from oracle import attention as oattn
from oracle import c_model
from oracle import cache as ocache

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


class Workload:
    """GPU cache for all batch elements plus oracle models for the sampled ones."""

    def __init__(self, cfgno, capacity_extra=512, oracle="numpy", **extra):
        from quantized_kv_cache_kivi_amd import kvq, synth
        self.kvq, self.synth = kvq, synth
        C = bench.CONFIGS[cfgno]
        self.cfgno, self.kw, self.seed, self.T0 = cfgno, dict(C["kw"], **extra), bench.SEEDS[cfgno], C["prefill"]
        if self.kw.get("window", 0) == 0:
            self.kw["capacity"] = 32 * ((self.T0 + capacity_extra + 31) // 32)
        self.gpu = kvq.Cache(kvq.make_config(**self.kw))
        self.B = self.kw["batch"]
        self.bs = sorted({0, self.B // 2, self.B - 1})
        okw = dict(self.kw)
        okw["batch"] = 1
        okw["capacity"] = self.gpu.layout.capacity
        self.c_oracle = oracle == "c"
        if self.c_oracle:
            self.models = {b: c_model.CModel(ocache.Config(**okw)) for b in self.bs}
        else:
            self.models = {b: ocache.CacheModel(ocache.Config(**okw), reserve=self.T0 + 64) for b in self.bs}
        self.kmult = bench.key_multipliers(cfgno, self.kw, self.seed, "cuda")
        self.L = self.kw["n_layers"]

    def push(self, layer, k, v, evict=True):
        self.gpu.kvq_select_sinks(layer, k)
        self.gpu.kvq_append(layer, k, v)
        if evict:
            self.gpu.kvq_evict(layer)
        for b, m in self.models.items():
            kh, vh = k[b:b + 1].cpu().numpy(), v[b:b + 1].cpu().numpy()
            m.select(layer, kh)
            m.append(layer, kh, vh)
            if evict:
                m.evict(layer)

    def rows(self, n, tag, planted=None):
        return bench.make_rows(self.cfgno, self.kw, n, self.seed, tag, "cuda", self.kmult, planted)

    def prefill(self, planted=None):
        for c, s0 in enumerate(range(0, self.T0, 4096)):
            n = min(4096, self.T0 - s0)
            pl = planted if s0 == 0 else None
            k, v = self.rows(n, 100 + 7 * c, pl)
            for layer in range(self.L):
                self.push(layer, k, v)
            _log(f"  prefill rows [{s0}, {s0 + n})")

    def state(self, b, layer=0):
        m = self.models[b]
        return m.state(layer) if self.c_oracle else (m.P[layer], m.lo[layer])

    def query(self, tag):
        dt = torch.float32 if self.kw.get("in_dtype") == "f32" else torch.float16
        return self.synth.normal((self.B, self.kw["n_q_heads"], self.kw["head_dim"]), self.seed, tag,
                                 "cuda").to(dt).contiguous()

    def check_attention(self, layer, q):
        out = torch.empty((self.B, self.kw["n_q_heads"], self.kw["head_dim"]), dtype=torch.float32, device="cuda")
        self.gpu.kvq_decode_attn(layer, q, out)
        torch.cuda.synchronize()
        got, qh = out.cpu().numpy(), q.cpu().numpy()
        worst = 0.0
        for b, m in self.models.items():
            if self.c_oracle:
                ref = m.decode_attention(layer, qh[b:b + 1], threads=bench.host_threads())
            else:
                ref = oattn.decode_attention(m, layer, qh[b:b + 1])
            worst = max(worst, rel_attn_err(got[b:b + 1], ref))
        assert worst <= TOL_ATTN, f"attention rel err {worst:.3e}"
        return worst

    def check_bytes(self, layer):
        kw, lay = self.kw, self.gpu.layout
        H, D, R, ns = kw["n_kv_heads"], kw["head_dim"], kw.get("residual", 0), kw.get("n_sink", 0)
        torch.cuda.synchronize()
        for b, m in self.models.items():
            for h in range(H):
                s = b * H + h
                img = m.image(layer, 0, h)
                rec = lay.record_bytes
                got = self.gpu.region(layer, "bulk", (s + 1) * lay.cap_blocks * rec)[s * lay.cap_blocks * rec:]
                got = got.cpu().numpy().reshape(lay.cap_blocks, rec)
                bad = np.flatnonzero((got != img["bulk"]).any(axis=1))
                assert bad.size == 0, f"b {b} h {h}: bulk slots differ: {bad[:8]}"
                for name, n in (("win_k", R), ("win_v", R), ("sink_k", ns), ("sink_v", ns)):
                    if n == 0:
                        continue
                    reg = self.gpu.region(layer, name, (s + 1) * n * D * 2)[s * n * D * 2:]
                    g = reg.cpu().numpy().view(np.uint16).reshape(n, D)
                    assert np.array_equal(g, img[name]), f"b {b} h {h}: {name} differs"
            if ns:
                pos, sc, cnt = m.sink_state(layer)
                gp = self.gpu.region(layer, "sink_pos", self.B * ns * 4).cpu().numpy().view(np.int32)
                gs = self.gpu.region(layer, "sink_score", self.B * ns * 4).cpu().numpy().view(np.uint32)
                gc = self.gpu.region(layer, "sink_count", self.B * 4).cpu().numpy().view(np.int32)
                assert np.array_equal(gp.reshape(self.B, ns)[b], pos[0]), (gp.reshape(self.B, ns)[b], pos[0])
                assert np.array_equal(gs.reshape(self.B, ns)[b], sc[0].view(np.uint32))
                assert gc[b] == cnt[0]

    def check_dequant(self, layer, positions):
        kw = self.kw
        H, D = kw["n_kv_heads"], kw["head_dim"]
        for which in (0, 1):
            for p0, cnt in positions:
                out = torch.empty((self.B, H, cnt, D), dtype=torch.int16, device="cuda")
                self.gpu.kvq_dequant(layer, which, p0, cnt, out)
                got = out.cpu().numpy().view(np.uint16)
                for b, m in self.models.items():
                    for h in range(H):
                        wk, pos = "k" if which == 0 else "v", list(range(p0, p0 + cnt))
                        ref = m.values(layer, 0, h, wk, pos)[1] if self.c_oracle else \
                            oattn.dequant16(m, layer, 0, h, wk, pos)
                        d = np.abs(got[b, h].astype(np.int32) - ref.astype(np.int32))
                        same = (got[b, h] >> 15) == (ref >> 15)
                        d = np.where(same, d, np.where((got[b, h] & 0x7FFF) + (ref & 0x7FFF) == 0, 0, 99))
                        assert int(d.max()) <= 1, f"dequant b {b} h {h} [{p0}, {p0 + cnt}) differs by {int(d.max())} ulp"


def _check_prefill_samples(w, layer, heads, queries, tag):
    """kvq_prefill_attn of the queries of all T0 positions, as bench.py times it; sampled (batch,
    head, query) outputs against the oracle."""
    kw = w.kw
    n = min(4096, w.T0)
    q = w.synth.normal((w.B, kw["n_q_heads"], n, kw["head_dim"]), w.seed, tag, "cuda").half().contiguous()
    out = torch.empty((w.B, kw["n_q_heads"], n, kw["head_dim"]), dtype=torch.float32, device="cuda")
    w.gpu.kvq_prefill_attn(layer, q, out)
    torch.cuda.synchronize()
    got, qh = out.cpu().numpy().astype(np.float64), q.cpu().numpy()
    worst = 0.0
    for b, m in w.models.items():
        ref = oattn.prefill_attention(m, layer, qh[b:b + 1], heads=heads, queries=queries)[0]
        g = got[b][np.ix_(heads, queries)]
        err = np.abs(g - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
        worst = max(worst, float(err.max()))
    assert worst <= TOL_ATTN, f"prefill attention rel err {worst:.3e}"
    return worst


def _decode_steps(w, steps, check_at, tag0):
    worst = 0.0
    for i in range(steps):
        k, v = w.rows(1, 10_000 + 3 * i)
        for layer in range(w.L):
            w.push(layer, k, v)
        if i in check_at:
            q = w.query(50_000 + tag0 + i)
            for layer in range(w.L):
                worst = max(worst, w.check_attention(layer, q))
            _log(f"  step {i}: attention ok (worst so far {worst:.2e})")
    return worst


def test_workload_tiny_streaming_int8():
    """12 layers, decode from empty through eviction (sink 4, window 256): bytes and attention."""
    w = Workload(1)
    checks = {0, 1, 3, 31, 32, 33, 255, 256, 259, 260, 261, 300, 499}
    worst = 0.0
    for i in range(500):
        k, v = w.rows(1, 10_000 + 3 * i)
        for layer in range(w.L):
            w.push(layer, k, v)
        if i in checks:
            q = w.query(50_000 + i)
            for layer in range(w.L):
                worst = max(worst, w.check_attention(layer, q))
            w.check_bytes(i % w.L)
            P, lo = w.gpu.kvq_get_state(0)
            assert w.gpu.kvq_account(0)["n_valid"] == min(P, 4 + 256) * w.B
            _log(f"[tiny] step {i}: P={P} lo={lo} ok (worst {worst:.2e})")
    w.check_dequant(0, [(w.state(0)[1], 16), (499, 1)])


def test_workload_kivi2_dynamic_sinks():
    """Batch 8, T = 4096 with 5 planted 25x sinks per batch element, then 64 decode steps."""
    from quantized_kv_cache_kivi_amd import synth
    w = Workload(2)
    planted = synth.planted_positions(w.B, w.kw["n_sink"], w.T0, w.seed, 11)
    w.prefill(planted)
    for b in w.bs:
        got = sorted(p for p, _ in w.models[b].sink_list(0, 0))
        assert got == sorted(planted[b]), (b, got, planted[b])
    w.check_bytes(0)
    w.check_attention(0, w.query(1))
    err = _check_prefill_samples(w, 0, [0, 13, 31], [0, 1, 555, 2047, 4095], 60_000)
    _log(f"[kivi2] prefill attention of 4096 queries: sampled rel err {err:.2e}")
    _decode_steps(w, 64, {0, 1, 31, 32, 63}, 0)
    w.check_bytes(0)
    w.check_dequant(0, [(0, 64), (4096 + 60, 4)])


def test_workload_kivi2_dynamic_sinks_rope_on_read():
    """The same workload with RoPE on read: decode attention (the matrix-core decode kernel) and prefill
    attention of the 4096 prefill queries, sampled against the oracle."""
    from quantized_kv_cache_kivi_amd import synth
    w = Workload(2, rope=True)
    planted = synth.planted_positions(w.B, w.kw["n_sink"], w.T0, w.seed, 11)
    w.prefill(planted)
    w.check_attention(0, w.query(1))
    err = _check_prefill_samples(w, 0, [0, 31], [0, 2047, 4095], 61_000)
    _log(f"[kivi2 rope] prefill attention sampled rel err {err:.2e}")
    _decode_steps(w, 4, {0, 3}, 0)


def test_workload_q2k_32k():
    """q2k, batch 16, T = 32768, 4 first sinks, fp16 window 128; then 34 decode steps, so the first
    block opened by decoding completes (step 31) and freezes; bytes after the prefill and at the end."""
    w = Workload(3, oracle="c")
    w.prefill()
    w.check_bytes(0)
    w.check_attention(0, w.query(1))
    _decode_steps(w, 34, {0, 1, 30, 31, 32, 33}, 0)
    w.check_bytes(0)
    w.check_dequant(0, [(0, 40), (32768 - 200, 234)])


def test_workload_turboquant_16k():
    """TurboQuant K4/V2, batch 8, T = 16384 (AR(1) channels); then 34 decode steps (a block completes)."""
    w = Workload(4, oracle="c")
    w.prefill()
    w.check_bytes(0)
    w.check_attention(0, w.query(1))
    _decode_steps(w, 34, {0, 1, 31, 32, 33}, 0)
    w.check_bytes(0)
    w.check_dequant(0, [(0, 33), (16384 - 31, 65)])


@pytest.mark.parametrize("kb,vb,dense", [(4, 4, False), (3, 3, True)])
def test_workload_turboquant_widths_16k(kb, vb, dense):
    """Config 4's shape with other TurboQuant widths on the matrix-core decode: K4/V4 (V centroids from
    the LDS table) and K3/V3 in the dense 8-in-3 stream; bytes after the prefill and after 3 steps."""
    w = Workload(4, oracle="c", k_bits=kb, v_bits=vb, tq_dense3=dense)
    w.prefill()
    w.check_bytes(0)
    w.check_attention(0, w.query(1))
    _decode_steps(w, 3, {0, 2}, 0)
    w.check_bytes(0)


def test_workload_long_streaming_int4():
    """Batch 64, full 65540-token cache (sink 4, W = 65536), then 256 steps of append + evict + attention.
    The ring (2050 blocks, 65600 slots) wraps at step 60; attention at steps 0, 1, 2, 31, 32, 33, 127,
    128 and 255 and every stored byte of the sampled streams after the prefill and after step 255."""
    w = Workload(5, oracle="c")
    w.prefill()
    w.check_bytes(0)
    w.check_attention(0, w.query(1))
    _decode_steps(w, 256, {0, 1, 2, 31, 32, 33, 127, 128, 255}, 0)
    w.check_bytes(0)
    P, lo = w.gpu.kvq_get_state(0)
    assert (P, lo) == (65540 + 256, 65540 + 256 - 65536) and P > w.gpu.layout.capacity
    assert w.gpu.kvq_account(0)["n_valid"] == (65536 + 4) * w.B
    assert (P, lo) == w.state(0)
    w.check_dequant(0, [(lo, 64), (P - 130, 130)])


def test_workload_long_streaming_int4_rope_on_read():
    """The long int4 stream with RoPE on read, against the C oracle: indices up to 65539 (where an fp32
    product of the angle would be off by up to 3.9e-3 rad) and 2050 bulk blocks per stream, so each wave
    of the matrix-core kernel walks hundreds of blocks with its query angle stepped per block and
    recomputed every 16th.  Attention after the prefill and at decode steps 0, 1 and 60 (the ring wraps)."""
    w = Workload(5, oracle="c", rope=True)
    w.prefill()
    w.check_attention(0, w.query(1))
    _decode_steps(w, 61, {0, 1, 60}, 0)
    assert w.gpu.kvq_get_state(0) == w.state(0)
