"""GPU parity of the whole-T KIVI cache (include/kvq_whole.h) against the oracle, through the C ABI.

Bar: after every append, the stored K and V codes (signed int8), the per-channel K scale and zero
and the per-row V scale and zero are bit-exact with the oracle at every stored slot; dequantised
values equal the oracle's fp32 values rounded once to fp16; decode attention is within 1e-3
(max over (b, query head) of ||o - o_ref||_inf / ||o_ref||_inf).  Cases cover int8 and int4, head_dim
32, 64 and 128, GQA 1, 2, 4 and 8, fp16 and fp32 input, first-N sinks with an evicting window that
wraps the ring several times, a cache that never evicts, chunks that span several 256-row tiles
and several attention splits, a chunk that straddles the sink boundary, and K channel outliers
(channel scales spread 6x).
"""
import numpy as np
import pytest
import torch

from harness import TOL_ATTN, stable_seed
from oracle import kivi_whole as okw
from quantized_kv_cache_kivi_amd import synth

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, chunks, evict after each chunk)
    "int8_d32_r1_f32_sink4_w40": (dict(n_layers=2, batch=1, n_kv_heads=4, n_q_heads=4, head_dim=32, bits=8, n_sink=4,
                                       window=40, in_dtype="f32"), [10] + [1] * 70 + [20, 1, 1], True),
    "int4_d128_r4_f16_sink2_w100": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, bits=4,
                                         n_sink=2, window=100), [1, 150, 33, 1, 1, 40, 1], True),
    "int8_d64_r2_f16_nowindow": (dict(n_layers=1, batch=2, n_kv_heads=3, n_q_heads=6, head_dim=64, bits=8,
                                      capacity=640), [1, 255, 257, 3], False),
    "int8_d128_r8_f32_splits": (dict(n_layers=1, batch=1, n_kv_heads=2, n_q_heads=16, head_dim=128, bits=8,
                                     n_sink=3, capacity=1024, in_dtype="f32"), [2, 700, 1], False),
    "int4_d32_r2_f16_sink8_w20": (dict(n_layers=1, batch=3, n_kv_heads=1, n_q_heads=2, head_dim=32, bits=4, n_sink=8,
                                       window=20), [5, 10, 30] + [1] * 40, True),
    # the one-launch append up to 32 rows and 4 tiles (992 + 32 = 1024 rows), two launches past either
    # bound; one decode split below 2 x 512 stored rows at head_dim 128 (2 x 256 at 32), two at it
    "int8_d128_r4_f16_launch_bounds": (dict(n_layers=1, batch=2, n_kv_heads=2, n_q_heads=8, head_dim=128, bits=8,
                                            capacity=1216), [992, 32, 1, 31, 1], False),
    "int4_d32_r1_f32_launch_bounds": (dict(n_layers=1, batch=1, n_kv_heads=3, n_q_heads=3, head_dim=32, bits=4,
                                           capacity=1088, in_dtype="f32"), [500, 11, 1, 33, 1], False),
}


def _log(*a):
    print(*a, flush=True)


class WPair:
    def __init__(self, seed, shift=None, spread=None, **kw):
        from quantized_kv_cache_kivi_amd import kvq
        self.ocfg = okw.WholeConfig(**kw)
        self.model = okw.WholeCache(self.ocfg)
        c = self.ocfg
        self.gcfg = kvq.make_whole_config(c.n_layers, c.batch, c.n_kv_heads, c.n_q_heads, c.head_dim, c.bits,
                                          c.n_sink, c.window, kw.get("capacity", 0), c.in_dtype)
        self.gpu = kvq.WholeCache(self.gcfg)
        assert self.gpu.layout.capacity == c.capacity
        self.seed = seed
        self.tag = 0
        self.dt = torch.float32 if c.in_dtype == "f32" else torch.float16
        self.mult = 6.0 ** synth.uniform(c.n_kv_heads * c.head_dim, seed, 999).reshape(c.n_kv_heads, 1, c.head_dim)
        if spread is not None:  # per-channel K spread and offset [n_kv_heads, 1, head_dim]
            self.mult = spread
        self.shift = shift

    def rows(self, n):
        c = self.ocfg
        self.tag += 1
        k = synth.normal((c.batch, c.n_kv_heads, n, c.head_dim), self.seed, 1000 + self.tag) * self.mult
        if self.shift is not None:
            k = k + self.shift
        v = synth.normal((c.batch, c.n_kv_heads, n, c.head_dim), self.seed, 5000 + self.tag)
        return k.to(self.dt).contiguous(), v.to(self.dt).contiguous()

    def push(self, layer, n, evict):
        k, v = self.rows(n)
        self.model.append(layer, k.numpy(), v.numpy())
        self.gpu.kvqw_append(layer, k.cuda(), v.cuda())
        if evict:
            self.model.evict(layer)
            self.gpu.kvqw_evict(layer)
        assert self.gpu.kvqw_get_state(layer) == (self.model.P[layer], self.model.lo[layer])

    def regions(self, layer):
        c, lay = self.ocfg, self.gpu.layout
        S, D, cap = c.batch * c.n_kv_heads, c.head_dim, c.capacity
        r = lambda name, nb: self.gpu.region(layer, name, nb).cpu().numpy()
        return dict(kq=r("k_codes", S * cap * D).view(np.int8).reshape(c.batch, c.n_kv_heads, cap, D),
                    vq=r("v_codes", S * cap * D).view(np.int8).reshape(c.batch, c.n_kv_heads, cap, D),
                    ks=r("k_scale", S * D * 2).view(np.uint16).reshape(c.batch, c.n_kv_heads, D),
                    kz=r("k_zero", S * D * 2).view(np.uint16).reshape(c.batch, c.n_kv_heads, D),
                    vs=r("v_scale", S * cap * 2).view(np.uint16).reshape(c.batch, c.n_kv_heads, cap),
                    vz=r("v_zero", S * cap * 2).view(np.uint16).reshape(c.batch, c.n_kv_heads, cap))

    def compare_bytes(self, layer):
        torch.cuda.synchronize()
        g = self.regions(layer)
        m = self.model
        sl = [m.slot(p) for p in m.stored(layer)]
        for name in ("ks", "kz"):
            assert np.array_equal(g[name], getattr(m, name)[layer]), name
        for name in ("kq", "vq"):
            a, b = g[name][:, :, sl], getattr(m, name)[layer][:, :, sl]
            assert np.array_equal(a, b), (name, int((a != b).sum()))
        for name in ("vs", "vz"):
            assert np.array_equal(g[name][:, :, sl], getattr(m, name)[layer][:, :, sl]), name

    def compare_attention(self, layer, tag, qscale=1.0):
        c = self.ocfg
        q = (synth.normal((c.batch, c.n_q_heads, c.head_dim), self.seed, 9000 + tag) * qscale).to(self.dt).contiguous()
        out = torch.full((c.batch, c.n_q_heads, c.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        self.gpu.kvqw_decode_attn(layer, q.cuda(), out)
        torch.cuda.synchronize()
        ref = self.model.decode_attention(layer, q.numpy())
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        err = float((np.abs(got - ref).max(-1) / np.abs(ref).max(-1)).max())
        assert err <= TOL_ATTN, f"attention rel err {err:.3e}"
        return err

    def compare_dequant(self, layer):
        c, m = self.ocfg, self.model
        P, lo = m.P[layer], m.lo[layer]
        runs = [(0, min(c.n_sink, P)), (max(lo, c.n_sink), P)]
        for a, z in runs:
            if z <= a:
                continue
            for which, name in ((0, "k"), (1, "v")):
                out = torch.empty((c.batch, c.n_kv_heads, z - a, c.head_dim), dtype=torch.int16, device="cuda")
                self.gpu.kvqw_dequant(layer, which, a, z - a, out)
                got = out.cpu().numpy().view(np.uint16)
                for b in range(c.batch):
                    for h in range(c.n_kv_heads):
                        want = m.values(layer, b, h, name, range(a, z)).astype(np.float16).view(np.uint16)
                        assert np.array_equal(got[b, h], want), (name, a, z)


@pytest.mark.parametrize("name", list(CASES))
def test_whole_parity(name):
    kw, chunks, evict = CASES[name]
    pair = WPair(seed=stable_seed(name, 997), **kw)
    worst = 0.0
    for step, n in enumerate(chunks):
        for layer in range(kw["n_layers"]):
            pair.push(layer, n, evict)
            last = step == len(chunks) - 1
            if n > 1 or step % 10 == 0 or last:
                pair.compare_bytes(layer)
                worst = max(worst, pair.compare_attention(layer, step))
            if n > 1 or last:
                pair.compare_dequant(layer)
        if n > 1 or step % 10 == 0:
            _log(f"[{name}] step {step} n={n} P={pair.model.P[0]} stored={len(pair.model.stored(0))}: "
                 f"bytes exact, attention worst {worst:.2e}")
    _log(f"[{name}] worst attention rel err {worst:.3e}")


def test_whole_rejects_bad_calls():
    from quantized_kv_cache_kivi_amd import kvq
    pair = WPair(seed=3, n_layers=1, batch=1, n_kv_heads=2, n_q_heads=2, head_dim=64, bits=8, n_sink=2, window=30)
    cap = pair.ocfg.capacity
    k, v = pair.rows(cap + 1)  # more rows than the ring holds
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvqw_append(0, k.cuda(), v.cuda())
    assert e.value.status == -3
    q = torch.zeros((1, 2, 64), dtype=torch.float16, device="cuda")
    out = torch.zeros((1, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvqw_decode_attn(0, q, out)  # empty
    assert e.value.status == -2
    for _ in range(3):
        pair.push(0, 20, True)  # P = 60, lo = 30: stored [0, 2) and [30, 60)
    o = torch.empty((1, 2, 5, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvqw_dequant(0, 0, 0, 5, o)  # crosses the evicted gap
    assert e.value.status == -2
    pair.gpu.kvqw_dequant(0, 0, 30, 5, o)
    acc = pair.gpu.kvqw_account(0)
    assert acc["n_stored"] == 32 and acc["current_length"] == 60
    assert acc["code_bytes"] + acc["meta_bytes"] == okw.stored_bytes(pair.ocfg, 32)
    assert acc["packed_int4_bytes"] == okw.stored_bytes(pair.ocfg, 32, packed_int4=True)
    assert acc["bf16_bytes"] == okw.dense_bytes(pair.ocfg, 32, 2)


def test_whole_bench_bandwidth_size():
    """The bench's bandwidth workload (batch 8, 8 KV / 32 q heads, d=128, int8, T=4096 then single
    rows, no eviction), in the launch configuration bench.py times: codes and metadata of every
    stream bit-exact, decode attention within 1e-3."""
    pair = WPair(seed=21, n_layers=1, batch=8, n_kv_heads=8, n_q_heads=32, head_dim=128, bits=8,
                 capacity=4096 + 64)
    pair.push(0, 4096, False)
    pair.compare_bytes(0)
    err = pair.compare_attention(0, 1)
    for i in range(3):
        pair.push(0, 1, False)
    pair.compare_bytes(0)
    err = max(err, pair.compare_attention(0, 2))
    _log(f"[whole bench size] P={pair.model.P[0]}: bytes exact, attention rel err {err:.2e}")


@pytest.mark.parametrize("D,dt,T0,cap", [(128, "f32", 300, 640), (32, "f16", 300, 640), (64, "f16", 1200, 1280)])
def test_whole_single_row_appends_keep_or_recode(D, dt, T0, cap):
    """Single-row appends after a long prefill, as in decoding: most channels keep their scale and zero
    (their stored codes are kept, not rewritten), a few widen (their stored rows are coded again); some
    channels sit far from zero with a tiny spread (fp32 input: |zero| / scale far above 2^22, where
    coding a stored value again may move its code, so those groups are always coded again).  Stored
    bytes stay equal to the oracle's after every append.  Up to 1024 stored rows a single-row append is
    one launch (the last tile of a stream finishes it); the 1200-row case takes the two-launch path."""
    H = 2
    spread = torch.full((H, 1, D), 1.0)
    shift = torch.zeros((H, 1, D))
    spread[0, 0, 3] = 1e-4 if dt == "f32" else 0.05
    shift[0, 0, 3] = 1000.0
    spread[1, 0, 17] = 1e-3
    shift[1, 0, 17] = -300.0
    pair = WPair(seed=31, shift=shift, spread=spread, n_layers=1, batch=2, n_kv_heads=H, n_q_heads=2 * H,
                 head_dim=D, bits=8, capacity=cap, in_dtype=dt)
    pair.push(0, T0, False)
    pair.compare_bytes(0)
    for i in range(40):
        pair.push(0, 1, False)
        if i % 8 == 7:
            pair.compare_bytes(0)
    pair.compare_bytes(0)
    err = pair.compare_attention(0, 3)
    _log(f"[single-row appends D={D} {dt} T0={T0}] bytes exact after 40 appends, attention rel err {err:.2e}")


def test_whole_tiny_fp32_query():
    """An fp32 query of magnitude 1e-36 at head_dim 128: the matrix-core kernel scales the folded query
    up by a power of two before its fp16 split (capped, so the factor stays finite); every score is ~0
    and the output is the plain mean of the V rows, as the oracle's."""
    pair = WPair(seed=41, n_layers=1, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=128, bits=8, capacity=1216,
                 in_dtype="f32")
    pair.push(0, 1100, False)
    err = max(pair.compare_attention(0, 1, qscale=1e-36), pair.compare_attention(0, 2, qscale=1e-20))
    _log(f"[tiny fp32 query] attention rel err {err:.2e}")
