"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every entry point of the C ABI is exposed under the same name.  Torch is used
for device memory and streams only: ``Cache`` owns the cache buffer and the
decode workspace as torch uint8 tensors and passes raw pointers and the
current HIP stream to the library.  Nothing here computes any step of the
method; if the shared library is missing the import fails loudly.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

FMT = {"kivi": 0, "q2k": 1, "tq": 2}
SINK = {"none": 0, "first_n": 1, "topk": 2}
IN_DTYPE = {"f16": 0, "f32": 1}
STATUS = {0: "KVQ_OK", -1: "KVQ_EINVAL", -2: "KVQ_ERANGE", -3: "KVQ_ECAPACITY", -4: "KVQ_EORDER", -5: "KVQ_EDEVICE"}


class KvqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "batch", "n_kv_heads", "n_q_heads", "head_dim", "format", "k_bits", "v_bits",
        "sink_mode", "n_sink", "window", "residual", "capacity", "in_dtype")] + [
        ("seed", ctypes.c_uint64), ("rope", ctypes.c_int32), ("rope_base", ctypes.c_float),
        ("tq_dense3", ctypes.c_int32)]


class kvq_bytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_valid", "n_compressed", "n_sink", "n_residual", "current_length",
        "compressed_bytes", "sink_fp16_bytes", "residual_fp16_bytes")]


class kvq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "layer_stride", "bulk", "record_bytes", "rec_k_codes", "rec_v_codes", "rec_k_meta", "rec_v_meta",
        "staging", "win_k", "win_v", "sink_k", "sink_v", "sink_pos", "sink_score", "sink_count", "decode_sync",
        "tables", "select_work", "total")] + [("cap_blocks", ctypes.c_int32), ("capacity", ctypes.c_int32)]


class kvqw_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "batch", "n_kv_heads", "n_q_heads", "head_dim", "bits", "n_sink", "window", "capacity",
        "in_dtype")]


class kvqw_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "layer_stride", "k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "sync", "total")] + [
        ("capacity", ctypes.c_int32), ("pad_", ctypes.c_int32)]


class kvqw_bytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_stored", "current_length", "code_bytes", "meta_bytes", "packed_int4_bytes", "bf16_bytes")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m quantized_kv_cache_kivi_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(kvq_config)
    wcfgp = ctypes.POINTER(kvqw_config)
    sig = {
        "kvq_config_check": (I32, [cfgp]),
        "kvq_required_bytes": (SZ, [cfgp]),
        "kvq_get_layout": (I32, [cfgp, ctypes.POINTER(kvq_layout)]),
        "kvq_workspace_bytes": (SZ, [cfgp]),
        "kvq_create": (I32, [cfgp, P, SZ, P, ctypes.POINTER(P)]),
        "kvq_destroy": (I32, [P]),
        "kvq_select_sinks": (I32, [P, I32, P, I32, P]),
        "kvq_append": (I32, [P, I32, P, P, I32, P]),
        "kvq_evict": (I32, [P, I32]),
        "kvq_decode_attn": (I32, [P, I32, P, P, F32, P, SZ, P]),
        "kvq_decode_attn_nomalloc": (I32, [P, I32, P, P, F32, P]),
        "kvq_decode_step": (I32, [P, I32, P, P, P, P, F32, P, SZ, P]),
        "kvq_stream_read": (I32, [P, ctypes.c_uint64, P, P]),
        "kvq_dequant": (I32, [P, I32, I32, I64, I32, P, P]),
        "kvq_prefill_attn": (I32, [P, I32, P, I32, P, F32, P]),
        "kvq_account": (I32, [P, I32, ctypes.POINTER(kvq_bytes), P]),
        "kvq_get_state": (I32, [P, I32, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "kvq_format_tables": (I32, [cfgp, P, P, P, P, P, P, P]),
        "kvq_last_error": (ctypes.c_char_p, []),
        "kvqw_config_check": (I32, [wcfgp]),
        "kvqw_required_bytes": (SZ, [wcfgp]),
        "kvqw_get_layout": (I32, [wcfgp, ctypes.POINTER(kvqw_layout)]),
        "kvqw_workspace_bytes": (SZ, [wcfgp]),
        "kvqw_create": (I32, [wcfgp, P, SZ, P, ctypes.POINTER(P)]),
        "kvqw_destroy": (I32, [P]),
        "kvqw_append": (I32, [P, I32, P, P, I32, P, SZ, P]),
        "kvqw_evict": (I32, [P, I32]),
        "kvqw_decode_attn": (I32, [P, I32, P, P, F32, P, SZ, P]),
        "kvqw_dequant": (I32, [P, I32, I32, I64, I32, P, P]),
        "kvqw_account": (I32, [P, I32, ctypes.POINTER(kvqw_bytes)]),
        "kvqw_get_state": (I32, [P, I32, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


lib = _load()
_select, _append, _evict, _decode = lib.kvq_select_sinks, lib.kvq_append, lib.kvq_evict, lib.kvq_decode_attn


def last_error():
    return lib.kvq_last_error().decode()


def _check(status):
    if status != 0:
        raise KvqError(status, last_error())


def make_config(n_layers, batch, n_kv_heads, n_q_heads, head_dim, fmt="kivi", k_bits=2, v_bits=2,
                sink_mode="none", n_sink=0, window=0, residual=0, capacity=0, in_dtype="f16", seed=0, rope=False,
                rope_base=0.0, tq_dense3=False):
    return kvq_config(n_layers, batch, n_kv_heads, n_q_heads, head_dim, FMT[fmt], k_bits, v_bits, SINK[sink_mode],
                      n_sink, window, residual, capacity, IN_DTYPE[in_dtype], seed, int(rope), rope_base,
                      int(tq_dense3))


def config_check(cfg):
    return lib.kvq_config_check(ctypes.byref(cfg))


def required_bytes(cfg):
    return lib.kvq_required_bytes(ctypes.byref(cfg))


def workspace_bytes(cfg):
    return lib.kvq_workspace_bytes(ctypes.byref(cfg))


def get_layout(cfg):
    lay = kvq_layout()
    _check(lib.kvq_get_layout(ctypes.byref(cfg), ctypes.byref(lay)))
    return lay


def format_tables(cfg):
    """Host tables the library computes: dict of fp32 lists."""
    d = cfg.head_dim
    if cfg.format == FMT["tq"] and d in (96, 160):
        d = 128 if d == 96 else 256  # one sign per stored coordinate (the padded width)
    kl, vl = 1 << cfg.k_bits, 1 << cfg.v_bits
    bufs = {"signs": (ctypes.c_float * d)(), "k_bnd": (ctypes.c_float * (kl - 1))(), "k_cen": (ctypes.c_float * kl)(),
            "v_bnd": (ctypes.c_float * (vl - 1))(), "v_cen": (ctypes.c_float * vl)(),
            "q2k_thr": (ctypes.c_float * 3)(), "q2k_lvl": (ctypes.c_float * 4)()}
    _check(lib.kvq_format_tables(ctypes.byref(cfg), *[ctypes.cast(b, ctypes.c_void_p) for b in bufs.values()]))
    return {k: list(v) for k, v in bufs.items()}


def kvq_stream_read(buf, nbytes, out):
    """Plain streaming read of the first nbytes of device tensor `buf` (include/kvq_bench.h)."""
    _check(lib.kvq_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), _stream(buf.device.index)))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev=None):
    """Handle of the current HIP stream of device `dev` (default: the current device)."""
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device() if dev is None else dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class Cache:
    """A cache bound to a torch-allocated device buffer on the current device."""

    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        self.layout = get_layout(cfg)
        nbytes = required_bytes(cfg)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(workspace_bytes(cfg), 16), dtype=torch.uint8, device=device)
        self.dev = self.buf.device.index
        self._ws = (self.ws.data_ptr(), self.ws.numel())
        h = ctypes.c_void_p()
        _check(lib.kvq_create(ctypes.byref(cfg), _ptr(self.buf), nbytes, _stream(self.dev), ctypes.byref(h)))
        self.handle = h

    def __del__(self, _destroy=lib.kvq_destroy):  # bound early: module globals may be gone at exit
        h = getattr(self, "handle", None)
        if h:
            _destroy(h)
            self.handle = None

    # entry points, same names as the C ABI (launches go to the current stream of the cache's device)
    def kvq_select_sinks(self, layer, k):
        _check(_select(self.handle, layer, k.data_ptr(), k.shape[2], _stream(self.dev)))

    def kvq_append(self, layer, k, v):
        _check(_append(self.handle, layer, k.data_ptr(), v.data_ptr(), k.shape[2], _stream(self.dev)))

    def kvq_evict(self, layer):
        _check(_evict(self.handle, layer))

    def kvq_decode_attn(self, layer, q, out, scale=0.0):
        _check(_decode(self.handle, layer, q.data_ptr(), out.data_ptr(), scale, self._ws[0], self._ws[1],
                       _stream(self.dev)))

    def kvq_decode_step(self, layer, k, v, q, out, scale=0.0):
        """select_sinks + append(1 row) + evict + decode_attn for the row k, v ([B][Hkv][1][D])."""
        _check(lib.kvq_decode_step(self.handle, layer, _ptr(k), _ptr(v), q.data_ptr(), out.data_ptr(), scale,
                                   self._ws[0], self._ws[1], _stream(self.dev)))

    def kvq_decode_attn_nomalloc(self, layer, q, out, scale=0.0):
        _check(lib.kvq_decode_attn_nomalloc(self.handle, layer, q.data_ptr(), out.data_ptr(), scale,
                                            _stream(self.dev)))

    def kvq_prefill_attn(self, layer, q, out, scale=0.0):
        _check(lib.kvq_prefill_attn(self.handle, layer, _ptr(q), q.shape[2], _ptr(out), scale, _stream(self.dev)))

    def kvq_dequant(self, layer, which, pos0, count, out):
        _check(lib.kvq_dequant(self.handle, layer, which, pos0, count, _ptr(out), _stream(self.dev)))

    def kvq_account(self, layer):
        b = kvq_bytes()
        _check(lib.kvq_account(self.handle, layer, ctypes.byref(b), _stream(self.dev)))
        return {n: getattr(b, n) for n, _ in kvq_bytes._fields_}

    def kvq_get_state(self, layer):
        P, lo = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.kvq_get_state(self.handle, layer, ctypes.byref(P), ctypes.byref(lo)))
        return P.value, lo.value

    # raw views of the documented storage regions (for tests)
    def region(self, layer, name, nbytes):
        off = layer * self.layout.layer_stride + getattr(self.layout, name)
        return self.buf[off: off + nbytes]


# ---- the whole-T KIVI cache (include/kvq_whole.h) ----

def make_whole_config(n_layers, batch, n_kv_heads, n_q_heads, head_dim, bits=8, n_sink=0, window=0, capacity=0,
                      in_dtype="f16"):
    return kvqw_config(n_layers, batch, n_kv_heads, n_q_heads, head_dim, bits, n_sink, window, capacity,
                       IN_DTYPE[in_dtype])


def whole_config_check(cfg):
    return lib.kvqw_config_check(ctypes.byref(cfg))


def whole_required_bytes(cfg):
    return lib.kvqw_required_bytes(ctypes.byref(cfg))


def whole_workspace_bytes(cfg):
    return lib.kvqw_workspace_bytes(ctypes.byref(cfg))


def whole_layout(cfg):
    lay = kvqw_layout()
    _check(lib.kvqw_get_layout(ctypes.byref(cfg), ctypes.byref(lay)))
    return lay


class WholeCache:
    """A whole-T KIVI cache bound to a torch-allocated device buffer, with its workspace."""

    def __init__(self, cfg, device="cuda"):
        self.cfg = cfg
        self.layout = whole_layout(cfg)
        nbytes = whole_required_bytes(cfg)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(whole_workspace_bytes(cfg), 16), dtype=torch.uint8, device=device)
        self.dev = self.buf.device.index
        h = ctypes.c_void_p()
        _check(lib.kvqw_create(ctypes.byref(cfg), _ptr(self.buf), nbytes, _stream(self.dev), ctypes.byref(h)))
        self.handle = h

    def __del__(self, _destroy=lib.kvqw_destroy):
        h = getattr(self, "handle", None)
        if h:
            _destroy(h)
            self.handle = None

    def kvqw_append(self, layer, k, v):
        _check(lib.kvqw_append(self.handle, layer, _ptr(k), _ptr(v), k.shape[2], _ptr(self.ws), self.ws.numel(),
                               _stream(self.dev)))

    def kvqw_evict(self, layer):
        _check(lib.kvqw_evict(self.handle, layer))

    def kvqw_decode_attn(self, layer, q, out, scale=0.0):
        _check(lib.kvqw_decode_attn(self.handle, layer, _ptr(q), _ptr(out), scale, _ptr(self.ws), self.ws.numel(),
                                    _stream(self.dev)))

    def kvqw_dequant(self, layer, which, pos0, count, out):
        _check(lib.kvqw_dequant(self.handle, layer, which, pos0, count, _ptr(out), _stream(self.dev)))

    def kvqw_account(self, layer):
        b = kvqw_bytes()
        _check(lib.kvqw_account(self.handle, layer, ctypes.byref(b)))
        return {n: getattr(b, n) for n, _ in kvqw_bytes._fields_}

    def kvqw_get_state(self, layer):
        P, lo = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.kvqw_get_state(self.handle, layer, ctypes.byref(P), ctypes.byref(lo)))
        return P.value, lo.value

    def region(self, layer, name, nbytes):
        off = layer * self.layout.layer_stride + getattr(self.layout, name)
        return self.buf[off: off + nbytes]
