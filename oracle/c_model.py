"""ctypes front end of the plain-C99 oracle in oracle/c (test infrastructure only).

``CModel`` replays the same select / append / evict calls as ``oracle.cache.CacheModel`` and answers
the same questions (stored bytes of a stream, committed sinks, values read, byte accounting) plus
fp64 decode attention on OpenMP threads.  The C code is the oracle here; this module only marshals
arrays.  ``build_library`` compiles it (gcc, -std=c99 -O2 -ffp-contract=off -fno-fast-math -fopenmp);
it shares no source with the HIP library.
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c")
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")
FLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall"]

FMT = {"kivi": 0, "q2k": 1, "tq": 2}
SINK = {"none": 0, "first_n": 1, "topk": 2}


def build_library(verbose=False):
    """Compile oracle/c/kvq_oracle.c into oracle/c/libkvq_oracle.so (always recompiles)."""
    cc = os.environ.get("CC", "gcc")
    tmp = LIB + ".tmp"
    cmd = [cc] + FLAGS + ["-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("C oracle build failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layers", "batch", "n_kv_heads", "n_q_heads", "head_dim", "fmt",
                                               "k_bits", "v_bits", "sink_mode", "n_sink", "window", "residual",
                                               "capacity", "in_f32", "tq_dense3")] + [("seed", ctypes.c_uint64),
                                                                                       ("rope", ctypes.c_int32),
                                                                                       ("rope_base", ctypes.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build_library()
        L = ctypes.CDLL(LIB)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "ko_create": (P, [ctypes.POINTER(_Cfg)]), "ko_destroy": (None, [P]),
            "ko_tq_signs": (I32, [ctypes.c_uint64, I32, P]), "ko_tq_codebook": (I32, [I32, I32, P, P]),
            "ko_q2k_grid": (I32, [P, P]), "ko_f32_to_f16": (None, [P, P, I64]),
            "ko_select": (I32, [P, I32, P, I32]), "ko_append": (I32, [P, I32, P, P, I32]),
            "ko_evict": (I32, [P, I32]), "ko_state": (I32, [P, I32, P, P]),
            "ko_record_layout": (I32, [P, P]),
            "ko_stream_image": (I32, [P, I32, I32, I32, P, P, P, P, P]),
            "ko_sink_state": (I32, [P, I32, I32, P, P, P]),
            "ko_values": (I32, [P, I32, I32, I32, I32, P, I32, P, P]),
            "ko_decode_attention": (I32, [P, I32, P, ctypes.c_double, P, I32]),
            "ko_account": (I32, [P, I32, I32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def tq_signs(seed, d):
    out = np.zeros(d, np.float32)
    lib().ko_tq_signs(seed, d, _p(out))
    return out


def tq_codebook(d, bits):
    b = np.zeros((1 << bits) - 1, np.float32)
    c = np.zeros(1 << bits, np.float32)
    assert lib().ko_tq_codebook(d, bits, _p(b), _p(c)) == 0
    return b, c


def q2k_grid():
    th, lv = np.zeros(3, np.float32), np.zeros(4, np.float32)
    lib().ko_q2k_grid(_p(th), _p(lv))
    return th, lv


def f32_to_f16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib().ko_f32_to_f16(_p(x), _p(out), x.size)
    return out


class CModel:
    """The C oracle's cache model; ``cfg`` is an ``oracle.cache.Config``."""

    def __init__(self, cfg):
        self.cfg = cfg
        c = _Cfg(cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim, FMT[cfg.fmt], cfg.k_bits,
                 cfg.v_bits, SINK[cfg.sink_mode], cfg.n_sink, cfg.window, cfg.residual, cfg.capacity,
                 int(cfg.in_dtype == "f32"), int(cfg.tq_dense3), cfg.seed, int(cfg.rope), float(cfg.rope_base))
        self.h = lib().ko_create(ctypes.byref(c))
        if not self.h:
            raise ValueError("C oracle rejected the configuration")
        lay = np.zeros(6, np.int32)
        lib().ko_record_layout(self.h, _p(lay))
        self.record_bytes, self.cap_blocks = int(lay[0]), int(lay[5])

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:
            _lib.ko_destroy(h)
            self.h = None

    def _in(self, x):
        if self.cfg.in_dtype == "f32":
            return np.ascontiguousarray(x, dtype=np.float32)
        return np.ascontiguousarray(np.asarray(x, dtype=np.float16).view(np.uint16))

    def select(self, layer, k):
        k = self._in(k)
        assert lib().ko_select(self.h, layer, _p(k), k.shape[2]) == 0

    def append(self, layer, k, v):
        k, v = self._in(k), self._in(v)
        st = lib().ko_append(self.h, layer, _p(k), _p(v), k.shape[2])
        if st == -3:
            raise AssertionError("capacity: append would overwrite a live block or exceed capacity")
        if st == -4:
            raise AssertionError("append without select of the same chunk")
        assert st == 0

    def evict(self, layer):
        assert lib().ko_evict(self.h, layer) == 0

    def state(self, layer):
        P, lo = ctypes.c_int64(), ctypes.c_int64()
        lib().ko_state(self.h, layer, ctypes.byref(P), ctypes.byref(lo))
        return P.value, lo.value

    def image(self, layer, b, h):
        c = self.cfg
        D, R, ns = c.store_dim, c.residual, c.n_sink  # fp16 rows are stored at the padded width
        out = {"bulk": np.zeros((self.cap_blocks, self.record_bytes), np.uint8),
               "win_k": np.zeros((R, D), np.uint16), "win_v": np.zeros((R, D), np.uint16),
               "sink_k": np.zeros((ns, D), np.uint16), "sink_v": np.zeros((ns, D), np.uint16)}
        assert lib().ko_stream_image(self.h, layer, b, h, *[_p(out[k]) for k in
                                                           ("bulk", "win_k", "win_v", "sink_k", "sink_v")]) == 0
        return out

    def sink_state(self, layer):
        c = self.cfg
        pos = np.full((c.batch, max(c.n_sink, 1)), -1, np.int32)
        sc = np.zeros((c.batch, max(c.n_sink, 1)), np.float32)
        cnt = np.zeros(c.batch, np.int32)
        for b in range(c.batch):
            n = ctypes.c_int32()
            lib().ko_sink_state(self.h, layer, b, _p(pos[b]), _p(sc[b]), ctypes.byref(n))
            cnt[b] = n.value
        return pos[:, :c.n_sink], sc[:, :c.n_sink], cnt

    def values(self, layer, b, h, which, positions):
        """(fp64 exact values, fp16 bit patterns of the fp32 formula) of `positions`."""
        pos = np.ascontiguousarray(positions, dtype=np.int64)
        D = self.cfg.head_dim
        o64 = np.zeros((len(pos), D), np.float64)
        o16 = np.zeros((len(pos), D), np.uint16)
        st = lib().ko_values(self.h, layer, b, h, 0 if which == "k" else 1, _p(pos), len(pos), _p(o64), _p(o16))
        assert st == 0, f"ko_values: {st}"
        return o64, o16

    def decode_attention(self, layer, q, scale=None, threads=1):
        c = self.cfg
        qa = self._in(q)
        out = np.zeros((c.batch, c.n_q_heads, c.head_dim), np.float64)
        sc = float(np.float32(scale)) if scale else 0.0
        assert lib().ko_decode_attention(self.h, layer, _p(qa), sc, _p(out), threads) == 0
        return out

    def account(self, layer, b):
        o = np.zeros(8, np.int64)
        lib().ko_account(self.h, layer, b, _p(o))
        keys = ("n_valid", "n_compressed", "n_sink", "n_residual", "current_length", "compressed_bytes",
                "sink_fp16_bytes", "residual_fp16_bytes")
        return {k: int(v) for k, v in zip(keys, o)}
