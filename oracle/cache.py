"""Cache state machine: append, sinks, eviction, stored bytes (test infrastructure only).

Follows the StreamingLLM + KIVI page ("Implementation": when the stored
length exceeds sink + window, drop the middle, keeping the first sinks and the
last window tokens; eviction runs after each per-layer append), the q2k page
("Summary": an fp16 overlay over the sink cells and the most recent N cells of
the quantized bulk, read exact) and the kivi_sink page ("How it works": sink
rows fp16 and never quantized, excluded from calibration; the fp16 residual
window composes with them).

Readings:

* Positions are absolute.  After ``evict`` the valid set is
  C u [lo, P) with lo = max(lo, P - W) (lo = 0 when W = 0), C the committed
  sinks.  Nothing moves: the bulk is a ring of 32-token block slots
  (slot = block mod cap/32) and eviction only advances lo.
* Read priority for a valid position p: sink pool if p is in C; else the
  fp16 window if p >= P - R; else the quantized bulk.
* "Replace sink rows by the nearest non-sink row before min/max" is read
  within the quantization group, where it equals excluding the sink rows
  (a duplicated in-group value changes neither min nor max).  The same
  exclusion applies to first-N sinks and to the q2k RMS.
* K blocks are re-quantized over the rows present on every append that
  touches them and freeze when complete (the group-size freezing of the
  StreamingLLM + KIVI page's "Caveats").  V rows and TurboQuant rows are
  final at append.
* Stored bytes of a block slot are those of the latest block mapped to the
  slot, as of its last append: rows not yet appended and sink rows hold code
  0 and (V) metadata 0.  Evicted blocks keep their bytes until overwritten.

Parity: the geometry is pinned by enumeration (|valid| = sink + window,
exact pool partition, overlay exactness) in tests/test_oracle_cache.py.
"""

from dataclasses import dataclass, replace

import numpy as np

from . import kivi, layout, q2k, sinks, turboquant
from .numerics import as_input, to_f16_bits

G = layout.G


@dataclass(frozen=True)
class Config:
    n_layers: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    fmt: str = "kivi"          # 'kivi' | 'q2k' | 'tq'
    k_bits: int = 2
    v_bits: int = 2
    sink_mode: str = "none"    # 'none' | 'first_n' | 'topk'
    n_sink: int = 0
    window: int = 0            # StreamingLLM W (0: never evict)
    residual: int = 0          # fp16 recent overlay R
    capacity: int = 0          # slots per stream (multiple of 32)
    in_dtype: str = "f16"      # 'f16' | 'f32'
    seed: int = 0
    rope: bool = False         # K and q handed over before RoPE, rotated on read (oracle/rope.py)
    rope_base: float = 10000.0
    tq_dense3: bool = False    # 3-bit TurboQuant codes as a dense 8-in-3 stream (else two per byte)

    @property
    def cap_blocks(self):
        return self.capacity // G

    @property
    def store_dim(self):
        """Width rows are stored and rotated at: TurboQuant pads a head_dim that is not a power of two
        with zeros to the next power of two (TurboQuant spec, "Hadamard Transform Detail") and keeps
        every rotated coordinate; other formats store head_dim."""
        if self.fmt == "tq":
            return 1 << (self.head_dim - 1).bit_length()
        return self.head_dim

    @property
    def gqa(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def defers_open_block(self):
        """Block formats with fp16 input and an fp16 window of at least one block (residual >= 32)
        quantize a block once, when its last row arrives, the way KIVI groups keys per channel only
        over full groups of tokens: while a block is open every row of it is in the fp16 window,
        which serves every read of it, and its record holds zero bytes from the append that opens
        it.  Otherwise (fp32 input, a shorter window, TurboQuant's per-token rows) an open block's
        record holds its rows so far, re-quantized on every append."""
        return self.fmt in ("kivi", "q2k") and self.in_dtype == "f16" and self.residual >= G

    def with_(self, **kw):
        return replace(self, **kw)


def default_capacity(window, max_len=0):
    """Slots per stream: one spare block beyond the window so that an append never hits a live block."""
    if window > 0:
        return G * (-(-(window + 1) // G) + 1)
    return G * (-(-max_len // G))


class TQTables:
    def __init__(self, cfg):
        self.signs = turboquant.signs(cfg.seed, cfg.store_dim)        # one per stored coordinate
        self.kb, self.kc = turboquant.codebook(cfg.head_dim, cfg.k_bits)  # Beta(head_dim/2, head_dim/2)
        self.vb, self.vc = turboquant.codebook(cfg.head_dim, cfg.v_bits)


def _blocks(x, P):
    """Rows [P, D] -> padded [nblk, 32, D] and presence mask [nblk, 32]."""
    nblk = -(-P // G)
    D = x.shape[1]
    xb = np.zeros((nblk * G, D), dtype=np.float32)
    xb[:P] = x[:P]
    pres = np.zeros(nblk * G, dtype=bool)
    pres[:P] = True
    return xb.reshape(nblk, G, D), pres.reshape(nblk, G)


def quantize_stream(cfg, K, V, sink_pos, P, tq=None):
    """Logical contents of one stream after P rows (all blocks 0 .. ceil(P/32)-1).

    K, V: fp32 [>= P, D] input rows (already in the input precision);
    sink_pos: committed sink positions (< P).  Returns a dict of per-block
    arrays: k_codes [nblk, 32, D], v_codes [nblk, 32, D], and the metadata.
    """
    nblk = -(-P // G)
    sink = np.zeros(nblk * G, dtype=bool)
    for p in sink_pos:
        if p < P:
            sink[p] = True
    sink = sink.reshape(nblk, G)
    kb, pres = _blocks(K, P)
    vb, _ = _blocks(V, P)
    calib = pres & ~sink
    out = {"nblk": nblk}
    if cfg.fmt == "kivi":
        kc, ks, kz = kivi.quantize_k_block(kb, calib, cfg.k_bits)
        vc, vs, vz = kivi.quantize_v_rows(vb.reshape(-1, cfg.head_dim), calib.reshape(-1), cfg.v_bits)
        out.update(k_codes=kc, k_scale=ks, k_zero=kz, v_codes=vc.reshape(nblk, G, -1),
                   v_scale=vs.reshape(nblk, G, -1), v_zero=vz.reshape(nblk, G, -1))
    elif cfg.fmt == "q2k":
        kc, kr = q2k.quantize_k_block(kb, calib)
        vc, vs = q2k.quantize_v_rows(vb.reshape(-1, cfg.head_dim), calib.reshape(-1))
        out.update(k_codes=kc, k_rms=kr, v_codes=vc.reshape(nblk, G, -1), v_scale=vs.reshape(nblk, G, -1))
    elif cfg.fmt == "tq":
        kc, kn = turboquant.quantize_rows(kb.reshape(-1, cfg.head_dim), tq.signs, tq.kb, calib.reshape(-1))
        vc, vn = turboquant.quantize_rows(vb.reshape(-1, cfg.head_dim), tq.signs, tq.vb, calib.reshape(-1))
        out.update(k_codes=kc.reshape(nblk, G, -1), k_norm=kn.reshape(nblk, G),
                   v_codes=vc.reshape(nblk, G, -1), v_norm=vn.reshape(nblk, G))
    else:
        raise ValueError(cfg.fmt)
    return out


def block_records(cfg, qs):
    """Packed block records [nblk, record_bytes] from quantize_stream output."""
    off, size, rec = layout.record_sections(cfg.fmt, cfg.store_dim, cfg.k_bits, cfg.v_bits, cfg.tq_dense3)
    nblk = qs["nblk"]
    out = np.zeros((nblk, rec), dtype=np.uint8)
    kb, vb = layout.slot_bits(cfg.k_bits, cfg.tq_dense3), layout.slot_bits(cfg.v_bits, cfg.tq_dense3)
    out[:, off["k_codes"]:off["k_codes"] + size["k_codes"]] = layout.pack_k_rows(qs["k_codes"], kb)
    out[:, off["v_codes"]:off["v_codes"] + size["v_codes"]] = layout.pack_v_tiles(qs["v_codes"], vb)
    if cfg.fmt == "kivi":
        km = np.concatenate([qs["k_scale"], qs["k_zero"]], axis=-1).astype("<u2").view(np.uint8)
        vm = np.concatenate([layout.pack_v_meta(qs["v_scale"]), layout.pack_v_meta(qs["v_zero"])], axis=-1)
        vm = vm.astype("<u2").view(np.uint8)
    elif cfg.fmt == "q2k":
        km = qs["k_rms"].astype("<u2").view(np.uint8)
        vm = layout.pack_v_meta(qs["v_scale"]).astype("<u2").view(np.uint8)
    else:
        km = qs["k_norm"].astype("<f4").view(np.uint8)
        vm = qs["v_norm"].astype("<f4").view(np.uint8)
    out[:, off["k_meta"]:off["k_meta"] + size["k_meta"]] = km.reshape(nblk, -1)
    out[:, off["v_meta"]:off["v_meta"] + size["v_meta"]] = vm.reshape(nblk, -1)
    return out


def stream_image(cfg, K, V, sink_list, P, tq=None):
    """Stored bytes of one stream after P rows.

    Returns dict: bulk uint8 [cap_blocks, record], win_k/win_v uint16 [R, D],
    sink_k/sink_v uint16 [n_sink, D], staging fp32 [P % 32, D] (the open
    block's raw rows; staging rows beyond P % 32 are not defined).
    """
    _, _, rec = layout.record_sections(cfg.fmt, cfg.store_dim, cfg.k_bits, cfg.v_bits, cfg.tq_dense3)
    cap_b = cfg.cap_blocks
    D = cfg.store_dim  # fp16 rows are stored at the padded width (zeros past head_dim)
    bulk = np.zeros((cap_b, rec), dtype=np.uint8)
    if P > 0:
        qs = quantize_stream(cfg, K, V, [p for p, _ in sink_list], P, tq)
        recs = block_records(cfg, qs)
        last = (P - 1) // G
        for slot in range(cap_b):
            if slot <= last:
                beta = slot + cap_b * ((last - slot) // cap_b)
                bulk[slot] = recs[beta]
        if cfg.defers_open_block and P % G:
            bulk[last % cap_b] = 0  # the open block's record: zero until the block completes
    R = cfg.residual
    win_k = np.zeros((R, D), dtype=np.uint16)
    win_v = np.zeros((R, D), dtype=np.uint16)
    Din = cfg.head_dim
    for rho in range(R):
        if rho <= P - 1:
            p = rho + R * ((P - 1 - rho) // R)
            win_k[rho, :Din] = to_f16_bits(K[p])
            win_v[rho, :Din] = to_f16_bits(V[p])
    sk = np.zeros((cfg.n_sink, D), dtype=np.uint16)
    sv = np.zeros((cfg.n_sink, D), dtype=np.uint16)
    for i, (p, _) in enumerate(sink_list):
        sk[i, :Din] = to_f16_bits(K[p])
        sv[i, :Din] = to_f16_bits(V[p])
    nst = P % G
    staging = np.array(K[P - nst:P], dtype=np.float32) if cfg.fmt != "tq" else np.zeros((0, D), np.float32)
    return {"bulk": bulk, "win_k": win_k, "win_v": win_v, "sink_k": sk, "sink_v": sv, "staging": staging}


class CacheModel:
    """Replays select / append / evict calls for every (layer, b, h) stream.

    Inputs are fp16 or fp32 arrays shaped [B, Hkv, n, D] exactly as handed to
    the library; they are kept (as fp32) so that every stored byte can be
    recomputed from the method's definition.
    """

    def __init__(self, cfg, reserve=0):
        self.cfg = cfg
        self.tq = TQTables(cfg) if cfg.fmt == "tq" else None
        L, B, H, D = cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.head_dim
        n0 = max(reserve, 64)
        self.K = [np.zeros((B, H, n0, D), np.float32) for _ in range(L)]
        self.V = [np.zeros((B, H, n0, D), np.float32) for _ in range(L)]
        self.P = [0] * L
        self.lo = [0] * L
        self.C = [[[] for _ in range(B)] for _ in range(L)]
        self.pending = [None] * L

    def _grow(self, layer, need):
        cur = self.K[layer].shape[2]
        if need <= cur:
            return
        new = max(need, 2 * cur)
        for arr in (self.K, self.V):
            a = arr[layer]
            b = np.zeros(a.shape[:2] + (new, a.shape[3]), np.float32)
            b[:, :, :cur] = a
            arr[layer] = b

    def select(self, layer, k_chunk):
        """TOPK mode: fold the chunk's key norms into the running top-k (before its append)."""
        cfg = self.cfg
        k = as_input(k_chunk, cfg.in_dtype)
        n = k.shape[2]
        P = self.P[layer]
        if cfg.sink_mode == "topk" and cfg.n_sink > 0:
            for b in range(cfg.batch):
                sc = sinks.token_scores(k[b])
                self.C[layer][b] = sinks.topk_commit(self.C[layer][b], range(P, P + n), sc, cfg.n_sink)
        self.pending[layer] = (P, n)

    def append(self, layer, k_chunk, v_chunk):
        cfg = self.cfg
        k = as_input(k_chunk, cfg.in_dtype)
        v = as_input(v_chunk, cfg.in_dtype)
        n = k.shape[2]
        P = self.P[layer]
        if cfg.sink_mode == "topk" and cfg.n_sink > 0:
            assert self.pending[layer] == (P, n), "append without select of the same chunk"
        self.pending[layer] = None
        if cfg.window == 0:
            assert P + n <= cfg.capacity, "capacity"
        else:
            last = (P + n - 1) // G
            assert (last - cfg.cap_blocks + 1) * G <= self.lo[layer], "capacity: append would overwrite a live block"
        self._grow(layer, P + n)
        self.K[layer][:, :, P:P + n] = k
        self.V[layer][:, :, P:P + n] = v
        self.P[layer] = P + n
        if cfg.sink_mode == "first_n" and cfg.n_sink > 0:
            for b in range(cfg.batch):
                self.C[layer][b] = sinks.first_n(P + n, cfg.n_sink)

    def evict(self, layer):
        if self.cfg.window > 0:
            self.lo[layer] = max(self.lo[layer], self.P[layer] - self.cfg.window)

    def sink_list(self, layer, b):
        """Committed sinks of (layer, b) that have been appended."""
        return [(p, s) for p, s in self.C[layer][b] if p < self.P[layer]]

    def image(self, layer, b, h):
        P = self.P[layer]
        return stream_image(self.cfg, self.K[layer][b, h], self.V[layer][b, h],
                            self.sink_list(layer, b), P, self.tq)

    def sink_state(self, layer):
        """positions int32 [B, n_sink] (-1 empty), scores fp32 [B, n_sink], count int32 [B]."""
        cfg = self.cfg
        pos = np.full((cfg.batch, cfg.n_sink), -1, np.int32)
        sc = np.zeros((cfg.batch, cfg.n_sink), np.float32)
        cnt = np.zeros(cfg.batch, np.int32)
        for b in range(cfg.batch):
            C = self.C[layer][b]
            cnt[b] = len(C)
            for i, (p, s) in enumerate(C):
                pos[b, i] = p
                sc[b, i] = s if cfg.sink_mode == "topk" else 0.0
        return pos, sc, cnt

    def valid(self, layer, b):
        """Valid positions with their read source: dict position -> 'sink' | 'window' | 'bulk'."""
        cfg = self.cfg
        P, lo = self.P[layer], self.lo[layer]
        C = {p for p, _ in self.sink_list(layer, b)}
        out = {}
        for p in sorted(C):
            out[p] = "sink"
        for p in range(lo, P):
            if p in C:
                continue
            out[p] = "window" if p >= P - cfg.residual else "bulk"
        return out
