// Host side of the C ABI: validation, storage layout, call-order state and
// launch glue.  Every compute step runs in the HIP kernels; this file only
// checks arguments, tracks (P, lo) per layer and issues launches.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvq_internal.h"

using namespace kvq;

namespace {

thread_local std::string g_err;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

}  // namespace

namespace kvq {
// The calling thread's error text, shared with the whole-T cache's entry points.
kvq_status set_error(kvq_status st, const char* msg) {
  g_err = msg;
  return st;
}
void clear_error() { g_err.clear(); }
}  // namespace kvq

namespace kvq {
// Width a row is stored and computed at: TurboQuant pads a head_dim that is not a power of two (96,
// 160) with zeros to the next power of two (128, 256), so the fast Walsh-Hadamard rotation applies
// ("TurboQuant KV Cache Compression — Spec", "Hadamard Transform Detail"), and keeps every rotated
// coordinate.
int stored_dim(const kvq_config& c) {
  if (c.format == KVQ_FMT_TQ && c.head_dim == 96) return 128;
  if (c.format == KVQ_FMT_TQ && c.head_dim == 160) return 256;
  return c.head_dim;
}
}  // namespace kvq

namespace {

struct RecordSections {
  uint64_t kc, vc, km, vm, rec;
};

// Bits a code occupies in storage: 3-bit TurboQuant codes use the page's per-byte packing, two
// codes per byte with two bits unused ([TQ] "Step 3: Packing"), i.e. 4-bit slots.
int slot_bits(int bits, int dense3 = 0) { return bits == 3 ? (dense3 ? 3 : 4) : bits; }

RecordSections record_sections(const kvq_config& c) {
  RecordSections r;
  const uint64_t D = stored_dim(c);
  r.kc = G * D * slot_bits(c.k_bits, c.tq_dense3) / 8;
  r.vc = G * D * slot_bits(c.v_bits, c.tq_dense3) / 8;
  if (c.format == KVQ_FMT_KIVI) {
    r.km = 2 * 2 * D;
    r.vm = 2 * 2 * G * (D / 32);
  } else if (c.format == KVQ_FMT_Q2K) {
    r.km = 2 * D;
    r.vm = 2 * G * (D / 32);
  } else {
    r.km = 4 * G;
    r.vm = 4 * G;
  }
  r.rec = r.kc + r.vc + r.km + r.vm;
  return r;
}

int32_t effective_capacity(const kvq_config& c) {
  if (c.capacity > 0) return c.capacity;
  if (c.window > 0) return G * ((c.window + 1 + G - 1) / G + 1);
  return 0;
}

kvq_status check(const kvq_config* c) {
  if (!c) return fail(KVQ_EINVAL, "config is NULL");
  if (c->n_layers < 1 || c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(KVQ_EINVAL, "n_layers, batch, n_kv_heads and n_q_heads must be >= 1");
  if (c->n_q_heads % c->n_kv_heads != 0 || c->n_q_heads / c->n_kv_heads > MAX_GQA)
    return fail(KVQ_EINVAL, "n_q_heads must be a multiple of n_kv_heads with ratio <= %d", MAX_GQA);
  const bool tq_pad = c->format == KVQ_FMT_TQ && (c->head_dim == 96 || c->head_dim == 160);
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 && !tq_pad)
    return fail(KVQ_EINVAL, "head_dim must be 32, 64 or 128, or 96 or 160 with TQ (got %d)", c->head_dim);
  if (tq_pad && c->sink_mode == KVQ_SINK_TOPK && c->n_sink > 0)
    return fail(KVQ_EINVAL, "top-k sink selection needs head_dim 32, 64 or 128");
  auto okb = [](int b) { return b == 2 || b == 4 || b == 8; };
  switch (c->format) {
    case KVQ_FMT_KIVI:
      if (!okb(c->k_bits) || !okb(c->v_bits)) return fail(KVQ_EINVAL, "KIVI bits must be 2, 4 or 8");
      break;
    case KVQ_FMT_Q2K:
      if (c->k_bits != 2 || c->v_bits != 4) return fail(KVQ_EINVAL, "Q2K needs k_bits = 2 and v_bits = 4");
      break;
    case KVQ_FMT_TQ:
      if (c->k_bits < 2 || c->k_bits > 4 || c->v_bits < 2 || c->v_bits > 4)
        return fail(KVQ_EINVAL, "TQ bits must be 2, 3 or 4");
      break;
    default:
      return fail(KVQ_EINVAL, "unknown format %d", c->format);
  }
  if (c->sink_mode < KVQ_SINK_NONE || c->sink_mode > KVQ_SINK_TOPK) return fail(KVQ_EINVAL, "unknown sink_mode");
  if (c->n_sink < 0 || c->n_sink > MAX_SINK) return fail(KVQ_EINVAL, "n_sink must be in [0, %d]", MAX_SINK);
  if (c->sink_mode == KVQ_SINK_NONE && c->n_sink != 0) return fail(KVQ_EINVAL, "n_sink > 0 needs a sink mode");
  if (c->window < 0 || c->residual < 0) return fail(KVQ_EINVAL, "window and residual must be >= 0");
  if (c->in_dtype != KVQ_IN_F16 && c->in_dtype != KVQ_IN_F32) return fail(KVQ_EINVAL, "in_dtype must be 0 or 1");
  if (c->rope != 0 && c->rope != 1) return fail(KVQ_EINVAL, "rope must be 0 or 1");
  if (c->rope && c->format == KVQ_FMT_TQ) return fail(KVQ_EINVAL, "rope on read is not available with TQ");
  if (c->tq_dense3 != 0 && c->tq_dense3 != 1) return fail(KVQ_EINVAL, "tq_dense3 must be 0 or 1");
  if (c->tq_dense3 && (c->format != KVQ_FMT_TQ || (c->k_bits != 3 && c->v_bits != 3)))
    return fail(KVQ_EINVAL, "tq_dense3 needs TQ with 3-bit K or V");
  if (c->capacity < 0 || c->capacity % G != 0) return fail(KVQ_EINVAL, "capacity must be a multiple of 32");
  const int32_t cap = effective_capacity(*c);
  if (cap < G) return fail(KVQ_EINVAL, "capacity must be given (>= 32) when window = 0");
  if (c->window > 0 && cap < G * ((c->window + G - 1) / G + 1))
    return fail(KVQ_EINVAL, "capacity %d too small for window %d (needs one spare block)", cap, c->window);
  if (c->residual > cap) return fail(KVQ_EINVAL, "residual larger than capacity");
  if (c->rope && (int64_t)cap + c->n_sink >= (int64_t(1) << 24))
    return fail(KVQ_EINVAL, "RoPE on read needs capacity + n_sink below 2^24 (indices exact in fp32)");
  g_err.clear();
  return KVQ_OK;
}

kvq_layout make_layout(const kvq_config& c) {
  kvq_layout L;
  std::memset(&L, 0, sizeof(L));
  const RecordSections rs = record_sections(c);
  const uint64_t S = (uint64_t)c.batch * c.n_kv_heads, D = stored_dim(c);
  const uint64_t esz = c.in_dtype == KVQ_IN_F32 ? 4 : 2;
  L.capacity = effective_capacity(c);
  L.cap_blocks = L.capacity / G;
  L.record_bytes = rs.rec;
  L.rec_k_codes = 0;
  L.rec_v_codes = rs.kc;
  L.rec_k_meta = rs.kc + rs.vc;
  L.rec_v_meta = rs.kc + rs.vc + rs.km;
  uint64_t off = 0;
  L.bulk = off;
  off = align256(off + S * L.cap_blocks * rs.rec);
  L.staging = off;
  if (c.format != KVQ_FMT_TQ) off = align256(off + S * G * D * esz);
  L.win_k = off;
  off = align256(off + S * c.residual * D * 2);
  L.win_v = off;
  off = align256(off + S * c.residual * D * 2);
  L.sink_k = off;
  off = align256(off + S * c.n_sink * D * 2);
  L.sink_v = off;
  off = align256(off + S * c.n_sink * D * 2);
  L.sink_pos = off;
  off = align256(off + (uint64_t)c.batch * c.n_sink * 4);
  L.sink_score = off;
  off = align256(off + (uint64_t)c.batch * c.n_sink * 4);
  L.sink_count = off;
  off = align256(off + (uint64_t)c.batch * 4);
  L.decode_sync = off;
  off = align256(off + S * 4);
  L.layer_stride = off;
  L.tables = (uint64_t)c.n_layers * L.layer_stride;
  L.select_work = L.tables + align256(sizeof(Tables));
  const uint64_t sel = c.sink_mode == KVQ_SINK_TOPK ? (uint64_t)c.batch * SELECT_GMAX * c.n_sink * 8 : 0;
  L.total = L.select_work + align256(sel);
  return L;
}

// Shapes the MFMA decode path covers (the generic kernel takes the rest; RoPE on read: KIVI with
// equal K and V widths).  The MFMA kernel reads a stream's ring through a buffer resource with
// 32-bit record offsets and a 31-bit size, so a ring of 2 GiB or more per stream goes to the generic
// kernel, which addresses with 64-bit pointers.
bool fast_path(const kvq_config& c) {
  const int r = c.n_q_heads / c.n_kv_heads;
  const uint64_t ring = (uint64_t)(effective_capacity(c) / G) * record_sections(c).rec;
  const bool kivi_eq = c.format == KVQ_FMT_KIVI && c.k_bits == c.v_bits;
  return ring < (uint64_t(1) << 31) && stored_dim(c) == 128 && c.in_dtype == KVQ_IN_F16 &&
         (r == 1 || r == 2 || r == 4 || r == 8) &&
         (c.rope ? kivi_eq
                 : (c.format == KVQ_FMT_Q2K || kivi_eq ||
                    (c.format == KVQ_FMT_TQ && c.k_bits >= 3 && c.v_bits >= 2)));
}

// Split-K policy over nblk bulk blocks.  MFMA path: 4 waves per workgroup, whole rounds of the
// workgroups the device holds at once (`slots`), at least 4 blocks (one per wave) per split, at most
// 64 splits.  `extra` fp16-row workgroups per stream run in the same launch, dispatched after the
// bulk: when the splits are short (<= 8 blocks per wave, about as long as an fp16 workgroup) they
// are fitted into the same round, otherwise they fill the slots the first finished splits free.
// Generic path: ~2048 workgroups of >= 2 blocks.  Never more than 64 splits.
int fast_splits(int streams, int nblk, int slots, int extra) {
  const int smax = std::max(1, std::min(64, nblk / 4));
  if (slots <= 0) slots = 1024;
  int best = 1;
  double best_eff = -1.0;
  for (int k = 1; k <= 8; ++k) {
    int s = std::max(1, std::min(smax, (int)std::lround((double)k * slots / streams)));
    const int bps = (nblk + s - 1) / s;
    s = (nblk + bps - 1) / bps;
    const long long items = (long long)streams * s, rounds = (items + slots - 1) / slots;
    const double eff = (double)items / (double)(rounds * slots);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
    if (eff >= 0.9) break;
  }
  const int bps = (nblk + best - 1) / best;
  if (extra > 0 && bps <= 32 && (long long)streams * (best + extra) > slots) {
    const int s2 = std::min(smax, slots / streams - extra);
    if (s2 >= 1) {
      const int b2 = (nblk + s2 - 1) / s2;
      best = (nblk + b2 - 1) / b2;
    }
  }
  return best;
}

int splits_for(const kvq_config& c, int nblk, int slots, int extra) {
  const int streams = c.batch * c.n_kv_heads;
  if (fast_path(c)) return fast_splits(streams, nblk, slots, extra);
  const int s = std::min((nblk + 1) / 2, std::max(1, (2048 + streams - 1) / streams));
  return std::max(1, std::min(s, 64));
}

// Block formats with fp16 input and an fp16 window of at least one block quantize a block once, when
// its last row arrives (KIVI groups keys per channel over full groups of tokens): while a block is
// open all its rows are in the fp16 window, which serves every read of them, and its record is zero.
bool defers_open_block(const kvq_config& c) {
  return c.format != KVQ_FMT_TQ && c.in_dtype == KVQ_IN_F16 && c.residual >= G;
}

// Upper bound of the splits of any decode call (sizes the workspace from the configuration alone).
int max_splits(const kvq_config& c) {
  const int nblk = effective_capacity(c) / G;
  if (fast_path(c)) return std::max(1, std::min(64, nblk / 4));
  return splits_for(c, nblk, 0, 0);
}

// RoPE caches with fp16 queries that the MFMA decode kernel does not cover decode on the prefill
// kernel (split over row blocks).
constexpr int ROPE_MAX_SPLITS = 64;
bool rope_decode_on_prefill(const kvq_config& c) {
  return c.rope && c.in_dtype == KVQ_IN_F16 && c.format != KVQ_FMT_TQ && !fast_path(c);
}

// fp16-row partials of a decode call: the MFMA path scores the window rows and the sinks in groups
// of fast_fp16_rows_per_group() rows; TurboQuant's generic kernel in one partial; other formats in
// the merge kernel.
int fp16_parts(const kvq_config& c, int64_t rows) {
  if (fast_path(c)) {
    const int per = fast_fp16_rows_per_group();
    return (int)((rows + per - 1) / per);
  }
  return c.format == KVQ_FMT_TQ || c.rope ? 1 : 0;
}

}  // namespace

struct kvq_cache {
  kvq_config cfg;
  kvq_layout lay;
  int slots;  // workgroups of the MFMA decode kernel the device holds at once (0: generic path)
  uint8_t* base;
  std::vector<int64_t> P, lo, pend_P;
  std::vector<int32_t> pend_n;
  Tables tables;
};

namespace {

Shape shape_of(const kvq_config& c) {
  Shape s;
  s.B = c.batch;
  s.Hkv = c.n_kv_heads;
  s.Hq = c.n_q_heads;
  s.D = stored_dim(c);
  s.Din = c.head_dim;
  s.fmt = c.format;
  s.kb = slot_bits(c.k_bits, c.tq_dense3);  // kernels address codes by their storage slots
  s.vb = slot_bits(c.v_bits, c.tq_dense3);
  s.sink_mode = c.n_sink > 0 ? c.sink_mode : KVQ_SINK_NONE;
  s.n_sink = c.n_sink;
  s.W = c.window;
  s.R = c.residual;
  s.in_f32 = c.in_dtype == KVQ_IN_F32;
  s.rope = c.rope;
  return s;
}

LayerView view_of(const kvq_cache* c, int layer) {
  const kvq_layout& L = c->lay;
  uint8_t* b = c->base + (uint64_t)layer * L.layer_stride;
  LayerView v;
  v.bulk = b + L.bulk;
  v.staging = b + L.staging;
  v.win_k = (uint16_t*)(b + L.win_k);
  v.win_v = (uint16_t*)(b + L.win_v);
  v.sink_k = (uint16_t*)(b + L.sink_k);
  v.sink_v = (uint16_t*)(b + L.sink_v);
  v.sink_pos = (int32_t*)(b + L.sink_pos);
  v.sink_score = (float*)(b + L.sink_score);
  v.sink_count = (int32_t*)(b + L.sink_count);
  v.decode_sync = (uint32_t*)(b + L.decode_sync);
  v.tables = (const Tables*)(c->base + L.tables);
  v.rec = (int64_t)L.record_bytes;
  v.k_codes = (int64_t)L.rec_k_codes;
  v.v_codes = (int64_t)L.rec_v_codes;
  v.k_meta = (int64_t)L.rec_k_meta;
  v.v_meta = (int64_t)L.rec_v_meta;
  v.cap_b = L.cap_blocks;
  return v;
}

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

kvq_status check_layer(const kvq_cache* c, int32_t layer) {
  if (!c) return fail(KVQ_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVQ_EINVAL, "layer %d out of range", layer);
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_config_check(const kvq_config* cfg) { return check(cfg); }

size_t kvq_required_bytes(const kvq_config* cfg) {
  if (check(cfg) != KVQ_OK) return 0;
  return (size_t)make_layout(*cfg).total;
}

kvq_status kvq_get_layout(const kvq_config* cfg, kvq_layout* out) {
  kvq_status st = check(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_EINVAL, "out is NULL");
  *out = make_layout(*cfg);
  return KVQ_OK;
}

size_t kvq_workspace_bytes(const kvq_config* cfg) {
  if (check(cfg) != KVQ_OK) return 0;
  const size_t streams = (size_t)cfg->batch * cfg->n_kv_heads;
  const size_t r = cfg->n_q_heads / cfg->n_kv_heads;
  const int parts = max_splits(*cfg) + std::max(1, fp16_parts(*cfg, (int64_t)cfg->residual + cfg->n_sink));
  size_t bytes = streams * (size_t)parts * r * (size_t)(stored_dim(*cfg) + 2) * sizeof(float);
  if (rope_decode_on_prefill(*cfg))  // row-block partials of the prefill kernel: up to 64 splits
    bytes = std::max(bytes, streams * r * (size_t)ROPE_MAX_SPLITS * (stored_dim(*cfg) + 4) * sizeof(float));
  return bytes;
}

kvq_status kvq_create(const kvq_config* cfg, void* dev_buf, size_t dev_bytes, void* stream, kvq_cache** out) {
  kvq_status st = check(cfg);
  if (st != KVQ_OK) return st;
  if (!dev_buf || !out) return fail(KVQ_EINVAL, "dev_buf and out must not be NULL");
  if (((uintptr_t)dev_buf & 255) != 0) return fail(KVQ_EINVAL, "dev_buf must be 256-byte aligned");
  const kvq_layout lay = make_layout(*cfg);
  if (dev_bytes < lay.total) return fail(KVQ_EINVAL, "dev_bytes %zu < required %llu", dev_bytes,
                                         (unsigned long long)lay.total);
  kvq_cache* c = new (std::nothrow) kvq_cache;
  if (!c) return fail(KVQ_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->cfg.capacity = lay.capacity;
  c->lay = lay;
  c->base = (uint8_t*)dev_buf;
  c->P.assign(cfg->n_layers, 0);
  c->lo.assign(cfg->n_layers, 0);
  c->pend_P.assign(cfg->n_layers, -1);
  c->pend_n.assign(cfg->n_layers, -1);
  make_tables(c->cfg, &c->tables);
  c->slots = fast_path(c->cfg) ? fast_resident_slots(shape_of(c->cfg)) : 0;
  st = static_ws_prepare();  // device address of the static decode workspace, once per device
  if (st != KVQ_OK) {
    delete c;
    return st;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemsetAsync(dev_buf, 0, lay.total, s);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipMemsetAsync");
  }
  if (cfg->n_sink > 0) {
    for (int l = 0; l < cfg->n_layers && e == hipSuccess; ++l)
      e = hipMemsetAsync(c->base + (uint64_t)l * lay.layer_stride + lay.sink_pos, 0xFF,
                         (size_t)cfg->batch * cfg->n_sink * 4, s);
    if (e != hipSuccess) {
      delete c;
      return hip_fail(e, "hipMemsetAsync");
    }
  }
  e = hipMemcpyAsync(c->base + lay.tables, &c->tables, sizeof(Tables), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host table copy must land before the handle is used
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "table upload");
  }
  *out = c;
  g_err.clear();
  return KVQ_OK;
}

kvq_status kvq_destroy(kvq_cache* c) {
  if (!c) return fail(KVQ_EINVAL, "cache is NULL");
  delete c;
  return KVQ_OK;
}

kvq_status kvq_select_sinks(kvq_cache* c, int32_t layer, const void* k, int32_t n, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!k || n < 1) return fail(KVQ_EINVAL, "k must not be NULL and n >= 1");
  c->pend_P[layer] = c->P[layer];
  c->pend_n[layer] = n;
  if (c->cfg.sink_mode != KVQ_SINK_TOPK || c->cfg.n_sink == 0) return KVQ_OK;
  if ((uintptr_t)k % 16 != 0) return fail(KVQ_EINVAL, "TOPK mode: k must be 16-byte aligned");
  // Every call commits min(n_sink - |C|, n) rows (the merged top-k holds at least that many new
  // rows, and new rows join only while the set has room), so |C| = min(n_sink, P): once n_sink rows
  // have arrived the set is full for good and the call has nothing to do.
  if (c->P[layer] >= c->cfg.n_sink) return KVQ_OK;
  SelectArgs a;
  a.sh = shape_of(c->cfg);
  a.lv = view_of(c, layer);
  a.k = k;
  a.work = (int2*)(c->base + c->lay.select_work);
  a.P = c->P[layer];
  a.n = n;
  hipError_t e = launch_select(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return KVQ_OK;
}

kvq_status kvq_append(kvq_cache* c, int32_t layer, const void* k, const void* v, int32_t n, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!k || !v || n < 1) return fail(KVQ_EINVAL, "k and v must not be NULL and n >= 1");
  const kvq_config& cf = c->cfg;
  const int64_t P = c->P[layer];
  if (P + n > (int64_t)INT32_MAX)
    return fail(KVQ_ERANGE, "append of %d rows at P=%lld: positions must stay below 2^31", n, (long long)P);
  if (cf.sink_mode == KVQ_SINK_TOPK && cf.n_sink > 0 && (c->pend_P[layer] != P || c->pend_n[layer] != n))
    return fail(KVQ_EORDER, "TOPK mode: call kvq_select_sinks on this chunk (P=%lld, n=%d) first", (long long)P, n);
  if (cf.window == 0) {
    if (P + n > cf.capacity)
      return fail(KVQ_ECAPACITY, "append of %d rows at P=%lld exceeds capacity %d", n, (long long)P, cf.capacity);
  } else {
    const int64_t last = (P + n - 1) / G;
    if ((last - c->lay.cap_blocks + 1) * G > c->lo[layer])
      return fail(KVQ_ECAPACITY, "append of %d rows at P=%lld would overwrite a live block (lo=%lld); evict first",
                  n, (long long)P, (long long)c->lo[layer]);
  }
  AppendArgs a;
  a.sh = shape_of(cf);
  a.lv = view_of(c, layer);
  a.k = k;
  a.v = v;
  a.P = P;
  a.n = n;
  a.blk0 = P / G;
  a.nblk = (int)((P + n - 1) / G - a.blk0 + 1);
  a.defer = defers_open_block(cf) ? 1 : 0;
  hipError_t e = launch_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  c->P[layer] = P + n;
  c->pend_P[layer] = -1;
  c->pend_n[layer] = -1;
  return KVQ_OK;
}

kvq_status kvq_evict(kvq_cache* c, int32_t layer) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->cfg.window > 0) c->lo[layer] = std::max(c->lo[layer], c->P[layer] - (int64_t)c->cfg.window);
  return KVQ_OK;
}

kvq_status kvq_decode_attn(kvq_cache* c, int32_t layer, const void* q, float* out, float scale, void* ws,
                           size_t ws_bytes, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (ws_bytes < kvq_workspace_bytes(&c->cfg)) return fail(KVQ_EINVAL, "ws_bytes too small");
  return kvq::decode_attn_ws(c, layer, q, out, scale, ws, ws_bytes, stream);
}

kvq_status kvq_decode_step(kvq_cache* c, int32_t layer, const void* k, const void* v, const void* q, float* out,
                           float scale, void* ws, size_t ws_bytes, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!k || !v || !q || !out || !ws) return fail(KVQ_EINVAL, "k, v, q, out and ws must not be NULL");
  if (ws_bytes < kvq_workspace_bytes(&c->cfg)) return fail(KVQ_EINVAL, "ws_bytes too small");
  const kvq_config& cf = c->cfg;
  const int64_t P = c->P[layer], lo = c->lo[layer];
  // One launch when the row changes no sink (the committed set is min(n_sink, P) rows: full, or
  // static), completes no block, and the decode kernel reads neither the open block's record (the
  // fp16 window covers it) nor the row's window slot (the row is scored from k and v).
  const bool aligned = (reinterpret_cast<uintptr_t>(k) % 16 == 0) && (reinterpret_cast<uintptr_t>(v) % 16 == 0);
  const bool fuse = c->slots > 0 && fast_path(cf) && defers_open_block(cf) && aligned && (P + 1) % G != 0 &&
                    (cf.n_sink == 0 || P >= cf.n_sink) && P + 1 <= (int64_t)INT32_MAX;
  if (!fuse) {
    if (cf.sink_mode == KVQ_SINK_TOPK && cf.n_sink > 0 && (st = kvq_select_sinks(c, layer, k, 1, stream)) != KVQ_OK)
      return st;
    if ((st = kvq_append(c, layer, k, v, 1, stream)) != KVQ_OK) return st;
    if ((st = kvq_evict(c, layer)) != KVQ_OK) return st;
    return kvq::decode_attn_ws(c, layer, q, out, scale, ws, ws_bytes, stream);
  }
  // the checks kvq_append makes
  if (cf.window == 0) {
    if (P + 1 > cf.capacity) return fail(KVQ_ECAPACITY, "append of 1 row at P=%lld exceeds capacity %d", (long long)P, cf.capacity);
  } else if ((P / G - c->lay.cap_blocks + 1) * G > lo) {
    return fail(KVQ_ECAPACITY, "append of 1 row at P=%lld would overwrite a live block (lo=%lld); evict first",
                (long long)P, (long long)lo);
  }
  c->P[layer] = P + 1;
  if (cf.window > 0) c->lo[layer] = std::max(lo, P + 1 - (int64_t)cf.window);
  st = kvq::decode_attn_ws(c, layer, q, out, scale, ws, ws_bytes, stream, k, v, P % G == 0 ? 1 : 0);
  if (st != KVQ_OK) {  // nothing launched: the call leaves the state as it found it
    c->P[layer] = P;
    c->lo[layer] = lo;
    return st;
  }
  c->pend_P[layer] = -1;
  c->pend_n[layer] = -1;
  return KVQ_OK;
}

}  // extern "C"

namespace kvq {

// Decode attention with the split partials in ws (ws_bytes long): fails with KVQ_ECAPACITY, launching
// nothing, if this call's partials do not fit.
kvq_status decode_attn_ws(kvq_cache* c, int32_t layer, const void* q, float* out, float scale, void* ws,
                          size_t ws_bytes, void* stream, const void* k1, const void* v1, int open_new) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!q || !out || !ws) return fail(KVQ_EINVAL, "q, out and ws must not be NULL");
  const kvq_config& cf = c->cfg;
  const size_t streams = (size_t)cf.batch * cf.n_kv_heads, r = cf.n_q_heads / cf.n_kv_heads;
  const int64_t P = c->P[layer], lo = c->lo[layer];
  if (P == 0) return fail(KVQ_ERANGE, "layer %d is empty", layer);
  DecodeArgs a;
  a.sh = shape_of(cf);
  a.lv = view_of(c, layer);
  a.q = q;
  a.out = out;
  a.ws = (float*)ws;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)cf.head_dim);
  a.P = P;
  a.lo = lo;
  a.k1 = k1;
  a.v1 = v1;
  a.open_new = open_new;
  a.bulk_lo = lo;
  a.bulk_hi = std::max(lo, P - (int64_t)cf.residual);
  // fp16 rows: window rows [bulk_hi, P) and at most min(n_sink, P) committed sinks (the kernels read
  // the committed count; groups past it write empty partials)
  const int64_t fp_rows = (P - a.bulk_hi) + std::min<int64_t>(cf.n_sink, P);
  const int fparts = fp16_parts(cf, fp_rows);
  if (rope_decode_on_prefill(cf)) {
    // RoPE on read with fp16 queries: the decode query is a one-query prefill chunk (its index is
    // that of position P - 1), run on the matrix-core prefill kernel split over row blocks
    if ((uintptr_t)q % 16 != 0 || (uintptr_t)out % 16 != 0 || (uintptr_t)ws % 16 != 0)
      return fail(KVQ_EINVAL, "RoPE decode: q, out and ws must be 16-byte aligned");
    PrefillArgs pa;
    pa.sh = a.sh;
    pa.lv = a.lv;
    pa.q = q;
    pa.out = out;
    pa.scale = a.scale;
    pa.P = P;
    pa.lo = lo;
    pa.bulk_hi = a.bulk_hi;
    pa.n = 1;
    pa.part = (float*)ws;
    const int nrb = prefill_row_blocks(pa);
    const int streams = cf.batch * cf.n_kv_heads;
    const int want = std::max(1, (2048 + streams - 1) / streams);  // ~2048 workgroups (1024: 147 us, 4096: 155 us)
    pa.splits = std::max(1, std::min({ROPE_MAX_SPLITS, want, nrb}));
    const size_t need = streams * r * (size_t)pa.splits * (stored_dim(cf) + 4) * sizeof(float);
    if (need > ws_bytes)
      return fail(KVQ_ECAPACITY, "decode attention needs %zu workspace bytes; %zu given", need, ws_bytes);
    hipError_t e = launch_prefill(pa, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode (RoPE) launch");
    return KVQ_OK;
  }
  if (a.bulk_hi > a.bulk_lo) {
    a.blk_first = a.bulk_lo / G;
    a.nblk = (int)((a.bulk_hi - 1) / G - a.blk_first + 1);
    const int s = splits_for(cf, a.nblk, c->slots, fparts);
    a.blocks_per_split = (a.nblk + s - 1) / s;
    a.splits = (a.nblk + a.blocks_per_split - 1) / a.blocks_per_split;
  } else {
    a.blk_first = 0;
    a.nblk = 0;
    a.splits = 0;
    a.blocks_per_split = 0;
  }
  a.fast = fast_path(cf);
  a.nparts = a.splits + fparts;
  const size_t need = streams * (size_t)std::max(1, a.nparts) * r * (stored_dim(cf) + 2) * sizeof(float);
  if (need > ws_bytes)
    return fail(KVQ_ECAPACITY, "decode attention needs %zu workspace bytes; %zu given", need, ws_bytes);
  hipError_t e = launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return KVQ_OK;
}

}  // namespace kvq

extern "C" {

kvq_status kvq_prefill_attn(kvq_cache* c, int32_t layer, const void* q, int32_t n, float* out, float scale,
                            void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!q || !out) return fail(KVQ_EINVAL, "q and out must not be NULL");
  const kvq_config& cf = c->cfg;
  const int64_t P = c->P[layer], lo = c->lo[layer];
  if (n < 1 || n > P)
    return fail(KVQ_ERANGE, "prefill attention of n=%d queries needs 1 <= n <= P=%lld (the last n positions)", n,
                (long long)P);
  const int sd = stored_dim(cf);
  if (sd != 32 && sd != 64 && sd != 128 && !(sd == 256 && cf.format == KVQ_FMT_TQ))
    return fail(KVQ_EINVAL, "prefill attention needs head_dim 32, 64, 96 (TQ), 128 or 160 (TQ)");
  if ((uintptr_t)q % 16 != 0 || (uintptr_t)out % 16 != 0) return fail(KVQ_EINVAL, "q and out must be 16-byte aligned");
  PrefillArgs a;
  a.sh = shape_of(cf);
  a.lv = view_of(c, layer);
  a.q = q;
  a.out = out;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)cf.head_dim);
  a.P = P;
  a.lo = lo;
  a.bulk_hi = std::max(lo, P - (int64_t)cf.residual);
  a.n = n;
  a.splits = 1;
  a.part = nullptr;
  hipError_t e = launch_prefill(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return KVQ_OK;
}

kvq_status kvq_dequant(kvq_cache* c, int32_t layer, int32_t which, int64_t pos0, int32_t count, uint16_t* out,
                       void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!out || (which != 0 && which != 1)) return fail(KVQ_EINVAL, "out must not be NULL and which in {0, 1}");
  if (count < 1 || pos0 < c->lo[layer] || pos0 + count > c->P[layer])
    return fail(KVQ_ERANGE, "positions [%lld, %lld) not inside the valid range [%lld, %lld)", (long long)pos0,
                (long long)(pos0 + count), (long long)c->lo[layer], (long long)c->P[layer]);
  DequantArgs a;
  a.sh = shape_of(c->cfg);
  a.lv = view_of(c, layer);
  a.which = which;
  a.P = c->P[layer];
  a.lo = c->lo[layer];
  a.pos0 = pos0;
  a.count = count;
  a.out = out;
  hipError_t e = launch_dequant(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return KVQ_OK;
}

kvq_status kvq_account(kvq_cache* c, int32_t layer, kvq_bytes* out, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_EINVAL, "out is NULL");
  const kvq_config& cf = c->cfg;
  const int B = cf.batch, ns = cf.n_sink;
  std::vector<int32_t> pos((size_t)B * std::max(ns, 1), -1), cnt(B, 0);
  hipStream_t s = (hipStream_t)stream;
  LayerView v = view_of(c, layer);
  hipError_t e = hipSuccess;
  if (ns > 0) {
    e = hipMemcpyAsync(pos.data(), v.sink_pos, (size_t)B * ns * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(cnt.data(), v.sink_count, (size_t)B * 4, hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "account copy");
  const int64_t P = c->P[layer], lo = c->lo[layer], R = cf.residual;
  const int64_t H = cf.n_kv_heads, D = stored_dim(cf);  // stored rows (TurboQuant pads 96 to 128, 160 to 256)
  const RecordSections rs = record_sections(cf);
  std::memset(out, 0, sizeof(*out));
  const int64_t wlo = std::max(lo, P - R);
  for (int b = 0; b < B; ++b) {
    std::vector<int64_t> sinks;
    for (int i = 0; i < cnt[b] && i < ns; ++i)
      if (pos[(size_t)b * ns + i] >= 0 && pos[(size_t)b * ns + i] < P) sinks.push_back(pos[(size_t)b * ns + i]);
    std::sort(sinks.begin(), sinks.end());
    int64_t n_win = std::max<int64_t>(0, P - wlo), n_bulk = std::max<int64_t>(0, wlo - lo);
    std::vector<int64_t> bulk_blocks_with_sink_only;
    for (int64_t p : sinks) {
      if (p >= wlo) --n_win;
      else if (p >= lo) --n_bulk;
    }
    // blocks holding >= 1 compressed row
    int64_t nblocks = 0;
    if (wlo > lo) {
      for (int64_t blk = lo / G; blk <= (wlo - 1) / G; ++blk) {
        const int64_t a = std::max(lo, blk * G), z = std::min(wlo, (blk + 1) * G);
        int64_t rows = z - a;
        for (int64_t p : sinks)
          if (p >= a && p < z) --rows;
        if (rows > 0) ++nblocks;
      }
    }
    const int64_t n_s = (int64_t)sinks.size();
    out->n_sink += n_s;
    out->n_residual += n_win;
    out->n_compressed += n_bulk;
    out->n_valid += n_s + n_win + n_bulk;
    int64_t meta = cf.format == KVQ_FMT_TQ ? n_bulk * 8 * H
                                           : nblocks * (int64_t)rs.km * H + n_bulk * (int64_t)(rs.vm / G) * H;
    out->compressed_bytes +=
        n_bulk * H * D * (slot_bits(cf.k_bits, cf.tq_dense3) + slot_bits(cf.v_bits, cf.tq_dense3)) / 8 + meta;
    out->sink_fp16_bytes += n_s * H * D * 2 * 2;
    out->residual_fp16_bytes += n_win * H * D * 2 * 2;
  }
  out->current_length = P;
  return KVQ_OK;
}

kvq_status kvq_get_state(const kvq_cache* c, int32_t layer, int64_t* P, int64_t* lo) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (P) *P = c->P[layer];
  if (lo) *lo = c->lo[layer];
  return KVQ_OK;
}

kvq_status kvq_format_tables(const kvq_config* cfg, float* signs, float* k_bnd, float* k_cen, float* v_bnd,
                             float* v_cen, float* q2k_thr, float* q2k_lvl) {
  kvq_status st = check(cfg);
  if (st != KVQ_OK) return st;
  Tables t;
  make_tables(*cfg, &t);
  const int kl = 1 << cfg->k_bits, vl = 1 << cfg->v_bits;
  if (signs) std::memcpy(signs, t.signs, sizeof(float) * stored_dim(*cfg));
  if (cfg->format == KVQ_FMT_TQ) {
    if (k_bnd) std::memcpy(k_bnd, t.k_bnd, sizeof(float) * (kl - 1));
    if (k_cen) std::memcpy(k_cen, t.k_cen, sizeof(float) * kl);
    if (v_bnd) std::memcpy(v_bnd, t.v_bnd, sizeof(float) * (vl - 1));
    if (v_cen) std::memcpy(v_cen, t.v_cen, sizeof(float) * vl);
  }
  if (q2k_thr) std::memcpy(q2k_thr, t.q2k_thr, sizeof(float) * 3);
  if (q2k_lvl) std::memcpy(q2k_lvl, t.q2k_lvl, sizeof(float) * 4);
  return KVQ_OK;
}

const char* kvq_last_error(void) { return g_err.c_str(); }

}  // extern "C"
