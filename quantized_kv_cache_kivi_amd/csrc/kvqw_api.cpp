// Host side of the whole-T KIVI cache (kvq_whole.h): validation, storage layout, (P, lo) per layer
// and launch glue.  Every compute step runs in the kernels of whole.hip.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "kvq_internal.h"
#include "whole_internal.h"

using namespace kvqw;

namespace {

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return kvq::set_error(st, buf);
}

uint64_t a256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

int32_t eff_cap(const kvqw_config& c) {
  if (c.capacity > 0) return c.capacity;
  if (c.window > 0) return 32 * ((c.n_sink + c.window + 32 + 31) / 32);
  return 0;
}

kvq_status check(const kvqw_config* c) {
  if (!c) return fail(KVQ_EINVAL, "config is NULL");
  if (c->n_layers < 1 || c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(KVQ_EINVAL, "n_layers, batch and head counts must be >= 1");
  if (c->n_q_heads % c->n_kv_heads != 0) return fail(KVQ_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  const int r = c->n_q_heads / c->n_kv_heads;
  if (r != 1 && r != 2 && r != 4 && r != 8) return fail(KVQ_EINVAL, "n_q_heads / n_kv_heads must be 1, 2, 4 or 8");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(KVQ_EINVAL, "head_dim must be 32, 64 or 128 (got %d)", c->head_dim);
  if (c->bits != 8 && c->bits != 4) return fail(KVQ_EINVAL, "bits must be 8 or 4");
  if (c->n_sink < 0 || c->window < 0) return fail(KVQ_EINVAL, "n_sink and window must be >= 0");
  if (c->in_dtype != KVQ_IN_F16 && c->in_dtype != KVQ_IN_F32) return fail(KVQ_EINVAL, "in_dtype must be 0 or 1");
  if (c->capacity < 0 || c->capacity % 32 != 0) return fail(KVQ_EINVAL, "capacity must be a multiple of 32");
  const int64_t cap = eff_cap(*c);
  if (cap == 0) return fail(KVQ_EINVAL, "capacity must be given when window = 0");
  if (cap <= c->n_sink) return fail(KVQ_EINVAL, "capacity %lld must exceed n_sink %d", (long long)cap, c->n_sink);
  if (c->window > 0 && cap - c->n_sink <= c->window)
    return fail(KVQ_EINVAL, "capacity - n_sink must exceed window (one appended row before eviction)");
  if ((int64_t)c->batch * c->n_kv_heads * cap * c->head_dim > ((int64_t)1 << 40))
    return fail(KVQ_EINVAL, "cache too large");
  kvq::clear_error();
  return KVQ_OK;
}

kvqw_layout make_layout(const kvqw_config& c) {
  kvqw_layout L;
  std::memset(&L, 0, sizeof(L));
  const uint64_t S = (uint64_t)c.batch * c.n_kv_heads, D = c.head_dim, cap = (uint64_t)eff_cap(c);
  L.capacity = (int32_t)cap;
  uint64_t off = 0;
  L.k_codes = off;
  off = a256(off + S * cap * D);
  L.v_codes = off;
  off = a256(off + S * cap * D);
  L.k_scale = off;
  off = a256(off + S * D * 2);
  L.k_zero = off;
  off = a256(off + S * D * 2);
  L.v_scale = off;
  off = a256(off + S * cap * 2);
  L.v_zero = off;
  off = a256(off + S * cap * 2);
  L.sync = off;
  off = a256(off + S * 4);
  L.layer_stride = off;
  L.total = (uint64_t)c.n_layers * off;
  return L;
}

// Workspace: append (tile extremes, previous K metadata) and decode (split partials) share it.
uint64_t tiles_max(const kvqw_config& c) { return ((uint64_t)eff_cap(c) + RPT - 1) / RPT; }
uint64_t ws_part_bytes(const kvqw_config& c) {
  return a256((uint64_t)c.batch * c.n_kv_heads * tiles_max(c) * 2 * c.head_dim * 4);
}
uint64_t ws_bytes_of(const kvqw_config& c) {
  const uint64_t S = (uint64_t)c.batch * c.n_kv_heads;
  const uint64_t app = ws_part_bytes(c) + a256(S * 2 * c.head_dim * 2);
  const uint64_t dec = a256(S * MAX_SPLITS * (uint64_t)(c.n_q_heads / c.n_kv_heads) * (c.head_dim + 2) * 4);
  return std::max(app, dec);
}

}  // namespace

struct kvqw_cache {
  kvqw_config cfg;
  kvqw_layout lay;
  uint8_t* base;
  std::vector<int64_t> P, lo;
};

namespace {

kvqw::Shape shape_of(const kvqw_config& c) {
  kvqw::Shape s;
  s.B = c.batch;
  s.H = c.n_kv_heads;
  s.Hq = c.n_q_heads;
  s.D = c.head_dim;
  s.bits = c.bits;
  s.in_f32 = c.in_dtype == KVQ_IN_F32;
  s.cap = c.capacity;
  return s;
}

View view_of(const kvqw_cache* c, int layer) {
  uint8_t* b = c->base + (uint64_t)layer * c->lay.layer_stride;
  View v;
  v.kc = (int8_t*)(b + c->lay.k_codes);
  v.vc = (int8_t*)(b + c->lay.v_codes);
  v.ks = (uint16_t*)(b + c->lay.k_scale);
  v.kz = (uint16_t*)(b + c->lay.k_zero);
  v.vs = (uint16_t*)(b + c->lay.v_scale);
  v.vz = (uint16_t*)(b + c->lay.v_zero);
  v.sync = (uint32_t*)(b + c->lay.sync);
  return v;
}

// Stored rows: the first min(n_sink, P) positions, then [max(lo, n_sink), P).
Rows rows_of(const kvqw_config& c, int64_t P, int64_t lo) {
  Rows r;
  const int64_t ns = c.n_sink, r0 = std::max(lo, ns);
  r.n_sink = c.n_sink;
  r.ring = c.capacity - c.n_sink;
  r.nsk = (int)std::min(ns, P);
  r.nring = (int)std::max<int64_t>(0, P - r0);
  r.rs0 = r.nring > 0 ? (int)((r0 - ns) % r.ring) : 0;
  return r;
}

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

kvq_status check_layer(const kvqw_cache* c, int32_t layer) {
  if (!c) return fail(KVQ_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVQ_EINVAL, "layer %d out of range", layer);
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvqw_config_check(const kvqw_config* cfg) { return check(cfg); }

size_t kvqw_required_bytes(const kvqw_config* cfg) {
  if (check(cfg) != KVQ_OK) return 0;
  return (size_t)make_layout(*cfg).total;
}

kvq_status kvqw_get_layout(const kvqw_config* cfg, kvqw_layout* out) {
  kvq_status st = check(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_EINVAL, "out is NULL");
  *out = make_layout(*cfg);
  return KVQ_OK;
}

size_t kvqw_workspace_bytes(const kvqw_config* cfg) {
  if (check(cfg) != KVQ_OK) return 0;
  return (size_t)ws_bytes_of(*cfg);
}

kvq_status kvqw_create(const kvqw_config* cfg, void* dev_buf, size_t dev_bytes, void* stream, kvqw_cache** out) {
  kvq_status st = check(cfg);
  if (st != KVQ_OK) return st;
  if (!dev_buf || !out) return fail(KVQ_EINVAL, "dev_buf and out must not be NULL");
  if (((uintptr_t)dev_buf & 255) != 0) return fail(KVQ_EINVAL, "dev_buf must be 256-byte aligned");
  const kvqw_layout lay = make_layout(*cfg);
  if (dev_bytes < lay.total)
    return fail(KVQ_EINVAL, "dev_bytes %zu < required %llu", dev_bytes, (unsigned long long)lay.total);
  kvqw_cache* c = new (std::nothrow) kvqw_cache;
  if (!c) return fail(KVQ_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->cfg.capacity = lay.capacity;
  c->lay = lay;
  c->base = (uint8_t*)dev_buf;
  c->P.assign(cfg->n_layers, 0);
  c->lo.assign(cfg->n_layers, 0);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemsetAsync(dev_buf, 0, lay.total, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipMemsetAsync");
  }
  *out = c;
  kvq::clear_error();
  return KVQ_OK;
}

kvq_status kvqw_destroy(kvqw_cache* c) {
  if (!c) return fail(KVQ_EINVAL, "cache is NULL");
  delete c;
  return KVQ_OK;
}

kvq_status kvqw_append(kvqw_cache* c, int32_t layer, const void* k, const void* v, int32_t n, void* ws,
                       size_t ws_bytes, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!k || !v || !ws || n < 1) return fail(KVQ_EINVAL, "k, v and ws must not be NULL and n >= 1");
  if ((uintptr_t)k % 16 != 0 || (uintptr_t)v % 16 != 0 || (uintptr_t)ws % 16 != 0)
    return fail(KVQ_EINVAL, "k, v and ws must be 16-byte aligned");
  const kvqw_config& cf = c->cfg;
  if (ws_bytes < ws_bytes_of(cf)) return fail(KVQ_EINVAL, "ws_bytes too small");
  const int64_t P = c->P[layer], lo = c->lo[layer], ns = cf.n_sink, ring = cf.capacity - cf.n_sink;
  if (P + n > (int64_t)INT32_MAX) return fail(KVQ_ERANGE, "positions must stay below 2^31");
  if (P + n > ns && P + n - std::max(lo, ns) > ring)
    return fail(KVQ_ECAPACITY, "append of %d rows at P=%lld (lo=%lld) needs %lld ring slots, the cache has %lld; "
                "evict first or raise capacity", n, (long long)P, (long long)lo,
                (long long)(P + n - std::max(lo, ns)), (long long)ring);
  AppendArgs a;
  a.sh = shape_of(cf);
  a.v = view_of(c, layer);
  a.old = rows_of(cf, P, lo);
  a.k = k;
  a.vin = v;
  a.n = n;
  a.nsk_new = (int)std::max<int64_t>(0, std::min<int64_t>(ns, P + n) - P);
  a.ps0 = (int)((std::max(P, ns) - ns) % ring);
  a.tiles = (a.old.nsk + a.old.nring + n + RPT - 1) / RPT;
  a.part = (float*)ws;
  a.oldm = (uint16_t*)((uint8_t*)ws + ws_part_bytes(cf));
  hipError_t e = launch_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  c->P[layer] = P + n;
  return KVQ_OK;
}

kvq_status kvqw_evict(kvqw_cache* c, int32_t layer) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (c->cfg.window > 0) c->lo[layer] = std::max(c->lo[layer], c->P[layer] - (int64_t)c->cfg.window);
  return KVQ_OK;
}

kvq_status kvqw_decode_attn(kvqw_cache* c, int32_t layer, const void* q, float* out, float scale, void* ws,
                            size_t ws_bytes, void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!q || !out || !ws) return fail(KVQ_EINVAL, "q, out and ws must not be NULL");
  if ((uintptr_t)ws % 16 != 0) return fail(KVQ_EINVAL, "ws must be 16-byte aligned");
  const kvqw_config& cf = c->cfg;
  if (ws_bytes < ws_bytes_of(cf)) return fail(KVQ_EINVAL, "ws_bytes too small");
  if (c->P[layer] == 0) return fail(KVQ_ERANGE, "layer %d is empty", layer);
  DecodeArgs a;
  a.sh = shape_of(cf);
  a.v = view_of(c, layer);
  a.rows = rows_of(cf, c->P[layer], c->lo[layer]);
  a.q = q;
  a.out = out;
  a.part = (float*)ws;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)cf.head_dim);
  const int nst = a.rows.nsk + a.rows.nring;
  // the matrix-core kernel (head_dim 128) takes 32-row blocks, four per wave at least (512 rows per
  // split: 26 us for the call on the batch-8, T = 4096 layer, against 31 us at 256 and 32 us at 1024;
  // loading each wave's next block ahead gained nothing); only the last split ends early
  const int min_rows = cf.head_dim == 128 ? 2 * MIN_SPLIT_ROWS : MIN_SPLIT_ROWS;
  const int splits = std::max(1, std::min(MAX_SPLITS, nst / min_rows));  // one split below 2 * min_rows
  a.rows_per_split = (nst + splits - 1) / splits;
  if (cf.head_dim == 128) a.rows_per_split = (a.rows_per_split + 31) / 32 * 32;
  a.splits = (nst + a.rows_per_split - 1) / a.rows_per_split;
  hipError_t e = launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return KVQ_OK;
}

kvq_status kvqw_dequant(kvqw_cache* c, int32_t layer, int32_t which, int64_t pos0, int32_t count, uint16_t* out,
                        void* stream) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!out || count < 1 || (which != 0 && which != 1))
    return fail(KVQ_EINVAL, "out must not be NULL, count >= 1, which 0 (K) or 1 (V)");
  if ((uintptr_t)out % 2 != 0) return fail(KVQ_EINVAL, "out must be 2-byte aligned");
  const kvqw_config& cf = c->cfg;
  const int64_t P = c->P[layer], lo = c->lo[layer], ns = cf.n_sink;
  const int64_t a_end = std::min(ns, P), b_start = std::max(lo, ns);  // stored: [0, a_end) and [b_start, P)
  const bool gap_hit = a_end < b_start && pos0 < b_start && pos0 + count > a_end;
  if (pos0 < 0 || pos0 + count > P || gap_hit)
    return fail(KVQ_ERANGE, "positions [%lld, %lld) are not all stored (P=%lld, lo=%lld, n_sink=%d)",
                (long long)pos0, (long long)(pos0 + count), (long long)P, (long long)lo, cf.n_sink);
  DequantArgs a;
  a.sh = shape_of(cf);
  a.v = view_of(c, layer);
  a.which = which;
  a.count = count;
  a.n_sink = cf.n_sink;
  a.ring = cf.capacity - cf.n_sink;
  a.pos0 = pos0;
  a.out = out;
  hipError_t e = launch_dequant(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return KVQ_OK;
}

kvq_status kvqw_account(const kvqw_cache* c, int32_t layer, kvqw_bytes* out) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_EINVAL, "out is NULL");
  const kvqw_config& cf = c->cfg;
  const Rows r = rows_of(cf, c->P[layer], c->lo[layer]);
  const int64_t S = (int64_t)cf.batch * cf.n_kv_heads, D = cf.head_dim, n = r.nsk + r.nring;
  std::memset(out, 0, sizeof(*out));
  out->n_stored = n;
  out->current_length = c->P[layer];
  out->code_bytes = S * 2 * n * D;
  out->meta_bytes = S * (2 * 2 * D + 2 * 2 * n);
  out->packed_int4_bytes = S * n * D + out->meta_bytes;
  out->bf16_bytes = S * 2 * 2 * n * D;
  return KVQ_OK;
}

kvq_status kvqw_get_state(const kvqw_cache* c, int32_t layer, int64_t* P, int64_t* lo) {
  kvq_status st = check_layer(c, layer);
  if (st != KVQ_OK) return st;
  if (P) *P = c->P[layer];
  if (lo) *lo = c->lo[layer];
  return KVQ_OK;
}

}  // extern "C"
