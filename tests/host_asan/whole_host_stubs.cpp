// CPU stand-ins for the HIP runtime and the whole-T kernel launches, so that the host code of the
// whole-T cache (kvqw_api.cpp) runs under AddressSanitizer and UBSan with the call sequences the bench
// uses (the page model: 12 layers, 4-token prompt, 524 steps; the batch-8 bandwidth layer).  Every launch
// checks that each pointer it would hand a kernel, and the extent the kernel would touch, lies inside the
// buffers the caller allocated.
#include <hip/hip_runtime_api.h>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>
#include "whole_internal.h"

struct Buf { const char* name; uint8_t* p; size_t n; };
std::vector<Buf> g_bufs;
static long g_checks = 0;
static void inside(const void* p, size_t n, const char* what) {
  ++g_checks;
  for (auto& b : g_bufs)
    if ((const uint8_t*)p >= b.p && (const uint8_t*)p + n <= b.p + b.n) return;
  fprintf(stderr, "OUT OF BOUNDS: %s %p + %zu\n", what, p, n);
  abort();
}

extern "C" {
hipError_t hipMemsetAsync(void* dst, int value, size_t sizeBytes, hipStream_t) {
  inside(dst, sizeBytes, "memset");
  memset(dst, value, sizeBytes);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace kvq {
static std::string g_err;
kvq_status set_error(kvq_status st, const char* msg) { g_err = msg; return st; }
void clear_error() { g_err.clear(); }
}

namespace kvqw {
static void view_ok(const Shape& sh, const View& v) {
  const size_t S = (size_t)sh.B * sh.H;
  inside(v.kc, S * sh.cap * sh.D, "kc");
  inside(v.vc, S * sh.cap * sh.D, "vc");
  inside(v.ks, S * sh.D * 2, "ks");
  inside(v.kz, S * sh.D * 2, "kz");
  inside(v.vs, S * sh.cap * 2, "vs");
  inside(v.vz, S * sh.cap * 2, "vz");
}
static void rows_ok(const Shape& sh, const Rows& r) {
  if (r.nsk < 0 || r.nring < 0 || r.nsk > r.n_sink || r.nring > r.ring || r.rs0 < 0 || r.rs0 >= (r.ring > 0 ? r.ring : 1) ||
      r.n_sink + r.ring != sh.cap) { fprintf(stderr, "bad rows\n"); abort(); }
}
hipError_t launch_append(const AppendArgs& a, hipStream_t) {
  view_ok(a.sh, a.v);
  rows_ok(a.sh, a.old);
  const size_t S = (size_t)a.sh.B * a.sh.H, esz = a.sh.in_f32 ? 4 : 2;
  inside(a.k, S * a.n * a.sh.D * esz, "k");
  inside(a.vin, S * a.n * a.sh.D * esz, "v");
  if (a.tiles < 1 || a.tiles * RPT < a.old.nsk + a.old.nring + a.n) { fprintf(stderr, "tiles\n"); abort(); }
  inside(a.part, S * a.tiles * 2 * a.sh.D * 4, "part");
  inside(a.oldm, S * 2 * a.sh.D * 2, "oldm");
  if (a.old.nsk + a.old.nring + a.n > a.sh.cap) { fprintf(stderr, "rows beyond capacity\n"); abort(); }
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  view_ok(a.sh, a.v);
  rows_ok(a.sh, a.rows);
  const size_t S = (size_t)a.sh.B * a.sh.H, r = a.sh.Hq / a.sh.H, esz = a.sh.in_f32 ? 4 : 2;
  inside(a.q, (size_t)a.sh.B * a.sh.Hq * a.sh.D * esz, "q");
  inside(a.out, (size_t)a.sh.B * a.sh.Hq * a.sh.D * 4, "out");
  if (a.splits < 1 || a.splits > MAX_SPLITS || a.rows_per_split < 1 ||
      (size_t)a.splits * a.rows_per_split < (size_t)(a.rows.nsk + a.rows.nring)) { fprintf(stderr, "splits\n"); abort(); }
  inside(a.part, S * a.splits * r * (a.sh.D + 2) * 4, "part");
  return hipSuccess;
}
hipError_t launch_dequant(const DequantArgs& a, hipStream_t) {
  view_ok(a.sh, a.v);
  inside(a.out, (size_t)a.sh.B * a.sh.H * a.count * a.sh.D * 2, "dequant out");
  return hipSuccess;
}
}  // namespace kvqw

static uint8_t* alloc(const char* name, size_t n) {
  uint8_t* p = (uint8_t*)aligned_alloc(256, (n + 255) / 256 * 256);
  memset(p, 0, n);
  g_bufs.push_back({name, p, n});
  return p;
}

static void run(const kvqw_config& cfg, int prompt, int steps, bool decode) {
  const size_t nb = kvqw_required_bytes(&cfg), wsb = kvqw_workspace_bytes(&cfg);
  uint8_t* dev = alloc("cache", nb);
  uint8_t* ws = alloc("ws", wsb);
  const int S = cfg.batch * cfg.n_kv_heads, D = cfg.head_dim, esz = cfg.in_dtype ? 4 : 2;
  uint8_t* k0 = alloc("k0", (size_t)S * prompt * D * esz);
  uint8_t* v0 = alloc("v0", (size_t)S * prompt * D * esz);
  uint8_t* k1 = alloc("k1", (size_t)S * D * esz);
  uint8_t* v1 = alloc("v1", (size_t)S * D * esz);
  uint8_t* q = alloc("q", (size_t)cfg.batch * cfg.n_q_heads * D * esz);
  float* out = (float*)alloc("out", (size_t)cfg.batch * cfg.n_q_heads * D * 4);
  kvqw_cache* c = nullptr;
  if (kvqw_create(&cfg, dev, nb, nullptr, &c) != KVQ_OK) { fprintf(stderr, "create failed\n"); abort(); }
  for (int l = 0; l < cfg.n_layers; ++l) {
    if (kvqw_append(c, l, k0, v0, prompt, ws, wsb, nullptr) != KVQ_OK) abort();
    kvqw_evict(c, l);
  }
  for (int i = 0; i < steps; ++i)
    for (int l = 0; l < cfg.n_layers; ++l) {
      if (kvqw_append(c, l, k1, v1, 1, ws, wsb, nullptr) != KVQ_OK) { fprintf(stderr, "append %d failed\n", i); abort(); }
      kvqw_evict(c, l);
      if (decode && kvqw_decode_attn(c, l, q, out, 0.f, ws, wsb, nullptr) != KVQ_OK) abort();
    }
  kvqw_destroy(c);
  g_bufs.clear();
}

int main() {
  kvqw_config page{};  // the page's model: 12 layers, batch 1, 8 heads, d=32, int8, sink 4 + window 256, fp32
  page.n_layers = 12; page.batch = 1; page.n_kv_heads = 8; page.n_q_heads = 8; page.head_dim = 32; page.bits = 8;
  page.n_sink = 4; page.window = 256; page.capacity = 0; page.in_dtype = 1;
  run(page, 4, 524, true);
  kvqw_config bw{};  // the bandwidth workload: 1 layer, batch 8, 8/32 heads, d=128, int8, T=4096, no eviction
  bw.n_layers = 1; bw.batch = 8; bw.n_kv_heads = 8; bw.n_q_heads = 32; bw.head_dim = 128; bw.bits = 8;
  bw.n_sink = 0; bw.window = 0; bw.capacity = 4096 + 64; bw.in_dtype = 0;
  run(bw, 4096, 24, true);
  printf("ok: %ld bounds checks, no host memory error\n", g_checks);
  return 0;
}
