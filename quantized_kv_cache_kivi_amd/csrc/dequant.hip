// Materialisation of cached values as fp16 (kvq_dequant): one wave per row.
//
// Read priority sink pool > fp16 window > bulk (q2k pull-request page,
// "Summary": the overlay over the sink cells and the recent cells reads
// exact).  Bulk values use each format's dequant formula in fp32 with the
// fp16 metadata cast to fp32 first ("StreamingLLM + KIVI — long-context decode
// without growing the KV cache", "Affine quantisation formula" and "The bug
// class the previous attempt hit", 2), then one rounding to fp16.  TurboQuant
// rows are looked up and rotated back, sigma * (c_d * FWHT(n * c[u]))
// ("TurboQuant KV Cache Compression — Spec", "Step 2", "Hadamard Transform
// Detail").
#include "device_common.h"

namespace kvq {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void k_dequant(DequantArgs a) {
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int D = sh.D, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = blockIdx.y, b = s / sh.Hkv;
  const int i = blockIdx.x * (NT / 64) + w;
  if (i >= a.count) return;
  const int64_t p = a.pos0 + i;
  const bool is_k = a.which == 0;
  uint16_t* out = a.out + ((int64_t)s * a.count + i) * sh.Din;  // rows of the caller's Din channels
  const bool act = 2 * lane < D;
  const bool wr = 2 * lane < sh.Din;  // Din is even: a lane writes both of its channels or neither
  // sink pool
  int slot = -1;
  if (sh.n_sink > 0) {
    const int cnt = lv.sink_count[b];
    for (int q = 0; q < cnt; ++q)
      if (lv.sink_pos[b * sh.n_sink + q] == p) slot = q;
  }
  if (slot >= 0 || p >= a.P - sh.R) {
    const uint16_t* src = slot >= 0 ? (is_k ? lv.sink_k : lv.sink_v) + ((int64_t)s * sh.n_sink + slot) * D
                                    : (is_k ? lv.win_k : lv.win_v) + ((int64_t)s * sh.R + p % sh.R) * D;
    if (wr) {
      out[2 * lane] = src[2 * lane];
      out[2 * lane + 1] = src[2 * lane + 1];
    }
    return;
  }
  const int64_t blk = p / G;
  const int t = (int)(p % G);
  const uint8_t* rec = lv.bulk + ((int64_t)s * lv.cap_b + blk % lv.cap_b) * lv.rec;
  const int nb = is_k ? sh.kb : sh.vb;
  const uint8_t* codes = rec + (is_k ? lv.k_codes : lv.v_codes);
  float x[2];
  uint32_t u[2];
  for (int e = 0; e < 2; ++e) {
    const int c = act ? 2 * lane + e : 0;
    int wd, k;
    if (nb == 3) {  // dense 3-bit stream
      u[e] = code3_at(codes, is_k ? k_bit3(t, c, D) : v_bit3(t, c, D));
      continue;
    }
    if (is_k) k_code_pos(t, c, D, nb, &wd, &k);
    else v_code_pos(t, c, D, nb, &wd, &k);
    u[e] = (reinterpret_cast<const uint32_t*>(codes)[wd] >> code_shift(k, nb)) & ((1u << nb) - 1u);
  }
  if (sh.fmt == KVQ_FMT_TQ) {
    const float nrm = reinterpret_cast<const float*>(rec + (is_k ? lv.k_meta : lv.v_meta))[t];
    const float* cen = is_k ? lv.tables->k_cen : lv.tables->v_cen;
    float y0 = act ? nrm * cen[u[0]] : 0.f, y1 = act ? nrm * cen[u[1]] : 0.f;
    wave_fwht(y0, y1, D, lane);
    const float cd = (float)(1.0 / __builtin_sqrt((double)D));
    x[0] = act ? lv.tables->signs[2 * lane] * (y0 * cd) : 0.f;
    x[1] = act ? lv.tables->signs[2 * lane + 1] * (y1 * cd) : 0.f;
  } else {
    const uint16_t* m = reinterpret_cast<const uint16_t*>(rec + (is_k ? lv.k_meta : lv.v_meta));
    const int ng = D / 32;
    for (int e = 0; e < 2; ++e) {
      const int c = act ? 2 * lane + e : 0;
      if (sh.fmt == KVQ_FMT_KIVI) {
        const int mi = v_meta_idx(t, c >> 5, ng);
        const float sc = is_k ? f16_val(m[c]) : f16_val(m[mi]);
        const float z = is_k ? f16_val(m[D + c]) : f16_val(m[G * ng + mi]);
        const float prod = (float)u[e] * sc;
        x[e] = prod + z;
      } else if (is_k) {
        x[e] = lv.tables->q2k_lvl[u[e]] * f16_val(m[c]);
      } else {
        x[e] = ((float)u[e] - 8.f) * f16_val(m[v_meta_idx(t, c >> 5, ng)]);
      }
    }
  }
  if (wr) {
    out[2 * lane] = f16_bits(x[0]);
    out[2 * lane + 1] = f16_bits(x[1]);
  }
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  dim3 grid((a.count + NT / 64 - 1) / (NT / 64), a.sh.B * a.sh.Hkv);
  hipLaunchKernelGGL(k_dequant, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
