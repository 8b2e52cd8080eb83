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

// MD: the widest stored row the instance takes (128, or 256 for TurboQuant rows of head_dim 160);
// lane l holds channels 128h + 2l + e in x[2h + e].
template <int MD>
__global__ __launch_bounds__(NT) void k_dequant(DequantArgs a) {
  constexpr int NK = MD / 64;
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int D = sh.D, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = blockIdx.y, b = s / sh.Hkv;
  const int i = blockIdx.x * (NT / 64) + w;
  if (i >= a.count) return;
  const int64_t p = a.pos0 + i;
  const bool is_k = a.which == 0;
  uint16_t* out = a.out + ((int64_t)s * a.count + i) * sh.Din;  // rows of the caller's Din channels
  // Din is even: a lane writes both channels of a pair or neither
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
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = row_chan(lane, k);
      if (c < sh.Din) out[c] = src[c];
    }
    return;
  }
  const int64_t blk = p / G;
  const int t = (int)(p % G);
  const uint8_t* rec = lv.bulk + ((int64_t)s * lv.cap_b + blk % lv.cap_b) * lv.rec;
  const int nb = is_k ? sh.kb : sh.vb;
  const uint8_t* codes = rec + (is_k ? lv.k_codes : lv.v_codes);
  float x[NK];
  uint32_t u[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int c0 = row_chan(lane, k), c = c0 < D ? c0 : 0;
    int wd, kk;
    if (nb == 3) {  // dense 3-bit stream
      u[k] = code3_at(codes, is_k ? k_bit3(t, c, D) : v_bit3(t, c, D));
      continue;
    }
    if (is_k) k_code_pos(t, c, D, nb, &wd, &kk);
    else v_code_pos(t, c, D, nb, &wd, &kk);
    u[k] = (reinterpret_cast<const uint32_t*>(codes)[wd] >> code_shift(kk, nb)) & ((1u << nb) - 1u);
  }
  if (sh.fmt == KVQ_FMT_TQ) {
    const float nrm = reinterpret_cast<const float*>(rec + (is_k ? lv.k_meta : lv.v_meta))[t];
    const float* cen = is_k ? lv.tables->k_cen : lv.tables->v_cen;
    float y[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) y[k] = row_chan(lane, k) < D ? nrm * cen[u[k]] : 0.f;
    row_fwht<MD>(y, D, lane);
    const float cd = (float)(1.0 / __builtin_sqrt((double)D));
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = row_chan(lane, k);
      x[k] = c < D ? lv.tables->signs[c] * (y[k] * cd) : 0.f;
    }
  } else {
    const uint16_t* m = reinterpret_cast<const uint16_t*>(rec + (is_k ? lv.k_meta : lv.v_meta));
    const int ng = D / 32;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c0 = row_chan(lane, k), c = c0 < D ? c0 : 0;
      if (sh.fmt == KVQ_FMT_KIVI) {
        const int mi = v_meta_idx(t, c >> 5, ng);
        const float sc = is_k ? f16_val(m[c]) : f16_val(m[mi]);
        const float z = is_k ? f16_val(m[D + c]) : f16_val(m[G * ng + mi]);
        const float prod = (float)u[k] * sc;
        x[k] = prod + z;
      } else if (is_k) {
        x[k] = lv.tables->q2k_lvl[u[k]] * f16_val(m[c]);
      } else {
        x[k] = ((float)u[k] - 8.f) * f16_val(m[v_meta_idx(t, c >> 5, ng)]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int c = row_chan(lane, k);
    if (c < sh.Din) out[c] = f16_bits(x[k]);
  }
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  dim3 grid((a.count + NT / 64 - 1) / (NT / 64), a.sh.B * a.sh.Hkv);
  if (a.sh.D > MAX_D) hipLaunchKernelGGL(k_dequant<MAX_SD>, grid, dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(k_dequant<MAX_D>, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
