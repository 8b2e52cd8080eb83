// Kernels of the whole-T KIVI cache (kvq_whole.h), following "StreamingLLM + KIVI — long-context
// decode without growing the KV cache": "KIVI — int8/int4 KV cache with greedy-lossless decode"
// (K per channel over every stored token, re-computed on each append; V per token), "Affine
// quantisation formula" (scale = max(1e-5, range / (qMax - qMin)), zero = min, signed codes),
// "Storage layout" (int8 rows, fp16 per-channel K and per-row V metadata) and "Caveats" (the
// whole stored K is re-quantised on every append).
//
// Every kernel streams int8 rows: a thread owns 8 channels of a row (one 8-byte code load, one
// 16- or 32-byte input load), D/8 neighbouring lanes cover a row, and a wave walks 512/D rows at
// a time.  Per-row reductions (V min/max, scores) are xor shuffles inside the D/8-lane group.
//   append   k_stats:   per tile of 256 stored + new rows, the channel min/max of the stored K
//                       (dequantised with the current metadata) and of the new rows; the new V rows
//                       are quantised and stored on the way;
//            k_requant: every tile reduces the per-tile extremes to the new metadata, codes its
//                       new rows from the input and codes again, from their dequantised values, the
//                       stored rows of the channel groups whose scale or zero changed (the others
//                       code to the same bytes); tile 0 writes the metadata.  The previous metadata
//                       is read from the copy k_stats left in the workspace, so no tile sees a
//                       half-written table.
//            A short append to a short cache (FUSE_ROWS, FUSE_TILES) is one launch of
//            k_append_one: one workgroup per stream does both steps over all its tiles.
//   decode   k_decode:  split-K over the stored rows: the query is folded with the K scales once
//                       per workgroup (q'_c = q_c s_c, kappa = sum_c q_c z_c), score = q'.u + kappa,
//                       online softmax per row group, V rows dequantised in fp32; one partial
//                       (acc, m, l) per split and head; the last split of a stream to finish merges
//                       the stream's partials in fixed split order and writes the output.
#include "whole_internal.h"

namespace kvqw {
namespace {

constexpr int NT = 256;
constexpr float EPS = 1e-5f;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ float lo16(uint32_t w) { return f16_val((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi16(uint32_t w) { return f16_val((uint16_t)(w >> 16)); }

// Values that another workgroup of the same launch reads are stored and read with device-scope
// relaxed atomics (coherent across the XCDs' L2 caches); a workgroup waits for its stores
// (vmcnt(0)) before it counts itself in the stream's arrival counter.
__device__ __forceinline__ void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Counts the workgroup in counter `ctr` once its stores have completed; true in the last of `n`
// workgroups, which also resets the counter to zero for the next launch.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, int n) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t k = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = k == (uint32_t)(n - 1);
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return last != 0;
}

// Slot of stored row j (sinks first, then the ring rows).
__device__ __forceinline__ int row_slot(const Rows& r, int j) {
  if (j < r.nsk) return j;
  int t = r.rs0 + (j - r.nsk);
  if (t >= r.ring) t -= r.ring;
  return r.n_sink + t;
}

// Slot of new row i of an append.
__device__ __forceinline__ int new_slot(const AppendArgs& a, int i) {
  if (i < a.nsk_new) return a.old.nsk + i;  // positions below n_sink: every earlier row is a sink
  int t = a.ps0 + (i - a.nsk_new);
  if (t >= a.old.ring) t -= a.old.ring;
  return a.old.n_sink + t;
}

// 8 consecutive input elements (fp16 or fp32), 16-byte aligned.
template <bool F32>
__device__ __forceinline__ void ld8(const void* p, int64_t i, float* x) {
  if constexpr (F32) {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i);
    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __builtin_bit_cast(float, w[e]);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = lo16(w[m]);
      x[2 * m + 1] = hi16(w[m]);
    }
  }
}

// u = q - qMin of 8 signed codes, as fp32 (exact).  For a two's-complement byte b of q, q + 128 is
// b ^ 0x80 (int8) and q + 8 is (b ^ 0x08) & 0x0F (int4, q in [-8, 7]): one or two bit operations per
// word, then a byte-to-float conversion per code.
__device__ __forceinline__ void codes8(uint2 w, int qmin, float* u) {
  uint32_t ww[2] = {w.x, w.y};
#pragma unroll
  for (int m = 0; m < 2; ++m) ww[m] = qmin == -128 ? ww[m] ^ 0x80808080u : (ww[m] ^ 0x08080808u) & 0x0F0F0F0Fu;
#pragma unroll
  for (int e = 0; e < 8; ++e) u[e] = (float)((ww[e >> 2] >> (8 * (e & 3))) & 0xFFu);
}

// Signed codes of 8 values against fp32 scale and zero: u = clamp(rint((x - z)/s), 0, L), q = u + qMin.
__device__ __forceinline__ uint2 quant8(const float* x, const float* s, const float* z, float L, int qmin) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float u = fminf(fmaxf(rintf((x[e] - z[e]) / s[e]), 0.f), L);
    w[e >> 2] |= ((uint32_t)((int)u + qmin) & 0xFFu) << (8 * (e & 3));
  }
  return make_uint2(w[0], w[1]);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void ld_meta8(const uint16_t* p, float* x) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    x[2 * m] = lo16(w[m]);
    x[2 * m + 1] = hi16(w[m]);
  }
}

// Channel extremes of the rows of tile `tile` this thread covers (rows rl, rl + RP, ... of the tile,
// channels 8 cg .. 8 cg + 7), folded into mn, mx: stored rows dequantised with the current metadata
// (so, zo), new rows from the input; the new V rows are quantised and stored on the way.
template <int D, bool F32>
__device__ __forceinline__ void tile_extremes(const AppendArgs& a, int s, int tile, const float* so, const float* zo,
                                              float* mn, float* mx) {
  constexpr int CG = D / 8, RP = NT / CG;
  const Shape sh = a.sh;
  const int tid = threadIdx.x, cg = tid % CG, rl = tid / CG;
  const int qmin = sh.bits == 8 ? -128 : -8;
  const float L = (float)((1 << sh.bits) - 1);
  const int nold = a.old.nsk + a.old.nring, ntot = nold + a.n;
  const int j0 = tile * RPT, j1 = min(ntot, j0 + RPT);
  const int64_t in0 = (int64_t)s * a.n;
  const int jo = min(j1, nold);
  if (j0 + rl < jo) {
    // stored rows: the dequantised value fl(fl(u s) + z) is non-decreasing in the code u (s > 0), so
    // its extremes over the rows are those of the extreme codes, reduced as integers.  Every load of
    // the thread is issued first; a row past the tile's stored rows repeats the thread's first row.
    constexpr int NR = RPT / RP;
    uint2 w[NR];
    const int8_t* kc = a.v.kc + (int64_t)s * sh.cap * D + 8 * cg;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int j = j0 + rl + r * RP;
      w[r] = *reinterpret_cast<const uint2*>(kc + (int64_t)row_slot(a.old, j < jo ? j : j0 + rl) * D);
    }
    // per word m: the even bytes (mask 0x00FF00FF) and the odd bytes (shifted down) as 16-bit lanes
    u16x2 lo[4], hi[4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t ww[2] = {w[r].x, w[r].y};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t u = qmin == -128 ? ww[m] ^ 0x80808080u : (ww[m] ^ 0x08080808u) & 0x0F0F0F0Fu;
        const u16x2 ev = __builtin_bit_cast(u16x2, u & 0x00FF00FFu), od = __builtin_bit_cast(u16x2, (u >> 8) & 0x00FF00FFu);
        lo[2 * m] = r == 0 ? ev : __builtin_elementwise_min(lo[2 * m], ev);
        hi[2 * m] = r == 0 ? ev : __builtin_elementwise_max(hi[2 * m], ev);
        lo[2 * m + 1] = r == 0 ? od : __builtin_elementwise_min(lo[2 * m + 1], od);
        hi[2 * m + 1] = r == 0 ? od : __builtin_elementwise_max(hi[2 * m + 1], od);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // byte e of word e / 4: lane (e & 3) >> 1 of the even (e even) or odd word
      const int wi = 2 * (e >> 2) + (e & 1), li = (e & 3) >> 1;
      const float ulo = (float)lo[wi][li], uhi = (float)hi[wi][li];
      mn[e] = fminf(mn[e], ulo * so[e] + zo[e]);  // two roundings (no contraction)
      mx[e] = fmaxf(mx[e], uhi * so[e] + zo[e]);
    }
  }
  for (int j = max(j0, nold) + rl; j < j1; j += RP) {  // new rows
    float x[8];
    const int i = j - nold;
    ld8<F32>(a.k, (in0 + i) * D + 8 * cg, x);
    // the new V row: per-token min/max over all channels, final at append
    float v[8];
    ld8<F32>(a.vin, (in0 + i) * D + 8 * cg, v);
    float vmn = v[0], vmx = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      vmn = fminf(vmn, v[e]);
      vmx = fmaxf(vmx, v[e]);
    }
#pragma unroll
    for (int o = CG / 2; o >= 1; o >>= 1) {
      vmn = fminf(vmn, __shfl_xor(vmn, o));
      vmx = fmaxf(vmx, __shfl_xor(vmx, o));
    }
    vmn = vmn + 0.f;
    vmx = vmx + 0.f;
    const uint16_t s16 = f16_bits(fmaxf(EPS, (vmx - vmn) / L)), z16 = f16_bits(vmn);
    float sv[8], zv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = f16_val(s16);
      zv[e] = f16_val(z16);
    }
    const int64_t ro = (int64_t)s * sh.cap + new_slot(a, i);
    *reinterpret_cast<uint2*>(a.v.vc + ro * D + 8 * cg) = quant8(v, sv, zv, L, qmin);
    if (cg == 0) {
      a.v.vs[ro] = s16;
      a.v.vz[ro] = z16;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = fminf(mn[e], x[e]);
      mx[e] = fmaxf(mx[e], x[e]);
    }
  }
}

// Per-channel extremes of the workgroup's threads (mn, mx of each row lane) into m0[c], m1[c]
// (c < D, threads tid < D).
template <int D>
__device__ __forceinline__ void block_extremes(const float* mn, const float* mx, float& m0, float& m1) {
  constexpr int CG = D / 8, RP = NT / CG;
  __shared__ float smn[RP * D], smx[RP * D];
  const int tid = threadIdx.x, cg = tid % CG, rl = tid / CG;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    smn[rl * D + 8 * cg + e] = mn[e];
    smx[rl * D + 8 * cg + e] = mx[e];
  }
  __syncthreads();
  m0 = INFINITY;
  m1 = -INFINITY;
  if (tid < D) {
    for (int r = 0; r < RP; ++r) {
      m0 = fminf(m0, smn[r * D + tid]);
      m1 = fmaxf(m1, smx[r * D + tid]);
    }
  }
}

template <int D, bool F32>
__global__ __launch_bounds__(NT) void k_stats(AppendArgs a) {
  constexpr int CG = D / 8;
  const int s = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x, cg = tid % CG;
  float so[8], zo[8], mn[8], mx[8];
  ld_meta8(a.v.ks + (int64_t)s * D + 8 * cg, so);
  ld_meta8(a.v.kz + (int64_t)s * D + 8 * cg, zo);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = INFINITY;
    mx[e] = -INFINITY;
  }
  tile_extremes<D, F32>(a, s, tile, so, zo, mn, mx);
  float m0, m1;
  block_extremes<D>(mn, mx, m0, m1);
  if (tid < D) {
    float* pp = a.part + ((int64_t)s * a.tiles + tile) * 2 * D;
    pp[tid] = m0;
    pp[D + tid] = m1;
    if (tile == 0) {
      a.oldm[(int64_t)s * 2 * D + tid] = a.v.ks[(int64_t)s * D + tid];
      a.oldm[(int64_t)s * 2 * D + D + tid] = a.v.kz[(int64_t)s * D + tid];
    }
  }
}

template <int D, bool F32>
__global__ __launch_bounds__(NT) void k_requant(AppendArgs a) {
  constexpr int CG = D / 8, RP = NT / CG;
  const Shape sh = a.sh;
  const int s = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  const int cg = tid % CG, rl = tid / CG;
  const int qmin = sh.bits == 8 ? -128 : -8;
  const float L = (float)((1 << sh.bits) - 1);
  const int nold = a.old.nsk + a.old.nring, ntot = nold + a.n;
  const int j0 = tile * RPT, j1 = min(ntot, j0 + RPT);
  __shared__ float sns[D], snz[D], sos[D], soz[D];
  constexpr int TG = NT / D;  // threads per channel for the tile reduction
  __shared__ float rmn[TG][D], rmx[TG][D];
  {
    // channel min/max over every row: the per-tile extremes (min and max are exact, so the
    // reduction order does not matter)
    const int c = tid % D, tg = tid / D;
    float m0 = INFINITY, m1 = -INFINITY;
    const float* pp = a.part + (int64_t)s * a.tiles * 2 * D;
#pragma unroll 4
    for (int t = tg; t < a.tiles; t += TG) {
      m0 = fminf(m0, pp[t * 2 * D + c]);
      m1 = fmaxf(m1, pp[t * 2 * D + D + c]);
    }
    rmn[tg][c] = m0;
    rmx[tg][c] = m1;
  }
  __syncthreads();
  if (tid < D) {
    float m0 = rmn[0][tid], m1 = rmx[0][tid];
#pragma unroll
    for (int t = 1; t < TG; ++t) {
      m0 = fminf(m0, rmn[t][tid]);
      m1 = fmaxf(m1, rmx[t][tid]);
    }
    m0 = m0 + 0.f;
    m1 = m1 + 0.f;
    const uint16_t s16 = f16_bits(fmaxf(EPS, (m1 - m0) / L)), z16 = f16_bits(m0);
    sns[tid] = f16_val(s16);
    snz[tid] = f16_val(z16);
    sos[tid] = f16_val(a.oldm[(int64_t)s * 2 * D + tid]);
    soz[tid] = f16_val(a.oldm[(int64_t)s * 2 * D + D + tid]);
    if (tile == 0) {
      a.v.ks[(int64_t)s * D + tid] = s16;
      a.v.kz[(int64_t)s * D + tid] = z16;
    }
  }
  __syncthreads();
  // A stored code u of a channel whose scale s and zero z did not change codes to u again:
  // fl(u s + z) - z and its quotient by s stay within 2^-24 (|z| / s + 3u) of u (u s is exact), below
  // 1/2 when |z| <= 2^22 s.  Such channels keep their stored bytes; a group of 8 channels is coded
  // again when any of them changed or fails the bound (a few per append in steady state).  The
  // tile's (stored row, group to code again) pairs are spread over all threads, so a few changed
  // groups cost a few pairs per thread.
  __shared__ int glist[CG];
  __shared__ int ngch;
  if (tid < 64) {
    bool same = true;
    if (tid < CG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * tid + e;
        same = same && sns[c] == sos[c] && snz[c] == soz[c] && fabsf(soz[c]) <= 4194304.f * sos[c];
      }
    }
    const uint64_t chg = __ballot(tid < CG && !same);
    if (tid < CG && !same) glist[__popcll(chg & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) ngch = __popcll(chg);
  }
  __syncthreads();
  const int64_t in0 = (int64_t)s * a.n;
  const int jo = min(j1, nold), ng = ngch;
  const int items = (jo > j0 ? jo - j0 : 0) * ng;
#pragma unroll 2
  for (int it = tid; it < items; it += NT) {  // stored rows of the changed groups, coded again in place
    const int j = j0 + it / ng, gsel = glist[it % ng];
    float x[8], gs[8], gz[8];
    int8_t* row = a.v.kc + ((int64_t)s * sh.cap + row_slot(a.old, j)) * D + 8 * gsel;
    codes8(*reinterpret_cast<const uint2*>(row), qmin, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = x[e] * sos[8 * gsel + e] + soz[8 * gsel + e];
      gs[e] = sns[8 * gsel + e];
      gz[e] = snz[8 * gsel + e];
    }
    *reinterpret_cast<uint2*>(row) = quant8(x, gs, gz, L, qmin);
  }
  float ns[8], nz[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ns[e] = sns[8 * cg + e];
    nz[e] = snz[8 * cg + e];
  }
  for (int j = max(j0, nold) + rl; j < j1; j += RP) {  // new rows
    float x[8];
    const int i = j - nold;
    ld8<F32>(a.k, (in0 + i) * D + 8 * cg, x);
    *reinterpret_cast<uint2*>(a.v.kc + ((int64_t)s * sh.cap + new_slot(a, i)) * D + 8 * cg) =
        quant8(x, ns, nz, L, qmin);
  }
}

// A short append to a short cache (at most FUSE_TILES tiles) by one workgroup per stream: the tiles'
// extremes in turn, then the new metadata, the new rows coded against it, and the stored rows of the
// channel groups whose scale or zero changed coded again (as k_stats + k_requant do over all tiles).
template <int D, bool F32>
__global__ __launch_bounds__(NT) void k_append_one(AppendArgs a) {
  constexpr int CG = D / 8;
  const Shape sh = a.sh;
  const int s = blockIdx.y, tid = threadIdx.x, cg = tid % CG;
  const int qmin = sh.bits == 8 ? -128 : -8;
  const float L = (float)((1 << sh.bits) - 1);
  const int nold = a.old.nsk + a.old.nring;
  __shared__ float sns[D], snz[D], sos[D], soz[D];
  __shared__ int glist[CG];
  __shared__ int ngch;
  {
    float so[8], zo[8], mn[8], mx[8];
    ld_meta8(a.v.ks + (int64_t)s * D + 8 * cg, so);
    ld_meta8(a.v.kz + (int64_t)s * D + 8 * cg, zo);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = INFINITY;
      mx[e] = -INFINITY;
    }
    for (int tile = 0; tile < a.tiles; ++tile) tile_extremes<D, F32>(a, s, tile, so, zo, mn, mx);
    float m0, m1;
    block_extremes<D>(mn, mx, m0, m1);
    if (tid < D) {
      m0 = m0 + 0.f;
      m1 = m1 + 0.f;
      const uint16_t s16 = f16_bits(fmaxf(EPS, (m1 - m0) / L)), z16 = f16_bits(m0);
      sns[tid] = f16_val(s16);
      snz[tid] = f16_val(z16);
      sos[tid] = f16_val(a.v.ks[(int64_t)s * D + tid]);
      soz[tid] = f16_val(a.v.kz[(int64_t)s * D + tid]);
      a.v.ks[(int64_t)s * D + tid] = s16;
      a.v.kz[(int64_t)s * D + tid] = z16;
    }
  }
  __syncthreads();
  if (tid < 64) {
    bool same = true;
    if (tid < CG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * tid + e;
        same = same && sns[c] == sos[c] && snz[c] == soz[c] && fabsf(soz[c]) <= 4194304.f * sos[c];
      }
    }
    const uint64_t chg = __ballot(tid < CG && !same);
    if (tid < CG && !same) glist[__popcll(chg & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) ngch = __popcll(chg);
  }
  __syncthreads();
  // stored rows of the changed groups, coded again in place: U (row, group) items per thread and
  // memory round trip (an item past the last repeats the thread's first and is not stored)
  constexpr int U = 16;
  const int ng = ngch, items = nold * ng;
  for (int it0 = tid; it0 < items; it0 += NT * U) {
    uint2 w[U];
    int8_t* rp[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int it = it0 + k * NT < items ? it0 + k * NT : it0;
      rp[k] = a.v.kc + ((int64_t)s * sh.cap + row_slot(a.old, it / ng)) * D + 8 * glist[it % ng];
      w[k] = *reinterpret_cast<const uint2*>(rp[k]);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int it = it0 + k * NT;
      if (it < items) {
        const int gsel = glist[it % ng];
        float x[8], gs[8], gz[8];
        codes8(w[k], qmin, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = x[e] * sos[8 * gsel + e] + soz[8 * gsel + e];
          gs[e] = sns[8 * gsel + e];
          gz[e] = snz[8 * gsel + e];
        }
        *reinterpret_cast<uint2*>(rp[k]) = quant8(x, gs, gz, L, qmin);
      }
    }
  }
  const int64_t in0 = (int64_t)s * a.n;
  for (int it = tid; it < a.n * CG; it += NT) {  // new rows
    const int i = it / CG, g = it % CG;
    float x[8], gs[8], gz[8];
    ld8<F32>(a.k, (in0 + i) * D + 8 * g, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gs[e] = sns[8 * g + e];
      gz[e] = snz[8 * g + e];
    }
    *reinterpret_cast<uint2*>(a.v.kc + ((int64_t)s * sh.cap + new_slot(a, i)) * D + 8 * g) = quant8(x, gs, gz, L, qmin);
  }
}

// The output of every query head of stream s, by the last split workgroup: the split partials
// (acc, m, l) merged in split order, MC partials per memory round trip (the running maximum and sums
// rescaled between chunks).
template <int D, int R>
__device__ void merge_last(const DecodeArgs& a, int s) {
  constexpr int MC = 16;
  const Shape sh = a.sh;
  const int b = s / sh.H, g = s % sh.H;
  const int64_t stride = (int64_t)R * (D + 2);
  for (int i = threadIdx.x; i < R * D; i += NT) {
    const int h = i / D, c = i % D;
    const float* base = a.part + ((int64_t)s * a.splits * R + h) * (D + 2);
    float M = -INFINITY, lv = 0.f, av = 0.f;
    for (int q0 = 0; q0 < a.splits; q0 += MC) {
      float mq[MC], lq[MC], xq[MC];
#pragma unroll
      for (int k = 0; k < MC; ++k) {  // past the last split: re-read it (no branch between the loads), unused
        const bool in = q0 + k < a.splits;
        const float* pq = base + (in ? q0 + k : a.splits - 1) * stride;
        const float m = ld_dev(pq + D), l = ld_dev(pq + D + 1), x = ld_dev(pq + c);
        mq[k] = in ? m : -INFINITY;
        lq[k] = in ? l : 0.f;
        xq[k] = in ? x : 0.f;
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < MC; ++k) Mn = fmaxf(Mn, mq[k]);
      const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);  // sums are 0 while M = -inf
      av = av * fo;
      lv = lv * fo;
#pragma unroll
      for (int k = 0; k < MC; ++k) {
        const float w = mq[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq[k] - Mn);
        av = av + xq[k] * w;
        lv = lv + lq[k] * w;
      }
      M = Mn;
    }
    a.out[((int64_t)b * sh.Hq + (int64_t)g * R + h) * D + c] = lv > 0.f ? av / lv : 0.f;
  }
}

// u = q - qMin of N codes held in N/4 words (see codes8).
template <int N>
__device__ __forceinline__ void codes_n(const uint32_t* w, int qmin, float* u) {
#pragma unroll
  for (int m = 0; m < N / 4; ++m) {
    const uint32_t x = qmin == -128 ? w[m] ^ 0x80808080u : (w[m] ^ 0x08080808u) & 0x0F0F0F0Fu;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[4 * m + e] = (float)((x >> (8 * e)) & 0xFFu);
  }
}

// CPL = 8 channels per lane (one 8-byte code load per row and operand); 16 channels per lane
// (16-byte loads, fewer shuffles) measured slower on the batch-8, T=4096, GQA-4 workload.
template <int D, int R, bool F32>
__global__ __launch_bounds__(NT) void k_decode(DecodeArgs a) {
  constexpr int CPL = 8;
  constexpr int CG = D / CPL, TPI = 64 / CG, NW = NT / 64, NWD = CPL / 4;
  const Shape sh = a.sh;
  const int s = blockIdx.y, split = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = s / sh.H, g = s % sh.H;
  const int cg = lane % CG, tau = lane / CG;
  const int qmin = sh.bits == 8 ? -128 : -8;
  __shared__ float sq[R][D], sqz[R][D], skap[R];
  __shared__ float smw[NW][R], slw[NW][R];
  __shared__ float sacc[NW][R][D];
  for (int i = tid; i < R * D; i += NT) {
    const int h = i / D, c = i % D;
    const int64_t qi = ((int64_t)b * sh.Hq + g * R + h) * D + c;
    const float qv = F32 ? static_cast<const float*>(a.q)[qi] : f16_val(static_cast<const uint16_t*>(a.q)[qi]);
    sq[h][c] = qv * f16_val(a.v.ks[(int64_t)s * D + c]);
    sqz[h][c] = qv * f16_val(a.v.kz[(int64_t)s * D + c]);
  }
  __syncthreads();
  if (wv == 0) {  // kappa_h = sum_c q_hc z_c: two channels per lane, then a wave sum
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float k = (lane < D ? sqz[h][lane] : 0.f) + (lane + 64 < D ? sqz[h][lane + 64] : 0.f);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) k = k + __shfl_xor(k, o);
      if (lane == 0) skap[h] = k;
    }
  }
  __syncthreads();
  float qf[R][CPL], kap[R], m[R], l[R], acc[R][CPL];
#pragma unroll
  for (int h = 0; h < R; ++h) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      qf[h][e] = sq[h][CPL * cg + e];
      acc[h][e] = 0.f;
    }
    kap[h] = skap[h];
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
  const float al = a.scale * LOG2E;
  const int nst = a.rows.nsk + a.rows.nring;
  const int j0 = split * a.rows_per_split, j1 = min(nst, j0 + a.rows_per_split);
  // NB rows per lane in flight: every row's codes are requested before the first is scored
  constexpr int STEP = NW * TPI, NB = 2;
  auto ld_codes = [&](const int8_t* p, uint32_t* w) {
    if constexpr (NWD == 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x;
      w[1] = x.y;
      w[2] = x.z;
      w[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x;
      w[1] = x.y;
    }
  };
  for (int j = j0 + wv * TPI + tau; j < j1; j += NB * STEP) {
    uint32_t kw[NB][NWD], vw[NB][NWD];
    uint16_t vsb[NB], vzb[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int jr = j + r * STEP < j1 ? j + r * STEP : j;  // past the end: reload row j, unused
      const int64_t ro = (int64_t)s * sh.cap + row_slot(a.rows, jr);
      ld_codes(a.v.kc + ro * D + CPL * cg, kw[r]);
      ld_codes(a.v.vc + ro * D + CPL * cg, vw[r]);
      vsb[r] = a.v.vs[ro];
      vzb[r] = a.v.vz[ro];
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (j + r * STEP >= j1) break;  // uniform over the row's lanes
      float uk[CPL], uv[CPL];
      codes_n<CPL>(kw[r], qmin, uk);
      codes_n<CPL>(vw[r], qmin, uv);
      const float vsf = f16_val(vsb[r]), vzf = f16_val(vzb[r]);
      float xv[CPL];
#pragma unroll
      for (int e = 0; e < CPL; ++e) xv[e] = __builtin_fmaf(uv[e], vsf, vzf);
#pragma unroll
      for (int h = 0; h < R; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) p = __builtin_fmaf(qf[h][e], uk[e], p);
#pragma unroll
        for (int o = CG / 2; o >= 1; o >>= 1) p = p + __shfl_xor(p, o);
        const float sc = (p + kap[h]) * al;
        if (sc > m[h]) {  // uniform over the row's lanes
          const float corr = __builtin_amdgcn_exp2f(m[h] - sc);  // 0 while m is -inf
          l[h] *= corr;
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[h][e] *= corr;
          m[h] = sc;
        }
        const float pw = __builtin_amdgcn_exp2f(sc - m[h]);
        l[h] += pw;
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[h][e] = __builtin_fmaf(pw, xv[e], acc[h][e]);
      }
    }
  }
  // row groups of the wave (lanes cg + CG*tau), then the waves through LDS
#pragma unroll
  for (int h = 0; h < R; ++h) {
    float M = m[h];
#pragma unroll
    for (int o = CG; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float w = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
    float lw = l[h] * w;
#pragma unroll
    for (int o = CG; o < 64; o <<= 1) lw = lw + __shfl_xor(lw, o);
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float aw = acc[h][e] * w;
#pragma unroll
      for (int o = CG; o < 64; o <<= 1) aw = aw + __shfl_xor(aw, o);
      acc[h][e] = aw;
    }
    m[h] = M;
    l[h] = lw;
  }
  if (tau == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) sacc[wv][h][CPL * cg + e] = acc[h][e];
      if (cg == 0) {
        smw[wv][h] = m[h];
        slw[wv][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < R * D; i += NT) {
    const int h = i / D, c = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, smw[w][h]);
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = smw[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(smw[w][h] - M);
      av = av + sacc[w][h][c] * wt;
      lv = lv + slw[w][h] * wt;
    }
    if (a.splits == 1) {  // the only split: its partial is the output
      a.out[((int64_t)(s / a.sh.H) * a.sh.Hq + (int64_t)(s % a.sh.H) * R + h) * D + c] = lv > 0.f ? av / lv : 0.f;
      continue;
    }
    float* pp = a.part + (((int64_t)s * a.splits + split) * R + h) * (D + 2);
    st_dev(pp + c, av);
    if (c == 0) {
      st_dev(pp + D, M);
      st_dev(pp + D + 1, lv);
    }
  }
  if (a.splits > 1 && arrive_last(a.v.sync + s, a.splits)) merge_last<D, R>(a, s);
}

// ---- Decode attention on the matrix cores (head_dim 128) ----
//
// Same split partials as k_decode, computed with v_mfma_f32_16x16x32_f16 per 32-row block of a wave:
//  * scores S[t][j] = sum_c u[t][c] q'[j][c] (+ kappa_j), u = q - qMin the unsigned code: A = the
//    block's K rows, two codes per register as fp16 subnormals (the byte of a 16-bit half is worth
//    u * 2^-24; bytes 0, 2 of a word with one mask, bytes 1, 3 after a shift), B = the folded query
//    q' = q s_K times a power of two qs (its largest magnitude near 2^14), split into fp16 hi
//    (column j) and lo (column R + j, times 2^11) halves with the same channel order;
//  * out[j][c] = sum_t (p_tj s_t) u[t][c] + sum_t p_tj z_t: A = the weights times the V scale times
//    a power of two ps (hi rows j, lo rows R + j), B = the V codes, 8 tokens of one channel per
//    lane, gathered from the rows' words with one byte permute per register; MFMA (g, b) covers the
//    channels 8n + 4g + b (n the column).  The zero term is a dot product per lane.
// ps starts at 2^12 and is lowered (the accumulators scaled exactly) when a block's largest V scale
// would take a weight operand past 2^14.
constexpr float MX_LO_UP = 2048.f, MX_LO_DOWN = 1.f / 2048.f;
constexpr float MX_CAP = 16384.f;  // largest magnitude an fp16 operand is scaled to
constexpr float MX_U = 16777216.f;  // 2^24: the value of a code's unit as an fp16 subnormal
constexpr int G = 32;              // rows per block of a wave

typedef _Float16 mxh8 __attribute__((ext_vector_type(8)));
typedef float mxf4 __attribute__((ext_vector_type(4)));
typedef uint32_t mxu4 __attribute__((ext_vector_type(4)));
typedef _Float16 mxh2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ mxf4 mx_mfma(const mxu4& a, const mxu4& b, mxf4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mxh8, a), __builtin_bit_cast(mxh8, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t mx_pk(float x, float y) {
  return __builtin_bit_cast(uint32_t, mxh2{(_Float16)x, (_Float16)y});
}
// hi = rn(x) as fp16 and lo = rn((x - hi) * 2^11): x - hi is exact in fp32
__device__ __forceinline__ float mx_lo(float x) { return (x - (float)(_Float16)x) * MX_LO_UP; }
// 2^floor(log2(MX_CAP / m)) for m > 0 (1 for m = 0): the power of two that takes m to about
// (2^13, 2^14] (the exponent bits of the quotient), at most 2^100 (a tiny fp32 query: the quotient
// would overflow, and its scores are ~0 anyway)
__device__ __forceinline__ float mx_pow2_for(float m) {
  return m > 0.f ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, fminf(MX_CAP / m, 0x1p100f)) & 0x7F800000u)
                 : 1.f;
}

template <int R, bool F32>
__global__ __launch_bounds__(NT) void k_decode_mx(DecodeArgs a) {
  constexpr int D = 128, NW = NT / 64;
  const Shape sh = a.sh;
  const int s = blockIdx.y, split = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, kg = lane >> 4;
  const int b = s / sh.H, g = s % sh.H;
  const bool b8 = sh.bits == 8;
  const uint32_t XR = b8 ? 0x80808080u : 0x08080808u;  // q - qMin of a two's-complement byte
  const uint32_t MH = b8 ? 0x00FF00FFu : 0x000F000Fu;  // bytes 0 and 2 of a word
  const uint32_t MB = b8 ? 0xFFFFFFFFu : 0x0F0F0F0Fu;  // every byte
  __shared__ float sq[R][D];           // q' = q s_K
  __shared__ float skap[R];            // kappa_j = sum_c q_jc z_c
  __shared__ float sqmax[NW];
  __shared__ alignas(16) float sp[NW][R][G + 4];  // a wave's weights of its current block [head][row]
  __shared__ float so[NW][2 * R][D];   // wave outputs (hi rows, lo rows)
  __shared__ float sm[NW][R], sl[NW][R], sz[NW][R], sps[NW];

  // ---- query fold, kappa, the query scale ----
  float qmx = 0.f;
  for (int i = tid; i < R * D; i += NT) {
    const int h = i / D, c = i % D;
    const int64_t qi = ((int64_t)b * sh.Hq + g * R + h) * D + c;
    const float qv = F32 ? static_cast<const float*>(a.q)[qi] : f16_val(static_cast<const uint16_t*>(a.q)[qi]);
    const float qf = qv * f16_val(a.v.ks[(int64_t)s * D + c]);
    sq[h][c] = qf;
    qmx = fmaxf(qmx, fabsf(qf));
    so[0][h][c] = qv * f16_val(a.v.kz[(int64_t)s * D + c]);  // q z, for kappa (so is free until the end)
  }
  for (int o = 32; o >= 1; o >>= 1) qmx = fmaxf(qmx, __shfl_xor(qmx, o));
  if (lane == 0) sqmax[wv] = qmx;
  __syncthreads();
  if (wv == 0) {  // kappa_h: two channels per lane, then a wave sum
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float k = so[0][h][lane] + so[0][h][lane + 64];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) k = k + __shfl_xor(k, o);
      if (lane == 0) skap[h] = k;
    }
  }
  float qm = sqmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) qm = fmaxf(qm, sqmax[w]);
  const float qs = mx_pow2_for(qm);
  // B operand of the scores: lane (column i16, group kg), chunk st holds channels 32 kg + 8 st + pi(e)
  // with pi = 0, 2, 1, 3, 4, 6, 5, 7 (the A register order below)
  mxu4 bq[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    uint32_t r4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c0 = 32 * kg + 8 * st + 4 * (r >> 1) + (r & 1);  // elements (c0, c0 + 2)
      float x0 = 0.f, x1 = 0.f;
      if (i16 < 2 * R) {
        const int h = i16 < R ? i16 : i16 - R;
        x0 = sq[h][c0] * qs;
        x1 = sq[h][c0 + 2] * qs;
        if (i16 >= R) {
          x0 = mx_lo(x0);
          x1 = mx_lo(x1);
        }
      }
      r4[r] = mx_pk(x0, x1);
    }
    bq[st] = mxu4{r4[0], r4[1], r4[2], r4[3]};
  }
  __syncthreads();  // kappa visible; so free again
  const float al = a.scale * LOG2E;
  const float kap = skap[i16 < R ? i16 : 0];
  const float sc_raw = MX_U / qs;

  const int nst = a.rows.nsk + a.rows.nring;
  const int j0 = split * a.rows_per_split, j1 = min(nst, j0 + a.rows_per_split);
  const int nblk = j1 > j0 ? (j1 - j0 + G - 1) / G : 0;
  float m_run = -INFINITY, l_run = 0.f, zacc = 0.f, ps = 4096.f;
  mxf4 acc[2][4];
#pragma unroll
  for (int gg = 0; gg < 2; ++gg)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) acc[gg][bb] = mxf4{0.f, 0.f, 0.f, 0.f};
  const int hm = i16 < R ? i16 : (i16 < 2 * R ? i16 - R : 0);  // head of A row i16 (weights operand)

  for (int kb = wv; kb < nblk; kb += NW) {
    const int jb = j0 + G * kb;
    // ---- loads: K rows 16 tau + i16 (channels 32 kg .. + 31); V rows 8 kg + e (channels 8 i16 .. + 7) ----
    uint4 kx[2][2];
    uint2 vx[8];
    float vsf[8], vzf[8];
    // a full block inside the sinks or inside the ring without its wrap has contiguous slots: one
    // base address per lane, rows at immediate offsets, the V metadata of 8 rows in one load each
    const int slot0 = row_slot(a.rows, jb);
    const bool contig = jb + G <= j1 && (jb + G <= a.rows.nsk ||
                                         (jb >= a.rows.nsk && slot0 + G <= a.rows.n_sink + a.rows.ring));
    if (contig) {  // uniform over the workgroup
      const int64_t ro0 = (int64_t)s * sh.cap + slot0;
      const int8_t* pk = a.v.kc + (ro0 + i16) * D + 32 * kg;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        kx[tau][0] = *reinterpret_cast<const uint4*>(pk + 16 * tau * D);
        kx[tau][1] = *reinterpret_cast<const uint4*>(pk + 16 * tau * D + 16);
      }
      const int8_t* pv = a.v.vc + (ro0 + 8 * kg) * D + 8 * i16;
#pragma unroll
      for (int e = 0; e < 8; ++e) vx[e] = *reinterpret_cast<const uint2*>(pv + e * D);
      // 8 consecutive fp16 values at an 8-element boundary (cap is a multiple of 8 rows, and so is
      // slot0 + 8 kg when slot0 is: otherwise read them one by one)
      const int64_t mo = ro0 + 8 * kg;
      if ((mo & 7) == 0) {
        const uint4 ws = *reinterpret_cast<const uint4*>(a.v.vs + mo);
        const uint4 wz = *reinterpret_cast<const uint4*>(a.v.vz + mo);
        const uint32_t sw[4] = {ws.x, ws.y, ws.z, ws.w}, zw[4] = {wz.x, wz.y, wz.z, wz.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          vsf[2 * m] = lo16(sw[m]);
          vsf[2 * m + 1] = hi16(sw[m]);
          vzf[2 * m] = lo16(zw[m]);
          vzf[2 * m + 1] = hi16(zw[m]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vsf[e] = f16_val(a.v.vs[mo + e]);
          vzf[e] = f16_val(a.v.vz[mo + e]);
        }
      }
    } else {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int j = jb + 16 * tau + i16;
        const int64_t ro = (int64_t)s * sh.cap + row_slot(a.rows, j < j1 ? j : j1 - 1);
        const uint4* p = reinterpret_cast<const uint4*>(a.v.kc + ro * D + 32 * kg);
        kx[tau][0] = p[0];
        kx[tau][1] = p[1];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = jb + 8 * kg + e;
        const int64_t ro = (int64_t)s * sh.cap + row_slot(a.rows, j < j1 ? j : j1 - 1);
        vx[e] = *reinterpret_cast<const uint2*>(a.v.vc + ro * D + 8 * i16);
        vsf[e] = j < j1 ? f16_val(a.v.vs[ro]) : 0.f;  // rows past the split: zero scale and zero
        vzf[e] = j < j1 ? f16_val(a.v.vz[ro]) : 0.f;
      }
    }
    // ---- scores ----
    mxf4 c[2] = {mxf4{0.f, 0.f, 0.f, 0.f}, mxf4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const uint4 w = kx[tau][st >> 1];
        const uint32_t x0 = ((st & 1) ? w.z : w.x) ^ XR, x1 = ((st & 1) ? w.w : w.y) ^ XR;
        const mxu4 A = mxu4{x0 & MH, (x0 >> 8) & MH, x1 & MH, (x1 >> 8) & MH};
        c[tau] = mx_mfma(A, bq[st], c[tau]);
      }
    // lane (column i16, group kg) holds rows 16 tau + 4 kg + e; the lo column of head j is j + R
    float y[2][4];
    float bm = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float hi = c[tau][e];
        const float lo = __shfl_xor(hi, R);
        const int j = jb + 16 * tau + 4 * kg + e;
        y[tau][e] = j < j1 ? __builtin_fmaf(__builtin_fmaf(lo, MX_LO_DOWN, hi), sc_raw, kap) * al : -INFINITY;
        bm = fmaxf(bm, y[tau][e]);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mnew = fmaxf(m_run, bm);
    const float f = mnew == m_run ? 1.f : (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew));
    m_run = mnew;
    float psum = 0.f;
    float pw[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[tau][e] = mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(y[tau][e] - mnew);
        psum += pw[tau][e];
      }
    l_run = l_run * f + psum;
    if (i16 < R) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        *reinterpret_cast<float4*>(&sp[wv][i16][16 * tau + 4 * kg]) =
            make_float4(pw[tau][0], pw[tau][1], pw[tau][2], pw[tau][3]);
    }
    // rescale: acc row 4 kg + e' belongs to head (4 kg + e') mod R, whose factor lane (head) holds
    const bool resc = __any(i16 < R && f != 1.f);
    if (resc) {
      zacc *= __shfl(f, hm);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float fe = __shfl(f, (4 * kg + e) % R);
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) acc[gg][bb][e] *= fe;
      }
    }
    // the weight scale: the block's largest V scale times ps stays within MX_CAP (weights <= 1)
    float smax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) smax = fmaxf(smax, vsf[e]);
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    if (smax * ps > MX_CAP) {  // uniform over the wave
      const float psn = mx_pow2_for(smax), fs = psn / ps;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) acc[gg][bb] *= fs;
      ps = psn;
    }
    __builtin_amdgcn_wave_barrier();
    // ---- A operand: row i16 = weights x V scale x ps of head hm (hi rows < R, lo rows R .. 2R - 1)
    //      over tokens 8 kg + e, the same rows as this lane's V loads ----
    const float4 pa = *reinterpret_cast<const float4*>(&sp[wv][hm][8 * kg]);
    const float4 pb = *reinterpret_cast<const float4*>(&sp[wv][hm][8 * kg + 4]);
    const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    uint32_t ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x0 = pv[2 * r] * vsf[2 * r] * ps, x1 = pv[2 * r + 1] * vsf[2 * r + 1] * ps;
      if (i16 >= R) {
        x0 = mx_lo(x0);
        x1 = mx_lo(x1);
      }
      if (i16 >= 2 * R) x0 = x1 = 0.f;
      ar[r] = mx_pk(x0, x1);
    }
    const mxu4 A = mxu4{ar[0], ar[1], ar[2], ar[3]};
    if (i16 < R) {
#pragma unroll
      for (int e = 0; e < 8; ++e) zacc = __builtin_fmaf(pv[e], vzf[e], zacc);
    }
    // ---- values: B (g, b) register r = byte b of word g of tokens 2r, 2r + 1 ----
    uint32_t xw[8][2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xw[e][0] = (vx[e].x ^ XR) & MB;
      xw[e][1] = (vx[e].y ^ XR) & MB;
    }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const uint32_t sel = (uint32_t)bb | 0x0C00u | ((uint32_t)(4 + bb) << 16) | 0x0C000000u;
        const mxu4 B = mxu4{__builtin_amdgcn_perm(xw[1][gg], xw[0][gg], sel), __builtin_amdgcn_perm(xw[3][gg], xw[2][gg], sel),
                            __builtin_amdgcn_perm(xw[5][gg], xw[4][gg], sel), __builtin_amdgcn_perm(xw[7][gg], xw[6][gg], sel)};
        acc[gg][bb] = mx_mfma(A, B, acc[gg][bb]);
      }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- wave results: l and the zero term summed over the row groups; acc rows to LDS ----
  l_run = l_run + __shfl_xor(l_run, 16);
  l_run = l_run + __shfl_xor(l_run, 32);
  zacc = zacc + __shfl_xor(zacc, 16);
  zacc = zacc + __shfl_xor(zacc, 32);
  if (lane < R) {
    sm[wv][lane] = m_run;
    sl[wv][lane] = l_run;
    sz[wv][lane] = zacc;
  }
  if (lane == 0) sps[wv] = ps;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * kg + e;
    if (m < 2 * R) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) so[wv][m][8 * i16 + 4 * gg + bb] = acc[gg][bb][e];
    }
  }
  __syncthreads();
  // ---- the workgroup's partial: waves merged in order ----
  for (int i = tid; i < R * D; i += NT) {
    const int h = i / D, c = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w][h]);
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = sm[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[w][h] - M);
      const float ov = __builtin_fmaf(__builtin_fmaf(so[w][R + h][c], MX_LO_DOWN, so[w][h][c]), MX_U / sps[w], sz[w][h]);
      av = av + ov * wt;
      lv = lv + sl[w][h] * wt;
    }
    if (a.splits == 1) {  // the only split: its partial is the output
      a.out[((int64_t)(s / a.sh.H) * a.sh.Hq + (int64_t)(s % a.sh.H) * R + h) * D + c] = lv > 0.f ? av / lv : 0.f;
      continue;
    }
    float* pp = a.part + (((int64_t)s * a.splits + split) * R + h) * (D + 2);
    st_dev(pp + c, av);
    if (c == 0) {
      st_dev(pp + D, M);
      st_dev(pp + D + 1, lv);
    }
  }
  if (a.splits > 1 && arrive_last(a.v.sync + s, a.splits)) merge_last<D, R>(a, s);
}

__global__ __launch_bounds__(NT) void k_dequant(DequantArgs a) {
  const Shape sh = a.sh;
  const int D = sh.D, CG = D / 8;
  const int s = blockIdx.y;
  const int idx = blockIdx.x * NT + threadIdx.x;
  const int row = idx / CG, cg = idx % CG;
  if (row >= a.count) return;
  const int64_t p = a.pos0 + row;
  const int sl = p < a.n_sink ? (int)p : a.n_sink + (int)((p - a.n_sink) % a.ring);
  const int64_t ro = (int64_t)s * sh.cap + sl;
  const int qmin = sh.bits == 8 ? -128 : -8;
  float u[8];
  codes8(*reinterpret_cast<const uint2*>((a.which == 0 ? a.v.kc : a.v.vc) + ro * D + 8 * cg), qmin, u);
  uint16_t* o = a.out + ((int64_t)s * a.count + row) * D + 8 * cg;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * cg + e;
    const float sc = a.which == 0 ? f16_val(a.v.ks[(int64_t)s * D + c]) : f16_val(a.v.vs[ro]);
    const float z = a.which == 0 ? f16_val(a.v.kz[(int64_t)s * D + c]) : f16_val(a.v.vz[ro]);
    o[e] = f16_bits(u[e] * sc + z);
  }
}

template <int D, bool F32>
hipError_t append_d(const AppendArgs& a, hipStream_t st) {
  const dim3 grid(a.tiles, a.sh.B * a.sh.H);
  if (a.n <= FUSE_ROWS && a.tiles <= FUSE_TILES) {  // one launch, one workgroup per stream
    hipLaunchKernelGGL((k_append_one<D, F32>), dim3(1, a.sh.B * a.sh.H), dim3(NT), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_stats<D, F32>), grid, dim3(NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_requant<D, F32>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int D, int R, bool F32>
hipError_t decode_r(const DecodeArgs& a, hipStream_t st) {
  if constexpr (D == 128) hipLaunchKernelGGL((k_decode_mx<R, F32>), dim3(a.splits, a.sh.B * a.sh.H), dim3(NT), 0, st, a);
  else hipLaunchKernelGGL((k_decode<D, R, F32>), dim3(a.splits, a.sh.B * a.sh.H), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t decode_d(const DecodeArgs& a, hipStream_t st) {
  switch (a.sh.Hq / a.sh.H) {
    case 1: return decode_r<D, 1, F32>(a, st);
    case 2: return decode_r<D, 2, F32>(a, st);
    case 4: return decode_r<D, 4, F32>(a, st);
    case 8: return decode_r<D, 8, F32>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool F32>
hipError_t decode_f(const DecodeArgs& a, hipStream_t st) {
  switch (a.sh.D) {
    case 32: return decode_d<32, F32>(a, st);
    case 64: return decode_d<64, F32>(a, st);
    case 128: return decode_d<128, F32>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool F32>
hipError_t append_f(const AppendArgs& a, hipStream_t st) {
  switch (a.sh.D) {
    case 32: return append_d<32, F32>(a, st);
    case 64: return append_d<64, F32>(a, st);
    case 128: return append_d<128, F32>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  return a.sh.in_f32 ? append_f<true>(a, st) : append_f<false>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  return a.sh.in_f32 ? decode_f<true>(a, st) : decode_f<false>(a, st);
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t st) {
  const int per = a.count * (a.sh.D / 8);
  hipLaunchKernelGGL(k_dequant, dim3((per + NT - 1) / NT, a.sh.B * a.sh.H), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvqw
