// MFMA decode attention over the packed bulk, head_dim 128 (gfx950).
//
// Writes the bulk split partials that the merge kernel of decode.hip combines
// with the fp16 rows; it replaces the generic bulk workgroups for KIVI (equal
// K/V widths 2, 4, 8) and q2k with GQA ratio 1, 2, 4 or 8.
//
// Per 32-token block and wave ("StreamingLLM + KIVI — long-context decode
// without growing the KV cache", "Affine quantisation formula": k = u*s + z per
// channel, v = u*s + z per token and 32-channel group; q2k pull-request page:
// k = level(u)*rms, v = (u - 8)*s):
//  * scores S^T[t][j] = sum_c u[t][c] * (q[j][c] s[c]) + sum_c z[c] q[j][c] on
//    the 16x16x32 f16 MFMA: codes enter as exact fp16 subnormals u * 2^-24,
//    the per-block folded query q*s is split into two fp16 halves (hi + lo)
//    so the contraction keeps ~22 bits; the zero-point term is a second MFMA
//    chain (every row of A = z).  q2k splits level(u) = c0 + c1 b0 + c2 b1 over
//    the two code bits (exact for a symmetric 4-level grid).
//  * online softmax in log2 units on 64 lanes (scores staged through LDS so
//    every lane works on live (head, token) pairs).
//  * out^T[c][j] += sum_t u[t][c] * (p[j][t] s[t][g]) on the MFMA (V codes are
//    stored in this operand order), weights split hi/lo; the zero-point term
//    sum_t p z is accumulated in fp32.
// Four waves per workgroup take interleaved blocks of the split and merge in
// LDS; the workgroup writes one partial.
#include "decode_shared.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int FD = 128;       // head_dim of this path
constexpr int NW = DNT / 64;  // waves per workgroup
constexpr float TWO24 = 16777216.0f;

__device__ __forceinline__ f4 mfma(const u4& a, const u4& b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                0, 0);
}

// Two fp32 values as fp16 hi halves (round toward zero) and the fp16 remainder.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const half2 h = __builtin_bit_cast(half2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  const float r0 = x0 - (float)h.x, r1 = x1 - (float)h.y;
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
}

// fp16 half `hi` (0: bits 0..15, 1: bits 16..31) of a word, as fp32.
__device__ __forceinline__ float h16(uint32_t w, int hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * hi)));
}

// 2^x on the transcendental unit (arguments here are <= 0; results below 2^-126 may flush to 0).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row-of-16 all-reductions with DPP lane permutations (no LDS crossbar): quad xor 1, quad xor 2,
// half-row mirror, row mirror.  Every lane of the row ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

// Operand of 8 consecutive codes (4 registers, 2 codes each as fp16 subnormals) from the
// lane's dwords d, for sub-block k (K-step of the K row chunk, or channel tile of the V chunk).
template <int B>
__device__ __forceinline__ u4 unpack(const uint32_t* d, int k) {
  u4 r;
  if constexpr (B == 2) {
    const uint32_t w = d[k >> 1] >> (8 * (k & 1));
    r.x = w & 0x00030003u;
    r.y = (w >> 2) & 0x00030003u;
    r.z = (w >> 4) & 0x00030003u;
    r.w = (w >> 6) & 0x00030003u;
  } else if constexpr (B == 4) {
    const uint32_t w = d[k];
    r.x = w & 0x000F000Fu;
    r.y = (w >> 4) & 0x000F000Fu;
    r.z = (w >> 8) & 0x000F000Fu;
    r.w = (w >> 12) & 0x000F000Fu;
  } else {
    const uint32_t w0 = d[2 * k], w1 = d[2 * k + 1];
    r.x = w0 & 0x00FF00FFu;
    r.y = (w0 >> 8) & 0x00FF00FFu;
    r.z = w1 & 0x00FF00FFu;
    r.w = (w1 >> 8) & 0x00FF00FFu;
  }
  return r;
}
// Single code bit `bit` (0 or 1) of 2-bit codes, as fp16 subnormals.
__device__ __forceinline__ u4 unpack_bit(const uint32_t* d, int k, int bit) {
  const uint32_t w = d[k >> 1] >> (8 * (k & 1) + bit);
  u4 r;
  r.x = w & 0x00010001u;
  r.y = (w >> 2) & 0x00010001u;
  r.z = (w >> 4) & 0x00010001u;
  r.w = (w >> 6) & 0x00010001u;
  return r;
}

template <int R>
struct alignas(16) FastWave {
  union {
    uint32_t qb[4][R][FD / 2];  // folded query per plane and half: [plane*2 + hl][head][channel pair]
    float o[R][FD];             // wave output for the workgroup merge
  } x;
  float ps[R][G];               // scores of the current block (log2 units), zero-point term not yet added
  float kp[R][64];              // zero-point term partials per head and compact lane
  uint32_t ab[2][4][R][4][4];   // weights x V scale: [hl][group][head][token group kg][pair of T(kg, e)]
  float f[R], zt[R][4], m[R], l[R];
};
template <int R>
struct FastSmem {
  FastWave<R> w[NW];
  int sinks[MAX_SINK];  // committed sink positions (< P) of this batch element
  int nsinks;
};

// 8 consecutive input elements (fp16 or fp32) starting at element i (a multiple of 8), as fp32.
__device__ __forceinline__ void ld8(const void* p, int64_t i, int in_f32, float* o) {
  if (in_f32) {
    const f4* q = reinterpret_cast<const f4*>(static_cast<const float*>(p) + i);
    const f4 x = q[0], y = q[1];
    o[0] = x[0], o[1] = x[1], o[2] = x[2], o[3] = x[3], o[4] = y[0], o[5] = y[1], o[6] = y[2], o[7] = y[3];
  } else {
    const u4 w = *reinterpret_cast<const u4*>(static_cast<const _Float16*>(p) + i);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = h16(ww[k], 0);
      o[2 * k + 1] = h16(ww[k], 1);
    }
  }
}
// 2 consecutive input elements starting at element i (even), as fp32.
__device__ __forceinline__ void ld2(const void* p, int64_t i, int in_f32, float* o) {
  if (in_f32) {
    const float2 x = *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
    o[0] = x.x, o[1] = x.y;
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const _Float16*>(p) + i);
    o[0] = h16(w, 0), o[1] = h16(w, 1);
  }
}

// What one lane reads from a block record: the K part is prefetched one block ahead, the V part
// is loaded when the block starts (it is needed only after the scores and the softmax).
template <int KB>
struct KPart {
  uint32_t kd[2][KB];  // K code rows i16 and 16 + i16, channels 32*kg .. 32*kg + 31
  uint32_t ks, kz;     // K scale (q2k: rms) and zero of channels 2*lane, 2*lane + 1
};
template <int VB>
struct VPart {
  uint32_t vd[2 * VB];  // V code chunk `lane`
  u4 vs, vz;            // V scale and zero of tokens 2*tp, 2*tp + 1, groups 0..3
};

template <bool Q2K, int KB>
__device__ __forceinline__ void load_k(KPart<KB>& d, const uint8_t* rec, const LayerView& lv, int lane) {
  const int i16 = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const uint8_t* src = rec + lv.k_codes + (16 * tau + i16) * (FD * KB / 8) + kg * 4 * KB;
    if constexpr (KB == 2) {
      const u2 x = *reinterpret_cast<const u2*>(src);
      d.kd[tau][0] = x.x, d.kd[tau][1] = x.y;
    } else {
#pragma unroll
      for (int k = 0; k < KB / 4; ++k) {
        const u4 x = reinterpret_cast<const u4*>(src)[k];
        d.kd[tau][4 * k] = x.x, d.kd[tau][4 * k + 1] = x.y, d.kd[tau][4 * k + 2] = x.z, d.kd[tau][4 * k + 3] = x.w;
      }
    }
  }
  d.ks = reinterpret_cast<const uint32_t*>(rec + lv.k_meta)[lane];
  d.kz = Q2K ? 0u : reinterpret_cast<const uint32_t*>(rec + lv.k_meta + 2 * FD)[lane];
}

template <bool Q2K, int VB>
__device__ __forceinline__ void load_v(VPart<VB>& d, const uint8_t* rec, const LayerView& lv, int lane) {
  const u4* src = reinterpret_cast<const u4*>(rec + lv.v_codes + lane * 8 * VB);
#pragma unroll
  for (int k = 0; k < VB / 2; ++k) {
    const u4 x = src[k];
    d.vd[4 * k] = x.x, d.vd[4 * k + 1] = x.y, d.vd[4 * k + 2] = x.z, d.vd[4 * k + 3] = x.w;
  }
  d.vs = *reinterpret_cast<const u4*>(rec + lv.v_meta + 16 * (lane & 15));
  if constexpr (!Q2K) d.vz = *reinterpret_cast<const u4*>(rec + lv.v_meta + 2 * G * (FD / 32) + 16 * (lane & 15));
  else d.vz = u4{0, 0, 0, 0};
}

template <int FMT, int KB, int VB, int R>
__device__ void fast_partial(const DecodeArgs& a, FastSmem<R>& F) {
  constexpr bool Q2K = FMT == KVQ_FMT_Q2K;
  constexpr int NPL = R <= 4 ? 1 : R / 4;  // (head, token pair) slots per lane in the compact phase
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, kg = lane >> 4;
  const int sigma = blockIdx.x, s = blockIdx.y, b = s / sh.Hkv, g = s % sh.Hkv;
  const int jj = i16 < R ? i16 : R - 1;  // head of this lane in MFMA B/C layouts (padding lanes mirror R-1)
  FastWave<R>& W = F.w[wv];

  const float qscale = a.scale * LOG2E;
  const float c0 = Q2K ? lv.tables->q2k_lvl[0] : 1.f;
  const float c1 = Q2K ? lv.tables->q2k_lvl[1] - lv.tables->q2k_lvl[0] : 1.f;
  const float c2 = Q2K ? lv.tables->q2k_lvl[2] - lv.tables->q2k_lvl[0] : 1.f;
  const int64_t qrow = ((int64_t)b * sh.Hq + (int64_t)g * R) * FD;

  stage_sinks(a, b, F.sinks, nullptr, &F.nsinks);
  // compact query: lane holds channels 2*lane, 2*lane+1 of every head (scaled to log2 units)
  float qc[R][2];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    ld2(a.q, qrow + j * FD + 2 * lane, sh.in_f32, qc[j]);
    qc[j][0] *= qscale;
    qc[j][1] *= qscale;
  }
  __syncthreads();

  float m_[NPL], l_[NPL], zacc[NPL][4];
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    m_[p] = -INFINITY;
    l_[p] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) zacc[p][q] = 0.f;
  }
  f4 acc[8];
#pragma unroll
  for (int mu = 0; mu < 8; ++mu) acc[mu] = f4{0.f, 0.f, 0.f, 0.f};

  const int first = sigma * a.blocks_per_split;
  const int lastb = min(a.nblk, first + a.blocks_per_split);
  const int nsink = F.nsinks;
  const int tp = i16;  // compact token pair
  auto rec_of = [&](int bi) {
    const int64_t blk = a.blk_first + bi;
    return lv.bulk + ((int64_t)s * lv.cap_b + blk % lv.cap_b) * lv.rec;
  };

  KPart<KB> kc, kn;
  if (first + wv < lastb) load_k<Q2K>(kc, rec_of(first + wv), lv, lane);
  for (int bi = first + wv; bi < lastb; bi += NW) {
    const uint8_t* rec = rec_of(bi);
    VPart<VB> vp;
    load_v<Q2K>(vp, rec, lv, lane);
    if (bi + NW < lastb) load_k<Q2K>(kn, rec_of(bi + NW), lv, lane);  // next block's K, in flight meanwhile
    const int64_t blk = a.blk_first + bi;

    // ---- fold the per-channel K scale into the query; zero-point partials (compact lanes) ----
    {
      const float s0 = h16(kc.ks, 0), s1 = h16(kc.ks, 1);
      const float z0 = Q2K ? c0 * s0 : h16(kc.kz, 0), z1 = Q2K ? c0 * s1 : h16(kc.kz, 1);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float x0 = qc[j][0] * s0, x1 = qc[j][1] * s1;
        uint32_t h, l;
        split2(x0 * c1, x1 * c1, h, l);
        W.x.qb[0][j][lane] = h;
        W.x.qb[1][j][lane] = l;
        if constexpr (Q2K) {
          split2(x0 * c2, x1 * c2, h, l);
          W.x.qb[2][j][lane] = h;
          W.x.qb[3][j][lane] = l;
        }
        W.kp[j][lane] = qc[j][0] * z0 + qc[j][1] * z1;
      }
    }
    // ---- scores (hi and lo chains accumulate separately) ----
    f4 sh_[2], sl_[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) sh_[tau] = sl_[tau] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u4 bh = *reinterpret_cast<const u4*>(&W.x.qb[0][jj][16 * kg + 4 * st]);
      const u4 bl = *reinterpret_cast<const u4*>(&W.x.qb[1][jj][16 * kg + 4 * st]);
      if constexpr (Q2K) {
        const u4 bh2 = *reinterpret_cast<const u4*>(&W.x.qb[2][jj][16 * kg + 4 * st]);
        const u4 bl2 = *reinterpret_cast<const u4*>(&W.x.qb[3][jj][16 * kg + 4 * st]);
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const u4 a0 = unpack_bit(kc.kd[tau], st, 0), a1 = unpack_bit(kc.kd[tau], st, 1);
          sh_[tau] = mfma(a0, bh, sh_[tau]);
          sl_[tau] = mfma(a0, bl, sl_[tau]);
          sh_[tau] = mfma(a1, bh2, sh_[tau]);
          sl_[tau] = mfma(a1, bl2, sl_[tau]);
        }
      } else {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const u4 a0 = unpack<KB>(kc.kd[tau], st);
          sh_[tau] = mfma(a0, bh, sh_[tau]);
          sl_[tau] = mfma(a0, bl, sl_[tau]);
        }
      }
    }
    float sc[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[tau][i] = (sh_[tau][i] + sl_[tau][i]) * TWO24;
    // mask tokens outside [bulk_lo, bulk_hi) and committed sinks (only blocks that need it)
    const int p0 = (int)(blk * G), blo = (int)a.bulk_lo, bhi = (int)a.bulk_hi;  // positions fit in int32
    bool full = p0 >= blo && p0 + G <= bhi;
    for (int q = 0; q < nsink && full; ++q) full = !(F.sinks[q] >= p0 && F.sinks[q] < p0 + G);
    if (!full) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = p0 + 16 * tau + 4 * kg + i;
          bool ok = p >= blo && p < bhi;
          for (int q = 0; q < nsink; ++q) ok = ok && F.sinks[q] != p;
          if (!ok) sc[tau][i] = -INFINITY;
        }
    }
    if (i16 < R) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        *reinterpret_cast<f4*>(&W.ps[i16][16 * tau + 4 * kg]) = f4{sc[tau][0], sc[tau][1], sc[tau][2], sc[tau][3]};
    }
    // ---- compact online softmax and weights x V scale ----
    bool resc = false;
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const int jr = kg + 4 * p;
      const bool live = (R % 4 == 0) || jr < R;
      const int j = live ? jr : R - 1;
      const f4 kq = *reinterpret_cast<const f4*>(&W.kp[j][4 * tp]);
      const float kap = row_sum16((kq[0] + kq[1]) + (kq[2] + kq[3]));
      float2 sv = *reinterpret_cast<const float2*>(&W.ps[j][2 * tp]);
      sv.x += kap;
      sv.y += kap;
      const float mx = row_max16(fmaxf(sv.x, sv.y));
      const float mnew = fmaxf(m_[p], mx);
      float f = 1.f, e0 = 0.f, e1 = 0.f;
      if (mnew != -INFINITY) {
        f = m_[p] == -INFINITY ? 0.f : (mnew == m_[p] ? 1.f : ex2(m_[p] - mnew));
        e0 = sv.x == -INFINITY ? 0.f : ex2(sv.x - mnew);
        e1 = sv.y == -INFINITY ? 0.f : ex2(sv.y - mnew);
      }
      const float sum = row_sum16(e0 + e1);
      if (live) {
        l_[p] = l_[p] * f + sum;
        m_[p] = mnew;
        if (tp == 0) W.f[j] = f;
      }
      resc = resc || (live && f != 1.f);
      // tokens 2tp, 2tp+1: position (kg_t, e) in the V operand order
      const int t0 = 2 * tp, kgt = (t0 & 15) >> 2, et = ((t0 >> 4) << 2) | (t0 & 3);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // vs / vz hold fp16 [t0: g0 g1 | g2 g3][t0+1: g0 g1 | g2 g3]
        const float s_t0 = h16(q < 2 ? vp.vs.x : vp.vs.y, q & 1), s_t1 = h16(q < 2 ? vp.vs.z : vp.vs.w, q & 1);
        const float a0 = e0 * s_t0, a1 = e1 * s_t1;
        uint32_t h, l;
        split2(a0, a1, h, l);
        if (live) {
          W.ab[0][q][j][kgt][et >> 1] = h;
          W.ab[1][q][j][kgt][et >> 1] = l;
          float zt;
          if constexpr (Q2K) zt = -8.f * (a0 + a1);
          else {
            const float z_t0 = h16(q < 2 ? vp.vz.x : vp.vz.y, q & 1);
            const float z_t1 = h16(q < 2 ? vp.vz.z : vp.vz.w, q & 1);
            zt = e0 * z_t0 + e1 * z_t1;
          }
          zacc[p][q] = zacc[p][q] * f + zt;
        }
      }
    }
    // ---- values ----
    if (__any(resc)) {
      const float fj = W.f[jj];
#pragma unroll
      for (int mu = 0; mu < 8; ++mu) acc[mu] *= fj;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u4 bh = *reinterpret_cast<const u4*>(&W.ab[0][q][jj][kg][0]);
      const u4 bl = *reinterpret_cast<const u4*>(&W.ab[1][q][jj][kg][0]);
#pragma unroll
      for (int mu = 2 * q; mu < 2 * q + 2; ++mu) {
        const u4 av = unpack<VB>(vp.vd, mu);
        acc[mu] = mfma(av, bh, acc[mu]);
        acc[mu] = mfma(av, bl, acc[mu]);
      }
    }
    kc = kn;
  }

  // ---- wave results: zero-point term, output, (m, l) ----
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int jr = kg + 4 * p;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float z = row_sum16(zacc[p][q]);
      if (jr < R && tp == 0) W.zt[jr][q] = z;
    }
    if (jr < R && tp == 0) {
      W.m[jr] = m_[p];
      W.l[jr] = l_[p];
    }
  }
  if (i16 < R) {
#pragma unroll
    for (int mu = 0; mu < 8; ++mu) {
      const float zt = W.zt[i16][mu >> 1];
      const int c = 16 * mu + 4 * kg;
      *reinterpret_cast<f4*>(&W.x.o[i16][c]) =
          f4{acc[mu][0] * TWO24 + zt, acc[mu][1] * TWO24 + zt, acc[mu][2] * TWO24 + zt, acc[mu][3] * TWO24 + zt};
    }
  }
  __syncthreads();
  // ---- merge the waves into the workgroup partial ----
  float* part = a.ws + ((int64_t)s * a.nparts + sigma) * R * (FD + 2);
  for (int idx = tid; idx < R * FD; idx += DNT) {
    const int j = idx / FD, c = idx % FD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, F.w[w].m[j]);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (F.w[w].m[j] != -INFINITY) v += F.w[w].x.o[j][c] * exp2f(F.w[w].m[j] - M);
    part[j * (FD + 2) + 2 + c] = v;
  }
  if (tid < R) {
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, F.w[w].m[tid]);
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (F.w[w].m[tid] != -INFINITY) L += F.w[w].l[tid] * exp2f(F.w[w].m[tid] - M);
    part[tid * (FD + 2)] = M;
    part[tid * (FD + 2) + 1] = L;
  }
}

template <int FMT, int KB, int VB, int R>
__global__ __launch_bounds__(DNT) void k_decode_fast(DecodeArgs a) {
  __shared__ FastSmem<R> S;
  fast_partial<FMT, KB, VB, R>(a, S);
}

template <int FMT, int KB, int VB>
hipError_t launch_r(const DecodeArgs& a, hipStream_t st) {
  const int r = a.sh.Hq / a.sh.Hkv;
  dim3 grid(a.splits, a.sh.B * a.sh.Hkv);  // bulk splits only: the merge kernel reads the fp16 rows
  switch (r) {
    case 1: hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 1>), grid, dim3(DNT), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 2>), grid, dim3(DNT), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 4>), grid, dim3(DNT), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 8>), grid, dim3(DNT), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Launches the MFMA kernel; the host only sets DecodeArgs::fast for shapes it covers.
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  if (sh.D != FD || a.splits == 0) return hipErrorInvalidValue;
  if (sh.fmt == KVQ_FMT_Q2K) return launch_r<KVQ_FMT_Q2K, 2, 4>(a, st);
  if (sh.fmt == KVQ_FMT_KIVI && sh.kb == sh.vb) {
    if (sh.kb == 2) return launch_r<KVQ_FMT_KIVI, 2, 2>(a, st);
    if (sh.kb == 4) return launch_r<KVQ_FMT_KIVI, 4, 4>(a, st);
    if (sh.kb == 8) return launch_r<KVQ_FMT_KIVI, 8, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
