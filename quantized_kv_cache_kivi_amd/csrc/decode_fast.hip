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
//  * scores S^T[t][j] = sum_c u[t][c] * (q[j][c] s[c]) + sum_c z[c] q[j][c].
//    The first sum runs on the 16x16x32 f16 MFMA: codes enter as exact fp16
//    subnormals, masked in place inside their packed word (a code at bit
//    position p of a 16-bit half is worth u * 2^(p-24); the query side carries
//    the compensating power of two), and the per-block folded query q*s is
//    split into fp16 hi + lo halves that occupy separate MFMA columns (head j
//    hi in column j, lo in column R + j), so one MFMA keeps ~22 bits.  q2k
//    splits level(u) = c0 + c1 b0 + c2 b1 over the two code bits (exact for a
//    symmetric 4-level grid).  The zero-point sum is a 64-lane reduction.
//  * online softmax in log2 units on 64 lanes (scores staged through LDS so
//    every lane works on live (head, token) pairs).
//  * out^T[c][j] += sum_t u[t][c] * (p[j][t] s[t][g]) on the MFMA (V codes are
//    stored in this operand order), weights split hi/lo into columns as above;
//    the zero-point term sum_t p z is accumulated in fp32.
// Four waves per workgroup take interleaved blocks of the split and merge in
// LDS; the workgroup writes one partial.
//
// Rounding: only this file's device code may contract a*b+c into one FMA; the
// result is within the same error budget (every product here feeds a sum).
// Range: the fp16 halves hold q*s*scale*log2(e) times at most 2^7 and V scale
// times at most 2^6; inputs whose products overflow fp16 there are outside the
// domain of this path.
#include "decode_shared.h"

#pragma clang fp contract(fast)

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int FD = 128;       // head_dim of this path
constexpr int NW = DNT / 64;  // waves per workgroup

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

// A operand of 8 consecutive codes (4 registers, 2 codes each as fp16 subnormals) from the lane's
// dwords d, for sub-block k (K step of the K row chunk, or channel tile of the V chunk).  Codes are
// masked where they sit when their bits lie below bit 10 of each 16-bit half; element pair r then
// carries the factor 2^code_pos<B>(r), which the B operand undoes.
template <int B>
__device__ __forceinline__ u4 codes_a(const uint32_t* d, int k) {
  u4 r;
  if constexpr (B == 2) {
    const uint32_t w = (k & 1) ? d[k >> 1] >> 8 : d[k >> 1];
    r.x = w & 0x00030003u;
    r.y = w & 0x000C000Cu;
    r.z = w & 0x00300030u;
    r.w = w & 0x00C000C0u;
  } else if constexpr (B == 4) {
    const uint32_t w = d[k], w8 = w >> 8;
    r.x = w & 0x000F000Fu;
    r.y = w & 0x00F000F0u;
    r.z = w8 & 0x000F000Fu;
    r.w = w8 & 0x00F000F0u;
  } else {
    const uint32_t w0 = d[2 * k], w1 = d[2 * k + 1];
    r.x = w0 & 0x00FF00FFu;
    r.y = __builtin_amdgcn_perm(w0, w0, 0x0C030C01u);  // bytes 1 and 3 moved to bytes 0 and 2
    r.z = w1 & 0x00FF00FFu;
    r.w = __builtin_amdgcn_perm(w1, w1, 0x0C030C01u);
  }
  return r;
}
// Bit position (within its 16-bit half) of the codes of element pair r in codes_a<B>.
template <int B>
constexpr int code_pos(int r) {
  return B == 2 ? 2 * r : B == 4 ? 4 * (r & 1) : 0;
}
// Single code bit `bit` (0 or 1) of 2-bit codes in place: element pair r sits at 2r + bit.
template <int BIT>
__device__ __forceinline__ u4 plane_a(const uint32_t* d, int k) {
  const uint32_t w = (k & 1) ? d[k >> 1] >> 8 : d[k >> 1];
  u4 r;
  r.x = w & (0x00010001u << BIT);
  r.y = w & (0x00040004u << BIT);
  r.z = w & (0x00100010u << BIT);
  r.w = w & (0x00400040u << BIT);
  return r;
}

template <int R, int NPLANE>
struct alignas(16) FastWave {
  static constexpr int NC = 2 * R;  // MFMA columns in use: hi halves of heads 0..R-1, then lo halves
  // Rows are padded by 16 bytes so that the 16 column lanes of an MFMA operand read (and the
  // 16-byte score stores) fall on distinct LDS banks.
  union {
    uint32_t qb[NPLANE][NC][FD / 2 + 4];  // folded query: [code plane][column][channel pair]
    float o[R][FD];                       // wave output for the workgroup merge
  } x;
  float ps[NC][G + 4];                    // raw score columns of the current block
  float kp[R][64 + 4];                    // zero-point term partials per head and compact lane
  uint32_t ab[4][NC][4 * 4 + 4];          // weights x V scale: [group][column][4 * token group + pair]
  float f[R], zt[R][4], m[R], l[R];
};
template <int R, int NPLANE>
struct FastSmem {
  FastWave<R, NPLANE> w[NW];
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

// What one lane reads from a block record (K and V parts of the next block are in flight while
// the current one is computed).
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

// One 32-token block of the wave: scores, online softmax, value accumulation.
template <int FMT, int KB, int VB, int R>
struct BlockState {
  static constexpr bool Q2K = FMT == KVQ_FMT_Q2K;
  static constexpr int NPLANE = Q2K ? 2 : 1;
  static constexpr int NPL = R <= 4 ? 1 : R / 4;  // (head, token pair) slots per lane in the compact phase
  static constexpr int PK = Q2K ? 7 : code_pos<KB>(3);  // largest in-place K code position
  static constexpr int PV = code_pos<VB>(3);            // largest in-place V code position
  float qc[R][2];        // query channels 2*lane, 2*lane + 1 of every head, log2 units
  float fa, fb;          // K fold factors of this lane (plane 0 / plane 1, q2k levels included)
  float fv;              // V weight factor of this lane's token pair
  float m_[NPL], l_[NPL], zacc[NPL][4];
  f4 acc[8];
};

template <int FMT, int KB, int VB, int R>
__device__ __forceinline__ void block_step(BlockState<FMT, KB, VB, R>& S,
                                           FastWave<R, BlockState<FMT, KB, VB, R>::NPLANE>& W,
                                           const int* sinks, const KPart<KB>& kc, const VPart<VB>& vp, int blk,
                                           int blo, int bhi, int sblk, int nsink, float c0, int lane) {
  using St = BlockState<FMT, KB, VB, R>;
  constexpr bool Q2K = St::Q2K;
  constexpr int NPL = St::NPL, NC = 2 * R;
  constexpr float SK = (float)(1u << (24 - St::PK));
  const int i16 = lane & 15, kg = lane >> 4, tp = i16;
  // MFMA column of this lane; padding lanes repeat the last column, so their score stores repeat
  // its values
  const int col = i16 < NC ? i16 : NC - 1;

  // ---- fold the per-channel K scale into the query (hi -> column j, lo -> column R + j) ----
  {
    const float s0 = h16(kc.ks, 0), s1 = h16(kc.ks, 1);
    const float z0 = Q2K ? c0 * s0 : h16(kc.kz, 0), z1 = Q2K ? c0 * s1 : h16(kc.kz, 1);
    const float sa0 = s0 * S.fa, sa1 = s1 * S.fa;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      uint32_t h, l;
      split2(S.qc[j][0] * sa0, S.qc[j][1] * sa1, h, l);
      W.x.qb[0][j][lane] = h;
      W.x.qb[0][R + j][lane] = l;
      if constexpr (Q2K) {
        split2(S.qc[j][0] * (s0 * S.fb), S.qc[j][1] * (s1 * S.fb), h, l);
        W.x.qb[St::NPLANE - 1][j][lane] = h;
        W.x.qb[St::NPLANE - 1][R + j][lane] = l;
      }
      W.kp[j][lane] = S.qc[j][0] * z0 + S.qc[j][1] * z1;
    }
  }
  // ---- scores: raw MFMA columns to LDS ----
  f4 c_[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const u4 b0 = *reinterpret_cast<const u4*>(&W.x.qb[0][col][16 * kg + 4 * st]);
    if constexpr (Q2K) {
      const u4 b1 = *reinterpret_cast<const u4*>(&W.x.qb[St::NPLANE - 1][col][16 * kg + 4 * st]);
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        c_[tau] = mfma(plane_a<0>(kc.kd[tau], st), b0, c_[tau]);
        c_[tau] = mfma(plane_a<1>(kc.kd[tau], st), b1, c_[tau]);
      }
    } else {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) c_[tau] = mfma(codes_a<KB>(kc.kd[tau], st), b0, c_[tau]);
    }
  }
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) *reinterpret_cast<f4*>(&W.ps[col][16 * tau + 4 * kg]) = c_[tau];

  // ---- compact online softmax and weights x V scale ----
  // tokens 2tp, 2tp+1 of the block; masked if outside [bulk_lo, bulk_hi) or a committed sink
  const int p0 = blk * G;
  bool ok0 = true, ok1 = true;
  if (p0 < blo || p0 + G > bhi || __any(sblk == blk)) {
    const int pa = p0 + 2 * tp;
    ok0 = pa >= blo && pa < bhi;
    ok1 = pa + 1 >= blo && pa + 1 < bhi;
    for (int q = 0; q < nsink; ++q) {
      ok0 = ok0 && sinks[q] != pa;
      ok1 = ok1 && sinks[q] != pa + 1;
    }
  }
  const int t0 = 2 * tp, kgt = (t0 & 15) >> 2, et = ((t0 >> 4) << 2) | (t0 & 3);  // V operand position
  bool resc = false;
  float fp_[NPL], zb[NPL][4];  // rescale factor and this block's zero-point terms per slot
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int jr = kg + 4 * p;
    const int j = jr < R ? jr : R - 1;  // lanes past the last head repeat it (identical stores)
    const f4 kq = *reinterpret_cast<const f4*>(&W.kp[j][4 * tp]);
    const float kap = row_sum16((kq[0] + kq[1]) + (kq[2] + kq[3]));
    const float2 hi = *reinterpret_cast<const float2*>(&W.ps[j][2 * tp]);
    const float2 lo = *reinterpret_cast<const float2*>(&W.ps[R + j][2 * tp]);
    const float sv0 = ok0 ? (hi.x + lo.x) * SK + kap : -INFINITY;
    const float sv1 = ok1 ? (hi.y + lo.y) * SK + kap : -INFINITY;
    const float mx = row_max16(fmaxf(sv0, sv1));
    const float mold = S.m_[p];
    const float mnew = fmaxf(mold, mx);
    float f = 1.f, e0 = 0.f, e1 = 0.f;
    if (mnew != -INFINITY) {
      f = mold == -INFINITY ? 0.f : (mnew == mold ? 1.f : ex2(mold - mnew));
      e0 = sv0 == -INFINITY ? 0.f : ex2(sv0 - mnew);
      e1 = sv1 == -INFINITY ? 0.f : ex2(sv1 - mnew);
    }
    const float sum = row_sum16(e0 + e1);
    S.l_[p] = S.l_[p] * f + sum;
    S.m_[p] = mnew;
    if (tp == 0) W.f[j] = f;
    fp_[p] = f;
    resc = resc || f != 1.f;
    const float e0v = e0 * S.fv, e1v = e1 * S.fv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // vs / vz hold fp16 [t0: g0 g1 | g2 g3][t0+1: g0 g1 | g2 g3]
      const float s_t0 = h16(q < 2 ? vp.vs.x : vp.vs.y, q & 1), s_t1 = h16(q < 2 ? vp.vs.z : vp.vs.w, q & 1);
      uint32_t h, l;
      split2(e0v * s_t0, e1v * s_t1, h, l);
      W.ab[q][j][4 * kgt + (et >> 1)] = h;
      W.ab[q][R + j][4 * kgt + (et >> 1)] = l;
      if constexpr (Q2K) {
        zb[p][q] = -8.f * (e0 * s_t0 + e1 * s_t1);
      } else {
        const float z_t0 = h16(q < 2 ? vp.vz.x : vp.vz.y, q & 1);
        const float z_t1 = h16(q < 2 ? vp.vz.z : vp.vz.w, q & 1);
        zb[p][q] = e0 * z_t0 + e1 * z_t1;
      }
    }
  }
  // ---- values (rare: rescale the running sums to a new maximum first) ----
  if (__any(resc)) {
    const float fc = W.f[i16 & (R - 1)];
#pragma unroll
    for (int mu = 0; mu < 8; ++mu) S.acc[mu] *= fc;
#pragma unroll
    for (int p = 0; p < NPL; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) S.zacc[p][q] *= fp_[p];
  }
#pragma unroll
  for (int p = 0; p < NPL; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) S.zacc[p][q] += zb[p][q];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u4 bq = *reinterpret_cast<const u4*>(&W.ab[q][col][4 * kg]);
#pragma unroll
    for (int mu = 2 * q; mu < 2 * q + 2; ++mu) S.acc[mu] = mfma(codes_a<VB>(vp.vd, mu), bq, S.acc[mu]);
  }
}

template <int FMT, int KB, int VB, int R>
__device__ void fast_partial(const DecodeArgs& a, FastSmem<R, BlockState<FMT, KB, VB, R>::NPLANE>& F) {
  using State = BlockState<FMT, KB, VB, R>;
  constexpr bool Q2K = State::Q2K;
  constexpr int NPL = State::NPL;
  constexpr float SV = (float)(1u << (24 - State::PV));
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform: keeps the loop scalar)
  const int i16 = lane & 15, kg = lane >> 4;
  const int sigma = blockIdx.x, s = blockIdx.y, b = s / sh.Hkv, g = s % sh.Hkv;
  auto& W = F.w[wv];

  const float qscale = a.scale * LOG2E;
  const float c0 = Q2K ? lv.tables->q2k_lvl[0] : 1.f;
  const float c1 = Q2K ? lv.tables->q2k_lvl[1] - lv.tables->q2k_lvl[0] : 1.f;
  const float c2 = Q2K ? lv.tables->q2k_lvl[2] - lv.tables->q2k_lvl[0] : 1.f;
  const int64_t qrow = ((int64_t)b * sh.Hq + (int64_t)g * R) * FD;

  stage_sinks(a, b, F.sinks, nullptr, &F.nsinks);
  State S;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    ld2(a.q, qrow + j * FD + 2 * lane, sh.in_f32, S.qc[j]);
    S.qc[j][0] *= qscale;
    S.qc[j][1] *= qscale;
  }
  {
    // channels 2*lane, 2*lane+1 are element pair (lane & 3) of their K step; the V weights of tokens
    // 2*i16, 2*i16+1 are element pair (et >> 1) of their token group
    const int rk = lane & 3;
    if constexpr (Q2K) {
      S.fa = ldexpf(c1, State::PK - 2 * rk);
      S.fb = ldexpf(c2, State::PK - 2 * rk - 1);
    } else {
      S.fa = ldexpf(1.f, State::PK - code_pos<KB>(rk));
      S.fb = 0.f;
    }
    const int t0 = 2 * i16, et = ((t0 >> 4) << 2) | (t0 & 3);
    S.fv = ldexpf(1.f, State::PV - code_pos<VB>(et >> 1));
  }
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    S.m_[p] = -INFINITY;
    S.l_[p] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) S.zacc[p][q] = 0.f;
  }
#pragma unroll
  for (int mu = 0; mu < 8; ++mu) S.acc[mu] = f4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const int nsink = __builtin_amdgcn_readfirstlane(F.nsinks);
  const int sblk = lane < nsink ? F.sinks[lane] / G : -1;  // block of sink `lane`
  const int first = sigma * a.blocks_per_split;
  const int lastb = min(a.nblk, first + a.blocks_per_split);
  const int blo = (int)a.bulk_lo, bhi = (int)a.bulk_hi;  // positions fit in int32 (checked on the host)
  const int blkf = (int)a.blk_first;
  const int slot0 = (int)(a.blk_first % lv.cap_b);  // ring slot of bulk block index 0
  const uint8_t* sbase = lv.bulk + (int64_t)s * lv.cap_b * lv.rec;
  auto rec_of = [&](int bi) {
    int sl = slot0 + bi;
    if (sl >= lv.cap_b) sl -= lv.cap_b;
    return sbase + (int64_t)sl * lv.rec;
  };

  // ping-pong buffers: the next block of this wave is in flight while the current one is computed
  KPart<KB> k0, k1;
  VPart<VB> v0, v1;
  int bi = first + wv;
  if (bi < lastb) {
    load_k<Q2K>(k0, rec_of(bi), lv, lane);
    load_v<Q2K>(v0, rec_of(bi), lv, lane);
  }
  while (bi < lastb) {
    if (bi + NW < lastb) {
      load_k<Q2K>(k1, rec_of(bi + NW), lv, lane);
      load_v<Q2K>(v1, rec_of(bi + NW), lv, lane);
    }
    block_step(S, W, F.sinks, k0, v0, blkf + bi, blo, bhi, sblk, nsink, c0, lane);
    bi += NW;
    if (bi >= lastb) break;
    if (bi + NW < lastb) {
      load_k<Q2K>(k0, rec_of(bi + NW), lv, lane);
      load_v<Q2K>(v0, rec_of(bi + NW), lv, lane);
    }
    block_step(S, W, F.sinks, k1, v1, blkf + bi, blo, bhi, sblk, nsink, c0, lane);
    bi += NW;
  }

  // ---- wave results: zero-point term, output (column j plus column R + j), (m, l) ----
  const int tp = i16;
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int jr = kg + 4 * p;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float z = row_sum16(S.zacc[p][q]);
      if (jr < R && tp == 0) W.zt[jr][q] = z;
    }
    if (jr < R && tp == 0) {
      W.m[jr] = S.m_[p];
      W.l[jr] = S.l_[p];
    }
  }
#pragma unroll
  for (int mu = 0; mu < 8; ++mu) {
    f4 lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = __shfl(S.acc[mu][i], lane + R);
    if (i16 < R) {
      const float zt = W.zt[i16][mu >> 1];
      const f4 v = S.acc[mu] + lo;
      *reinterpret_cast<f4*>(&W.x.o[i16][16 * mu + 4 * kg]) =
          f4{v[0] * SV + zt, v[1] * SV + zt, v[2] * SV + zt, v[3] * SV + zt};
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

// Waves per SIMD the register allocation targets: 3 where the kernel fits 168 VGPRs without spilling
// (2-bit K codes, at most 4 heads per KV head), else 2.
template <int FMT, int KB, int VB, int R>
constexpr int waves_target() {
  return (R <= 4 && KB == 2) ? 3 : 2;
}

template <int FMT, int KB, int VB, int R>
__global__ __launch_bounds__(DNT) __attribute__((amdgpu_waves_per_eu(waves_target<FMT, KB, VB, R>())))
void k_decode_fast(DecodeArgs a) {
  __shared__ FastSmem<R, BlockState<FMT, KB, VB, R>::NPLANE> S;
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

template <int FMT, int KB, int VB>
int slots_r(int r, int per_cu) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (r) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 1>, DNT, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 2>, DNT, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 4>, DNT, 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 8>, DNT, 0); break;
    default: break;
  }
  return e == hipSuccess ? nb * per_cu : 0;
}

}  // namespace

int fast_resident_slots(const Shape& sh) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess)
    return 0;
  const int r = sh.Hq / sh.Hkv;
  if (sh.D != FD) return 0;
  if (sh.fmt == KVQ_FMT_Q2K) return slots_r<KVQ_FMT_Q2K, 2, 4>(r, cus);
  if (sh.fmt == KVQ_FMT_KIVI && sh.kb == sh.vb) {
    if (sh.kb == 2) return slots_r<KVQ_FMT_KIVI, 2, 2>(r, cus);
    if (sh.kb == 4) return slots_r<KVQ_FMT_KIVI, 4, 4>(r, cus);
    if (sh.kb == 8) return slots_r<KVQ_FMT_KIVI, 8, 8>(r, cus);
  }
  return 0;
}

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
