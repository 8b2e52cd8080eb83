// MFMA decode attention, head_dim 128, fp16 query (gfx950).
//
// One launch of k_decode_fast does a whole decode call: workgroup (stream
// blockIdx.x, part blockIdx.y) streams the packed bulk of split blockIdx.y of
// the stream when blockIdx.y < splits, else it scores 64 of the stream's fp16
// rows (window rows minus committed sinks, then the sink pool), and writes one
// online-softmax partial.  The partials are stored with device-scope atomic
// stores (they reach the point of coherence of every XCD), the workgroup waits
// for its stores, then counts itself in the stream's arrival counter; the
// workgroup that arrives last merges the stream's partials in fixed order
// (device-scope loads) and writes the output, so no second launch is needed.
// The counter is reset by that workgroup (zero between calls).
//
// Bulk, per 32-token block and wave ("StreamingLLM + KIVI — long-context decode
// without growing the KV cache", "Affine quantisation formula": k = u*s + z per
// channel, v = u*s + z per token and 32-channel group; q2k pull-request page,
// "Summary": k = level(u)*rms, v = (u - 8)*s):
//  * scores: S[t][j] = sum_c u[t][c] * (q[j][c] s[c]) + sum_c z[c] q[j][c].
//    The first sum runs on the 16x16x32 f16 MFMA.  Codes enter as exact fp16
//    subnormals masked in place inside their packed word (a code at bit p of a
//    16-bit half is worth u * 2^(p-24)); the query side is the exact product
//    q*s of two fp16 pairs split into an fp16 hi half (column j) and lo half
//    (column R + j) with one packed multiply and one packed fma, both then
//    scaled by 2^-p, so the MFMA keeps ~22 bits.  q2k splits level(u) = c0 + c1 b0 + c2 b1 over the
//    two code bits (exact for a symmetric 4-level grid) into two accumulators
//    that share the query operand.  The zero-point (q2k: c0) sum is a packed
//    dot product per lane, summed over the wave through LDS.
//  * online softmax in log2 units on 64 lanes (scores staged through LDS so
//    every lane holds one (head, token pair)); the row maximum is reduced only
//    when some score exceeds the running maximum, and the denominators stay per
//    lane until the end of the split.
//  * out^T[c][j] += sum_t u[t][c] * (p[j][t] s[t][g]) on the MFMA (V codes are
//    stored in this operand order); the weights times the V scale are split
//    hi/lo the same way (packed fp16 product of fp16 halves of p and the fp16
//    scale); the zero-point term sum_t p z is a packed dot product per lane.
//  * TurboQuant ("TurboQuant KV Cache Compression — Spec", "Optimization: Fused
//    dequant-dot"): scores against the rotated query (computed once), K
//    centroids as fp16 hi and lo halves from a 16-entry LDS table; V2 as two
//    +-1 bit planes (the symmetric 4-level grid), V3/V4 as centroids from a
//    second table; 3-bit codes in 4-bit slots or in the dense 8-in-3 stream.
// Four waves per workgroup take interleaved blocks of the split, each with the
// next block in flight while it computes one, and merge in LDS; the workgroup
// writes one partial.
//
// Rounding: this file may contract a*b+c into one fma (every product here
// feeds a sum).  Range: the query operand holds q*s and the weight operand
// p*s*2^(PV-p) (weights p <= 1, PV the largest V code position: 6 for 2-bit,
// 4 for 4-bit, 0 for 8-bit codes), both in fp16: |q*s| must stay below 65504
// and a V scale below 2^(16-PV).
#include "decode_shared.h"

#pragma clang fp contract(fast)

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u3 __attribute__((ext_vector_type(3)));

constexpr int FD = 128;       // head_dim of this path
constexpr int NW = DNT / 64;  // waves per workgroup
constexpr int FPR = 64;       // fp16 rows per fp16 workgroup
// The lo halves of the split query operand (all formats, times 2^9) and of TurboQuant's V weights
// (times 2^11) are stored scaled up, in the range of the hi halves, and the lo columns are scaled
// back when combined: products of two fp16 subnormals lose precision on the matrix cores.
constexpr float LO_UP = 2048.f, LO_DOWN = 1.f / 2048.f;
constexpr float LOK_UP = 512.f, LOK_DOWN = 1.f / 512.f;

__device__ __forceinline__ f4 mfma(const u4& a, const u4& b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ h2 H2(uint32_t w) { return __builtin_bit_cast(h2, w); }
// Partials are written, and read back by the merging workgroup, with device-scope relaxed atomics:
// those accesses are coherent across the XCDs' L2 caches, and the counter increment that publishes
// a partial is issued only after its stores have completed (vmcnt(0)).
__device__ __forceinline__ void st_part(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_part(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bits of a 32-bit word as fp32.  Vector components pass through this scalar parameter: with this
// toolchain, __builtin_bit_cast applied directly to an ext_vector component (v.y) reads component 0.
__device__ __forceinline__ float F32(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ uint32_t F32bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t U32(h2 x) { return __builtin_bit_cast(uint32_t, x); }

// The exact product of two fp16 pairs as fp16 hi = rn(a*b) and lo = rn(a*b - hi).
__device__ __forceinline__ void mul_split(h2 a, h2 b, uint32_t& hi, uint32_t& lo) {
  const h2 h = a * b;
  hi = U32(h);
  lo = U32(__builtin_elementwise_fma(a, b, -h));
}
// (a*b) + c*b split the same way, for a value given as fp16 halves a + c.
__device__ __forceinline__ void mul_split2(h2 a, h2 c, h2 b, uint32_t& hi, uint32_t& lo) {
  const h2 h = a * b;
  hi = U32(h);
  lo = U32(__builtin_elementwise_fma(c, b, __builtin_elementwise_fma(a, b, -h)));
}
// a.x*b.x + a.y*b.y + acc in fp32.
__device__ __forceinline__ float dot2(h2 a, h2 b, float acc) { return __builtin_amdgcn_fdot2(a, b, acc, false); }

// fp16 half `hi` (0: bits 0..15, 1: bits 16..31) of a word, as fp32.
__device__ __forceinline__ float h16(uint32_t w, int hi) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * hi)));
}

// 2^x on the transcendental unit (results below 2^-126 may flush to 0; 2^-inf = 0).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row-of-16 all-reductions with DPP lane permutations: quad xor 1, quad xor 2, half-row mirror,
// row mirror.  Every lane of the row ends with the same value.
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
// Single code bit BIT (0 or 1) of 2-bit codes in place: element pair r sits at bit 2r + BIT.
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

// A operands (fp16 hi and lo halves) of the 8 TurboQuant K centroids coded in word w: element pair
// r holds the codes at bits 4r and 16 + 4r (word-interleaved 4-bit codes).  The centroid of a code
// is one dword (hi | lo << 16) of a 16-entry LDS table (a wave reads at most 16 distinct dwords).
__device__ __forceinline__ void tq_cen_a(uint32_t w, const uint32_t* tab, u4& ah, u4& al) {
  uint32_t hh[4], ll[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t e0 = tab[(w >> (4 * r)) & 0xFu], e1 = tab[(w >> (16 + 4 * r)) & 0xFu];
    hh[r] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);  // low halves of e0, e1
    ll[r] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);  // high halves of e0, e1
  }
  ah = u4{hh[0], hh[1], hh[2], hh[3]};
  al = u4{ll[0], ll[1], ll[2], ll[3]};
}

// The same for 8 dense 3-bit codes: channel 2r + e of the step at bits 6r + 3e of x (the step's
// 24-bit field of the dense stream), table entries 0..7.
__device__ __forceinline__ void tq_cen_a3(uint32_t x, const uint32_t* tab, u4& ah, u4& al) {
  uint32_t hh[4], ll[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t e0 = tab[(x >> (6 * r)) & 7u], e1 = tab[(x >> (6 * r + 3)) & 7u];
    hh[r] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
    ll[r] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
  }
  ah = u4{hh[0], hh[1], hh[2], hh[3]};
  al = u4{ll[0], ll[1], ll[2], ll[3]};
}
// The 24-bit field of group g of 8 dense 3-bit codes (bits 24 g .. 24 g + 23) in a lane's words:
// K steps (three words per row chunk) and V channel tiles (six words per chunk).
__device__ __forceinline__ uint32_t dense3_step(const uint32_t* k, int g) {
  const uint32_t* w = k + 3 * (g >> 2);
  const int st = g & 3;
  return st == 0 ? w[0] : st == 1 ? __builtin_amdgcn_alignbit(w[1], w[0], 24)
                        : st == 2 ? __builtin_amdgcn_alignbit(w[2], w[1], 16) : w[2] >> 8;
}

// Signed plane of code bit BIT of 2-bit codes, from the complemented code words nd: every element
// is s = 2 * bit - 1 as fp16 +-1.0 (`one16` = 0x3C003C00; the sign bit is set where the code bit is
// 0).  Planes of +-1 keep a symmetric 4-level grid free of a constant term, so sums over many
// tokens do not cancel; normal (not subnormal) operands keep the products with small weights exact
// (products of two fp16 subnormals lose precision on the matrix cores).  `one16` is passed in as a
// value (not a literal) so that the merge of sign and magnitude stays one and-or.
template <int BIT>
__device__ __forceinline__ u4 splane_a(const uint32_t* nd, int k, uint32_t one16) {
  const int base = (k & 1) ? 8 : 0;
  const uint32_t w = nd[k >> 1];
  uint32_t o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t sgn = w << (15 - (base + 2 * r + BIT));  // complemented bit -> bits 15 and 31
    o[r] = (sgn & 0x80008000u) | one16;
  }
  return u4{o[0], o[1], o[2], o[3]};
}

template <int R, bool RP>
struct alignas(16) FastWave {
  static constexpr int NC = 2 * R;  // MFMA columns in use: hi halves of heads 0..R-1, then lo halves
  static constexpr int QV = RP ? 2 : 1;  // query operands: RoPE keeps one per 16-token row tile
  // Rows are padded by 16 bytes so that the 16 column lanes of an MFMA operand read (and the
  // 16-byte score stores) fall on distinct LDS banks.
  union {
    uint32_t qb[QV][NC][FD / 2 + 4];  // query operand: [row tile][column][channel pair]
    float o[R][FD];                   // wave output for the workgroup merge
  } x;
  float ps[NC][G + 4];            // raw score columns of the current block
  float kp[RP ? 1 : R][64 + 4];   // zero-point (q2k: c0) term per head and lane (not with RoPE)
  uint32_t km[RP ? 2 : 1][RP ? 64 : 1];  // RoPE: the block's K scales and zeros, channel pairs
  uint32_t ab[4][NC][4 * 4 + 4];  // weights x V scale: [group][column][4 * token group + pair]
  float zt[R][4], m[R], l[R];
};
template <int R, bool RP>
struct FastSmem {
  FastWave<R, RP> w[NW];
  // RoPE: cos, sin of i * theta_f for rows i < 16, [i][2 f + (0: cos, 1: sin)], rows padded by 16
  // bytes (the 16 row lanes of a read fall on distinct banks)
  float rk[RP ? 16 : 1][RP ? 2 * 64 + 4 : 1];
  int sinks[MAX_SINK];  // committed sink positions (< P) of this batch element
  int nsinks;
  uint32_t tq_tab[32];  // TurboQuant K centroids, then V centroids times 8 (4-bit V slots): fp16 hi | lo << 16
};
// LDS of an fp16-row workgroup (shares the allocation of the bulk workgroups).
template <int R>
struct FpSmem {
  uint32_t q[R][FD / 2];    // query, fp16 pairs
  float sc[R][FPR];         // scores, then weights, of the workgroup's rows
  float red[NW][R][FD];     // per row group value sums
  float m[R], l[R];
  int spos[MAX_SINK], sslot[MAX_SINK];
  int nsink;
};
template <int R, bool RP>
union DecSmem {
  FastSmem<R, RP> bulk;
  FpSmem<R> fp;
  float rot[2][FD];  // the merging workgroup: TurboQuant outputs rotated back, two heads at a time
};

// What one lane reads from a block record.
template <int KB, int VB>
struct Blk {
  uint32_t kd[2][KB];  // K code rows i16 and 16 + i16, channels 32*kg .. 32*kg + 31 (RoPE: channels
                       // 16*kg .. 16*kg + 15 in kd[.][0, KB/2), their partners + 64 in kd[.][KB/2, KB))
  uint32_t ks, kz;     // K scale (q2k: rms) and zero of channels 2*lane, 2*lane + 1
                       // (TurboQuant: fp32 K norms of tokens 2*i16, 2*i16 + 1)
  uint32_t vd[2 * VB]; // V code chunk `lane`
  u4 vs, vz;           // V scale and zero of tokens 2*i16, 2*i16 + 1: [group][token] fp16
                       // (TurboQuant: vs.x, vs.y = fp32 V norms of tokens 2*i16, 2*i16 + 1)
};

// Per-lane byte offsets, inside a block record, of what load_blk reads.
struct BlkOffs {
  uint32_t k[2], ks, kz, v, vs, vz;
};
template <int FMT, int KB, int VB, bool RP>
__device__ __forceinline__ BlkOffs blk_offsets(const LayerView& lv, int lane) {
  const int i16 = lane & 15, kg = lane >> 4;
  BlkOffs o;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)  // a code row is FD * KB / 8 bytes; RoPE: 16 channels are 2 * KB bytes
    o.k[tau] = (uint32_t)(lv.k_codes + (16 * tau + i16) * (FD * KB / 8) + kg * (RP ? 2 : 4) * KB);
  if constexpr (FMT == KVQ_FMT_TQ) {  // per-token fp32 norms: tokens 2*i16, 2*i16 + 1
    o.ks = (uint32_t)(lv.k_meta + 8 * i16);
    o.kz = o.ks;
    o.vs = (uint32_t)(lv.v_meta + 8 * i16);
    o.vz = o.vs;
  } else {
    o.ks = (uint32_t)(lv.k_meta + 4 * lane);
    o.kz = (uint32_t)(lv.k_meta + 2 * FD + 4 * lane);
    o.vs = (uint32_t)(lv.v_meta + 16 * i16);
    o.vz = (uint32_t)(lv.v_meta + 2 * G * (FD / 32) + 16 * i16);
  }
  o.v = (uint32_t)(lv.v_codes + lane * 8 * VB);
  return o;
}

// One block record into registers: buffer loads from the stream's ring with the record's byte
// offset in a scalar register and fixed per-lane offsets (no address arithmetic per block).
template <int FMT, int KB, int VB, bool RP>
__device__ __forceinline__ void load_blk(Blk<KB, VB>& d, __amdgpu_buffer_rsrc_t rs, uint32_t rec_off,
                                         const BlkOffs& o) {
  constexpr bool Q2K = FMT == KVQ_FMT_Q2K, TQ = FMT == KVQ_FMT_TQ;
  // the loads of one record stay together and in this order (scheduling barriers), so the wait
  // counts the compiler derives for each block are the count of loads issued after it
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    if constexpr (RP) {  // channels 16*kg .. 16*kg + 15 and the same + 64 (8 * KB bytes further)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t off = o.k[tau] + hf * 8 * KB;
        if constexpr (KB == 2) {
          d.kd[tau][hf] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, rec_off, 0);
        } else if constexpr (KB == 4) {
          const u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, rec_off, 0);
          d.kd[tau][2 * hf] = x.x, d.kd[tau][2 * hf + 1] = x.y;
        } else {
          const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, rec_off, 0);
          d.kd[tau][4 * hf] = x.x, d.kd[tau][4 * hf + 1] = x.y, d.kd[tau][4 * hf + 2] = x.z, d.kd[tau][4 * hf + 3] = x.w;
        }
      }
    } else if constexpr (KB == 2) {
      const u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k[tau], rec_off, 0);
      d.kd[tau][0] = x.x, d.kd[tau][1] = x.y;
    } else if constexpr (KB == 3) {  // TurboQuant's dense 3-bit stream: 32 codes in 3 words
      const u3 x = __builtin_amdgcn_raw_buffer_load_b96(rs, o.k[tau], rec_off, 0);
      d.kd[tau][0] = x.x, d.kd[tau][1] = x.y, d.kd[tau][2] = x.z;
    } else {
#pragma unroll
      for (int k = 0; k < KB / 4; ++k) {
        const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k[tau] + 16 * k, rec_off, 0);
        d.kd[tau][4 * k] = x.x, d.kd[tau][4 * k + 1] = x.y, d.kd[tau][4 * k + 2] = x.z, d.kd[tau][4 * k + 3] = x.w;
      }
    }
  }
  if constexpr (TQ) {
    const u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, o.ks, rec_off, 0);
    d.ks = x.x, d.kz = x.y;
  } else {
    d.ks = __builtin_amdgcn_raw_buffer_load_b32(rs, o.ks, rec_off, 0);
    d.kz = Q2K ? 0u : __builtin_amdgcn_raw_buffer_load_b32(rs, o.kz, rec_off, 0);
  }
  if constexpr (VB == 3) {  // TurboQuant's dense 3-bit stream: 64 codes of the chunk in 6 words
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u3 x = __builtin_amdgcn_raw_buffer_load_b96(rs, o.v + 12 * k, rec_off, 0);
      d.vd[3 * k] = x.x, d.vd[3 * k + 1] = x.y, d.vd[3 * k + 2] = x.z;
    }
  } else {
#pragma unroll
    for (int k = 0; k < VB / 2; ++k) {
      const u4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, o.v + 16 * k, rec_off, 0);
      d.vd[4 * k] = x.x, d.vd[4 * k + 1] = x.y, d.vd[4 * k + 2] = x.z, d.vd[4 * k + 3] = x.w;
    }
  }
  if constexpr (TQ) {
    const u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, o.vs, rec_off, 0);
    d.vs = u4{x.x, x.y, 0u, 0u};
    d.vz = u4{0, 0, 0, 0};
  } else {
    d.vs = __builtin_amdgcn_raw_buffer_load_b128(rs, o.vs, rec_off, 0);
    if constexpr (!Q2K) d.vz = __builtin_amdgcn_raw_buffer_load_b128(rs, o.vz, rec_off, 0);
    else d.vz = u4{0, 0, 0, 0};
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, int KB, int VB, int R>
struct Fast {
  static constexpr bool Q2K = FMT == KVQ_FMT_Q2K;
  static constexpr bool TQ = FMT == KVQ_FMT_TQ;
  static constexpr int NC = 2 * R;
  static constexpr int NPL = R <= 4 ? 1 : R / 4;  // (head, token pair) slots per lane in the compact phase
  static constexpr int NKA = Q2K ? 2 : 1;         // K accumulators per token tile (q2k: one per code bit)
};

// RoPE on read ("StreamingLLM + KIVI — long-context decode without growing the KV cache", "RoPE
// caveat"): a bulk row at position p (>= lo, like the query's own position P - 1) has index
// (sinks below lo) + p - lo, so q(P-1) . k(p) = q R((P-1-p) theta) . k: the query turns by
// (P - 1 - p0 - 16 tau) theta per 16-token row tile tau of a block at p0 (the MFMA column operand of
// that tile), the key of row i16 of the tile by i16 theta (a per-lane constant), dequantized in
// fp32 and split into fp16 hi + lo halves for the MFMA.  Per-lane state of a wave:
template <int R>
struct RopeLane {
  f2 ql[R], qh[R];           // query channels fp, fp + 1 and fp + 64, fp + 65 (fp = 2 * (lane & 31))
  float c[2], s[2];          // cos, sin of the current block's query angle, frequencies fp, fp + 1
  float cst[2], sst[2];      // cos, sin of one wave step (NW blocks) at those frequencies
  const float* rk;           // cos, sin of i16 * theta_f, f = 16 * kg + 0..15 (LDS)
};

// Dword index, inside a query operand row, of the channel pair (c, c + 1) (c even) in the RoPE
// K order: step st < 2 takes channels 16 kg + 8 st .. + 7, step st >= 2 the same + 64.
__device__ __forceinline__ int rope_qpair(int c) {
  const int h = c >> 6, x = c & 63;
  return 16 * (x >> 4) + 4 * (2 * h + ((x >> 3) & 1)) + ((x >> 1) & 3);
}
// Codes of the channel pair (8 sp + 2 r, + 1) of half hf (channels 16 kg .. + 15, or + 64) of a
// RoPE code row, masked in place as two fp16 subnormals u * 2^(p - 24), p = rope_pos<KB>(r) (a dword
// holds the 16 / KB channel pairs i at bits KB i (even channel) and 16 + KB i (odd); codes above bit
// 7 of a half are shifted down first).
template <int KB>
constexpr int rope_pos(int r) {
  return KB == 2 ? 2 * r : KB == 4 ? 4 * (r & 1) : 0;
}
template <int KB>
__device__ __forceinline__ uint32_t rope_codes(const uint32_t* kd, int hf, int sp, int r) {
  if constexpr (KB == 2) {
    const uint32_t w = sp ? kd[hf] >> 8 : kd[hf];
    return w & (0x00030003u << (2 * r));
  } else if constexpr (KB == 4) {
    const uint32_t w = kd[2 * hf + sp];
    return (r >= 2 ? w >> 8 : w) & (0x000F000Fu << (4 * (r & 1)));
  } else {
    const uint32_t w = kd[4 * hf + 2 * sp + (r >> 1)];
    return ((r & 1) ? w >> 8 : w) & 0x00FF00FFu;
  }
}
// fp16 hi = rn(a), rn(b) and lo = rn((x - hi) * up) of two fp32 values, packed pairs (the lo halves
// as one mixed-precision fma each: exact product hi * up, one rounding).
__device__ __forceinline__ void split16(float a, float b, float up, uint32_t& hi, uint32_t& lo) {
  const h2 h = h2{(_Float16)a, (_Float16)b};
  hi = U32(h);
  const _Float16 l0 = (_Float16)__builtin_fmaf((float)h.x, -up, a * up);
  const _Float16 l1 = (_Float16)__builtin_fmaf((float)h.y, -up, b * up);
  lo = U32(h2{l0, l1});
}
// The same without scaling, hi rounded toward zero: lo = rn(x - hi).  nm1 is -1 held in a register (an fma by a literal -1
// would be rewritten as a subtraction, which the mixed-precision fma does not cover).
__device__ __forceinline__ void split16u(float a, float b, float nm1, uint32_t& hi, uint32_t& lo) {
  const h2 h = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(a, b));  // one instruction per pair
  hi = U32(h);
  lo = U32(h2{(_Float16)__builtin_fmaf((float)h.x, nm1, a), (_Float16)__builtin_fmaf((float)h.y, nm1, b)});
}

// Per-lane state of a wave over its blocks.
template <int FMT, int KB, int VB, int R>
struct State {
  using F = Fast<FMT, KB, VB, R>;
  h2 q2[R];             // query channels 2*lane, 2*lane + 1 (fp16)
  h2 fa2, fa2l;         // 2^-pos of their K element pair (lo halves: times 2^11)
  float cs, kc;         // score = fma(raw, cs, kappa * kc), log2 units (TurboQuant: raw * cs * K norm)
  float vb, vg;         // TurboQuant V level = cm + vb * s0 + vg * s1, s = 2 * bit - 1
  uint32_t one16;       // TurboQuant: fp16 pair (1.0, 1.0)
  float lf, ifv;        // -log2 and 2^ of the V position factor of this lane's token pair
  float m_[F::NPL], lfm[F::NPL], l_[F::NPL], zacc[F::NPL][4];
  f4 acc[8];
};

template <int FMT, int KB, int VB, int R, bool RP>
__device__ __forceinline__ void block_step(State<FMT, KB, VB, R>& S, FastWave<R, RP>& W, const RopeLane<R>& Q,
                                           const int* sinks, const Blk<KB, VB>& d, int blk, int blo, int bhi,
                                           int sblk, int nsink, float q2k_w, const uint32_t* tab, int lane) {
  using F = Fast<FMT, KB, VB, R>;
  constexpr bool Q2K = F::Q2K;
  constexpr bool TQ = F::TQ;
  constexpr int NPL = F::NPL;
  const int i16 = lane & 15, kg = lane >> 4, tp = i16;
  // MFMA column of this lane; padding lanes repeat the last column (identical values, identical stores)
  const int col = i16 < F::NC ? i16 : F::NC - 1;

  // ---- query operand: the exact products q * s split hi (column j) / lo (R + j), times 2^-pos ----
  // (TurboQuant: the rotated query, written once before the loop; RoPE: the turned query of each
  // row tile, and the block's K scales and zeros for the dequantization)
  if constexpr (RP) {
    W.km[0][lane] = d.ks;
    W.km[1][lane] = d.kz;
    const int tq = lane >> 5, fp = 2 * (lane & 31);
    const int il = rope_qpair(fp), ih = rope_qpair(64 + fp);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float x0 = Q.ql[j].x, x1 = Q.ql[j].y, y0 = Q.qh[j].x, y1 = Q.qh[j].y;
      uint32_t h, l;
      split16(x0 * Q.c[0] - y0 * Q.s[0], x1 * Q.c[1] - y1 * Q.s[1], LOK_UP, h, l);
      W.x.qb[tq][j][il] = h;
      W.x.qb[tq][R + j][il] = l;
      split16(y0 * Q.c[0] + x0 * Q.s[0], y1 * Q.c[1] + x1 * Q.s[1], LOK_UP, h, l);
      W.x.qb[tq][j][ih] = h;
      W.x.qb[tq][R + j][ih] = l;
    }
  } else if constexpr (!TQ) {
    const h2 s2 = H2(d.ks);
    const h2 z2 = Q2K ? s2 : H2(d.kz);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      uint32_t h, l;
      mul_split(S.q2[j], s2, h, l);
      W.x.qb[0][j][lane] = U32(H2(h) * S.fa2);
      W.x.qb[0][R + j][lane] = U32(H2(l) * S.fa2l);
      W.kp[j][lane] = dot2(S.q2[j], z2, 0.f);
    }
  }
  // ---- scores: raw MFMA columns to LDS ----
  if constexpr (RP) {
    // keys k = u s + z per channel (fp32), turned by i16 theta in (f, f + 64) pairs, split into fp16
    // hi and lo halves (two MFMA products per step into one accumulator; a lo half below the fp16
    // normal range keeps its absolute precision, 2^-25, and meets a normal query half)
    f4 c0[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
    float nm1 = -1.f;
    asm("" : "+v"(nm1));  // opaque to the optimizer (no instruction)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      const u4 sl = *reinterpret_cast<const u4*>(&W.km[0][8 * kg + 4 * sp]);
      const u4 zl = *reinterpret_cast<const u4*>(&W.km[1][8 * kg + 4 * sp]);
      const u4 sh = *reinterpret_cast<const u4*>(&W.km[0][32 + 8 * kg + 4 * sp]);
      const u4 zh = *reinterpret_cast<const u4*>(&W.km[1][32 + 8 * kg + 4 * sp]);
      const uint32_t slv[4] = {sl.x, sl.y, sl.z, sl.w}, zlv[4] = {zl.x, zl.y, zl.z, zl.w};
      const uint32_t shv[4] = {sh.x, sh.y, sh.z, sh.w}, zhv[4] = {zh.x, zh.y, zh.z, zh.w};
      // scales times 2^(24 - p): the codes enter as fp16 subnormals u * 2^(p - 24)
      float sls[4][2], shs[4][2];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          constexpr float one = 1.f;
          const float f = __builtin_ldexpf(one, 24 - rope_pos<KB>(r));
          sls[r][e] = h16(slv[r], e) * f;
          shs[r][e] = h16(shv[r], e) * f;
        }
      float kc[8], ks[8];  // frequencies 16 kg + 8 sp + 0..7
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f4 t = *reinterpret_cast<const f4*>(Q.rk + 16 * sp + 4 * m);
        kc[2 * m] = t[0], ks[2 * m] = t[1], kc[2 * m + 1] = t[2], ks[2 * m + 1] = t[3];
      }
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        uint32_t ahl[4], all[4], ahh[4], alh[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float rl[2], rh[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float kl = __builtin_fmaf(h16(rope_codes<KB>(d.kd[tau], 0, sp, r), e), sls[r][e], h16(zlv[r], e));
            const float kh = __builtin_fmaf(h16(rope_codes<KB>(d.kd[tau], 1, sp, r), e), shs[r][e], h16(zhv[r], e));
            const int fi = 2 * r + e;
            rl[e] = kl * kc[fi] - kh * ks[fi];
            rh[e] = kh * kc[fi] + kl * ks[fi];
          }
          split16u(rl[0], rl[1], nm1, ahl[r], all[r]);
          split16u(rh[0], rh[1], nm1, ahh[r], alh[r]);
        }
        const u4 bl = *reinterpret_cast<const u4*>(&W.x.qb[tau][col][16 * kg + 4 * sp]);
        const u4 bh = *reinterpret_cast<const u4*>(&W.x.qb[tau][col][16 * kg + 4 * (sp + 2)]);
        c0[tau] = mfma(u4{ahl[0], ahl[1], ahl[2], ahl[3]}, bl, c0[tau]);
        c0[tau] = mfma(u4{ahh[0], ahh[1], ahh[2], ahh[3]}, bh, c0[tau]);
        c0[tau] = mfma(u4{all[0], all[1], all[2], all[3]}, bl, c0[tau]);
        c0[tau] = mfma(u4{alh[0], alh[1], alh[2], alh[3]}, bh, c0[tau]);
      }
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
      *reinterpret_cast<f4*>(&W.ps[col][16 * tau + 4 * kg]) = c0[tau];
  } else {
    f4 c0[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
    f4 c1[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u4 b = *reinterpret_cast<const u4*>(&W.x.qb[0][col][16 * kg + 4 * st]);
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        if constexpr (Q2K) {
          c0[tau] = mfma(plane_a<0>(d.kd[tau], st), b, c0[tau]);
          c1[tau] = mfma(plane_a<1>(d.kd[tau], st), b, c1[tau]);
        } else if constexpr (TQ) {  // centroid hi halves, then lo halves, into one accumulator
          u4 ah, al;
          if constexpr (KB == 3) tq_cen_a3(dense3_step(d.kd[tau], st), tab, ah, al);
          else tq_cen_a(d.kd[tau][st], tab, ah, al);
          c0[tau] = mfma(ah, b, c0[tau]);
          c0[tau] = mfma(al, b, c0[tau]);
        } else {
          c0[tau] = mfma(codes_a<KB>(d.kd[tau], st), b, c0[tau]);
        }
      }
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f4 c = c0[tau];
      if constexpr (Q2K) c = c0[tau] + c1[tau] * q2k_w;
      *reinterpret_cast<f4*>(&W.ps[col][16 * tau + 4 * kg]) = c;
    }
  }

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
  float y0[NPL], y1[NPL];
  bool grow = false;
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int jr = kg + 4 * p;
    const int j = jr < R ? jr : R - 1;  // lanes past the last head repeat it (identical stores)
    const f2 hi = *reinterpret_cast<const f2*>(&W.ps[j][2 * tp]);
    const f2 lo = *reinterpret_cast<const f2*>(&W.ps[R + j][2 * tp]);
    if constexpr (TQ) {  // score = scale * K norm * (rotated query . centroids)
      y0[p] = ok0 ? __builtin_fmaf(lo.x, LOK_DOWN, hi.x) * (S.cs * F32(d.ks)) : -INFINITY;
      y1[p] = ok1 ? __builtin_fmaf(lo.y, LOK_DOWN, hi.y) * (S.cs * F32(d.kz)) : -INFINITY;
    } else {
      float kap = 0.f;  // RoPE: the zeros are inside the dequantized keys
      if constexpr (!RP) {
        const f4 kq = *reinterpret_cast<const f4*>(&W.kp[j][4 * tp]);
        kap = row_sum16((kq[0] + kq[1]) + (kq[2] + kq[3])) * S.kc;
      }
      y0[p] = ok0 ? __builtin_fmaf(__builtin_fmaf(lo.x, LOK_DOWN, hi.x), S.cs, kap) : -INFINITY;
      y1[p] = ok1 ? __builtin_fmaf(__builtin_fmaf(lo.y, LOK_DOWN, hi.y), S.cs, kap) : -INFINITY;
    }
    grow = grow || fmaxf(y0[p], y1[p]) > S.m_[p];
  }
  // a new running maximum somewhere in the wave: reduce the row maxima and rescale
  const bool resc = __any(grow);
  float fc = 1.f;  // rescale factor of the head of this lane's MFMA column (i16 % R)
  if (resc) {
    float fp[NPL];
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const float mold = S.m_[p];
      const float mnew = fmaxf(mold, row_max16(fmaxf(y0[p], y1[p])));
      const float f = mold == mnew ? 1.f : (mold == -INFINITY ? 0.f : ex2(mold - mnew));
      S.m_[p] = mnew;
      S.lfm[p] = mnew == -INFINITY ? 0.f : S.lf - mnew;
      S.l_[p] *= f;
#pragma unroll
      for (int q = 0; q < 4; ++q) S.zacc[p][q] *= f;
      fp[p] = f;
    }
    // head h sits in row h % 4 of slot h / 4 (every lane of a row holds its factor): a lane
    // exchange instead of an LDS round trip
    const int hc = i16 % R, src = 16 * (hc & 3);
    fc = __shfl(fp[0], src);
    if constexpr (NPL > 1) {
      const float f1 = __shfl(fp[1], src);
      fc = hc < 4 ? fc : f1;
    }
  }
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int jr = kg + 4 * p;
    const int j = jr < R ? jr : R - 1;
    // weights times the V position factor of this token pair; masked tokens give 2^-inf = 0
    const float e0 = ex2(y0[p] + S.lfm[p]), e1 = ex2(y1[p] + S.lfm[p]);
    S.l_[p] = __builtin_fmaf(e0 + e1, S.ifv, S.l_[p]);
    if constexpr (TQ && VB != 2) {
      // 3- and 4-bit V codes: the centroids (times 8) from the LDS table are the A operand, the
      // weights times the V norm (times 1/8, so that they stay in the fp16 range) the B operand
      const float w0 = e0 * F32(d.vs.x) * 0.125f, w1 = e1 * F32(d.vs.y) * 0.125f;
      const h2 wh = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(w0, w1));
      const h2 wl = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz((w0 - (float)wh.x) * LO_UP,
                                                                       (w1 - (float)wh.y) * LO_UP));
      W.ab[0][j][4 * kgt + (et >> 1)] = U32(wh);
      W.ab[0][R + j][4 * kgt + (et >> 1)] = U32(wl);
      continue;
    } else if constexpr (TQ) {
      // V level = cm + vb * s0 + vg * s1 (s = 2 * bit - 1) in the rotated domain, times the V
      // norm: the two signed bit planes take the weights w * vb and w * vg (split hi/lo), the cm
      // term is sum_t w (cm = 0 for the symmetric grids the library builds)
      const float w0 = e0 * F32(d.vs.x), w1 = e1 * F32(d.vs.y);
      S.zacc[p][0] += w0 + w1;
      const float xb0 = w0 * S.vb, xb1 = w1 * S.vb, xg0 = w0 * S.vg, xg1 = w1 * S.vg;
      const h2 bh = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(xb0, xb1));
      const h2 bl = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz((xb0 - (float)bh.x) * LO_UP,
                                                                       (xb1 - (float)bh.y) * LO_UP));
      const h2 gh = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(xg0, xg1));
      const h2 gl = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz((xg0 - (float)gh.x) * LO_UP,
                                                                       (xg1 - (float)gh.y) * LO_UP));
      W.ab[0][j][4 * kgt + (et >> 1)] = U32(bh);
      W.ab[0][R + j][4 * kgt + (et >> 1)] = U32(bl);
      W.ab[1][j][4 * kgt + (et >> 1)] = U32(gh);
      W.ab[1][R + j][4 * kgt + (et >> 1)] = U32(gl);
      continue;
    }
    const h2 ph = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(e0, e1));
    const h2 pl = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(e0 - (float)ph.x, e1 - (float)ph.y));
    const uint32_t vs[4] = {d.vs.x, d.vs.y, d.vs.z, d.vs.w};
    const uint32_t vz[4] = {d.vz.x, d.vz.y, d.vz.z, d.vz.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const h2 s2 = H2(vs[q]);  // V scales of tokens t0, t0 + 1 in group q
      uint32_t h, l;
      mul_split2(ph, pl, s2, h, l);
      W.ab[q][j][4 * kgt + (et >> 1)] = h;
      W.ab[q][R + j][4 * kgt + (et >> 1)] = l;
      const h2 z2 = Q2K ? s2 : H2(vz[q]);
      S.zacc[p][q] = dot2(ph, z2, dot2(pl, z2, S.zacc[p][q]));
    }
  }
  // ---- values (rare: rescale the running sums to a new maximum first) ----
  if (resc) {
#pragma unroll
    for (int mu = 0; mu < 8; ++mu) S.acc[mu] *= fc;
  }
  if constexpr (TQ && VB != 2) {  // centroid hi halves, then lo halves, into one accumulator
    const u4 b0 = *reinterpret_cast<const u4*>(&W.ab[0][col][4 * kg]);
#pragma unroll
    for (int mu = 0; mu < 8; ++mu) {
      u4 ah, al;
      if constexpr (VB == 3) tq_cen_a3(dense3_step(d.vd, mu), tab + 16, ah, al);
      else tq_cen_a(d.vd[mu], tab + 16, ah, al);
      S.acc[mu] = mfma(ah, b0, S.acc[mu]);
      S.acc[mu] = mfma(al, b0, S.acc[mu]);
    }
  } else if constexpr (TQ) {
    const u4 b0 = *reinterpret_cast<const u4*>(&W.ab[0][col][4 * kg]);
    const u4 b1 = *reinterpret_cast<const u4*>(&W.ab[1][col][4 * kg]);
    const uint32_t nd[4] = {~d.vd[0], ~d.vd[1], ~d.vd[2], ~d.vd[3]};
#pragma unroll
    for (int mu = 0; mu < 8; ++mu) {
      S.acc[mu] = mfma(splane_a<0>(nd, mu, S.one16), b0, S.acc[mu]);
      S.acc[mu] = mfma(splane_a<1>(nd, mu, S.one16), b1, S.acc[mu]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u4 bq = *reinterpret_cast<const u4*>(&W.ab[q][col][4 * kg]);
#pragma unroll
      for (int mu = 2 * q; mu < 2 * q + 2; ++mu) S.acc[mu] = mfma(codes_a<VB>(d.vd, mu), bq, S.acc[mu]);
    }
  }
}

template <int FMT, int KB, int VB, int R, bool RP>
__device__ void bulk_partial(const DecodeArgs& a, FastSmem<R, RP>& F, int sigma) {
  using Fc = Fast<FMT, KB, VB, R>;
  using St = State<FMT, KB, VB, R>;
  constexpr bool Q2K = Fc::Q2K;
  constexpr bool TQ = Fc::TQ;
  constexpr int NPL = Fc::NPL;
  constexpr int PV = code_pos<VB>(3);
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform: keeps the loop scalar)
  const int i16 = lane & 15, kg = lane >> 4;
  const int s = blockIdx.x, b = s / sh.Hkv, g = s % sh.Hkv;
  auto& W = F.w[wv];

  const int first = sigma * a.blocks_per_split;
  const int lastb = min(a.nblk, first + a.blocks_per_split);
  const int blo = (int)a.bulk_lo, bhi = (int)a.bulk_hi;  // positions fit in int32 (checked on the host)
  const int blkf = (int)a.blk_first;
  const int slot0 = (int)(a.blk_first % lv.cap_b);  // ring slot of bulk block index 0
  // the stream's ring as a buffer resource (every record offset fits in 32 bits: checked on the host)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(lv.bulk + (int64_t)s * lv.cap_b * lv.rec), 0, (int)(lv.cap_b * lv.rec), 0x00020000);
  const BlkOffs bo = blk_offsets<FMT, KB, VB, RP>(lv, lane);
  auto rec_of = [&](int bi) -> uint32_t {
    bi = bi < lastb ? bi : lastb - 1;  // past the split: re-read its last block (a cache hit), never used
    int sl = slot0 + bi;
    if (sl >= lv.cap_b) sl -= lv.cap_b;
    return (uint32_t)sl * (uint32_t)lv.rec;
  };
  // Two register buffers: the next block of this wave is in flight while the current one is
  // computed (a deeper ring costs the registers of a third wave per SIMD, which hides more).  The
  // wave's first block is requested together with the prologue's loads, and the prologue ends by
  // waiting for all of them, so the loop is entered with no load in flight and its back edge
  // carries exactly one block (the compiler's wait counts inside the loop then stay exact).
  Blk<KB, VB> d0, d1;
  int bi = first + wv;
  if (bi < lastb) load_blk<FMT, KB, VB, RP>(d0, rs, rec_of(bi), bo);
  St S;
  const float al = a.scale * LOG2E;
  float q2k_w = 0.f, tq_c0 = 0.f;
  float sg0 = 0.f, sg1 = 0.f, kcen = 0.f, vcen = 0.f;
  if constexpr (TQ) {
    // rotated-domain centroids enter the MFMA as real values: no code-position factor
    S.cs = al;
    S.kc = 0.f;
    // level(u) = cm + vb * s0 + vg * s1 for u = b0 + 2 b1, s = 2b - 1: exact when the grid has
    // c0 + c3 = c1 + c2 (the symmetric Lloyd-Max grid, where cm = 0)
    const float c0 = lv.tables->v_cen[0], c3 = lv.tables->v_cen[3];
    S.vb = 0.5f * (lv.tables->v_cen[1] - c0);
    S.vg = 0.5f * (lv.tables->v_cen[2] - c0);
    tq_c0 = VB == 2 ? 0.5f * (c0 + c3) : 0.f;  // 4-bit V slots: centroids from the table, no cm term
    sg0 = lv.tables->signs[2 * lane];
    sg1 = lv.tables->signs[2 * lane + 1];
    // 1 in every lane, as a per-lane run-time value (bit 29 of the fp32 +-1 sign entries), so the
    // fp16 pair (1.0, 1.0) lives in a vector register and each plane register is one shift plus one
    // and-or
    const uint32_t one = (F32bits(sg0) >> 29) & 1u;
    S.one16 = one * 0x3C003C00u;
    kcen = tid < 16 ? lv.tables->k_cen[tid] : 0.f;
    vcen = tid < 16 ? 8.f * lv.tables->v_cen[tid] : 0.f;
  } else if constexpr (Q2K) {
    const float c0 = lv.tables->q2k_lvl[0], c1 = lv.tables->q2k_lvl[1] - c0, c2 = lv.tables->q2k_lvl[2] - c0;
    S.cs = ldexpf(c1 * al, 24);
    S.kc = c0 * al;
    q2k_w = c2 / (2.f * c1);  // the b1 accumulator carries an extra factor 2 (bit 2r + 1)
  } else {  // codes enter as u * 2^(pos - 24) (RoPE: as dequantized keys)
    S.cs = RP ? al : ldexpf(al, 24);
    S.kc = RP ? 0.f : al;
  }
  RopeLane<R> Q;
  int kq = 0;  // RoPE: P - 1 - p0 - 16 tau of the wave's current block (tau = lane >> 5)
  if constexpr (RP) {
    const int fp = 2 * (lane & 31);
    const _Float16* qs = static_cast<const _Float16*>(a.q) + ((int64_t)b * sh.Hq + (int64_t)g * R) * FD;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const h2 lo2 = H2(*reinterpret_cast<const uint32_t*>(qs + j * FD + fp));
      const h2 hi2 = H2(*reinterpret_cast<const uint32_t*>(qs + j * FD + 64 + fp));
      Q.ql[j] = f2{(float)lo2.x, (float)lo2.y};
      Q.qh[j] = f2{(float)hi2.x, (float)hi2.y};
    }
    for (int idx = tid; idx < 16 * 64; idx += DNT) {
      const int i = idx >> 6, f = idx & 63;
      F.rk[i][2 * f] = lv.tables->rope_row[i][f][0];
      F.rk[i][2 * f + 1] = lv.tables->rope_row[i][f][1];
    }
    Q.rk = &F.rk[i16][2 * 16 * kg];
    kq = (int)(a.P - 1 - (int64_t)(blkf + bi) * G) - 16 * (lane >> 5);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float th = lv.tables->rope_inv[fp + e];
      rope_cs(kq, th, Q.c[e], Q.s[e]);
      rope_cs(NW * G, th, Q.cst[e], Q.sst[e]);
    }
  }
  // next block of the wave: the query angle steps back by NW * G positions (a rotation; every 16th
  // step recomputed from the index, so rounding does not accumulate)
  int nstep = 0;
  auto rope_next = [&]() {
    if constexpr (RP) {
      kq -= NW * G;
      if ((++nstep & 15) == 0) {
        const int fp = 2 * (lane & 31);
#pragma unroll
        for (int e = 0; e < 2; ++e) rope_cs(kq, lv.tables->rope_inv[fp + e], Q.c[e], Q.s[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float c = Q.c[e], sn = Q.s[e];
          Q.c[e] = __builtin_fmaf(c, Q.cst[e], sn * Q.sst[e]);
          Q.s[e] = __builtin_fmaf(sn, Q.cst[e], -c * Q.sst[e]);
        }
      }
    }
  };
  {
    const int64_t qrow = ((int64_t)b * sh.Hq + (int64_t)g * R) * sh.Din;  // query rows of Din channels
    const int pk = Q2K ? 2 * (lane & 3) : code_pos<KB>(lane & 3);
    const _Float16 fa = (_Float16)ldexpf(1.f, -pk);
    S.fa2 = h2{fa, fa};
    const _Float16 fal = (_Float16)ldexpf(1.f, 9 - pk);
    S.fa2l = h2{fal, fal};
#pragma unroll
    for (int j = 0; j < R; ++j)
      S.q2[j] = H2(2 * lane < sh.Din
                       ? *reinterpret_cast<const uint32_t*>(static_cast<const _Float16*>(a.q) + qrow + j * sh.Din + 2 * lane)
                       : 0u);  // channels past Din are the zero padding
    // weights carry 2^(PV - pv): the V codes of this lane's token pair sit at bit pv (TurboQuant's
    // signed planes are +-1 at every position: no factor)
    const int t0 = 2 * i16, et = ((t0 >> 4) << 2) | (t0 & 3);
    const int pv = TQ ? PV : code_pos<VB>(et >> 1);
    S.lf = (float)(PV - pv);
    S.ifv = ldexpf(1.f, pv - PV);
  }
  stage_sinks(a, b, F.sinks, nullptr, &F.nsinks);
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    S.m_[p] = -INFINITY;
    S.lfm[p] = 0.f;
    S.l_[p] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) S.zacc[p][q] = 0.f;
  }
#pragma unroll
  for (int mu = 0; mu < 8; ++mu) S.acc[mu] = f4{0.f, 0.f, 0.f, 0.f};
  if constexpr (TQ) {
    if (tid < 16) {  // K centroid table: fp16 hi and lo halves
      const _Float16 h = (_Float16)kcen, hv = (_Float16)vcen;
      F.tq_tab[tid] = U32(h2{h, (_Float16)(kcen - (float)h)});
      F.tq_tab[16 + tid] = U32(h2{hv, (_Float16)(vcen - (float)hv)});
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the query, the sink list and the first block
  __syncthreads();
  if constexpr (TQ) {
    // rotated query q~ = c_d * FWHT(sigma * q) ("TurboQuant KV Cache Compression — Spec", "Step 1:
    // Random Rotation"; "Optimization: Fused dequant-dot": scores in the rotated domain), split into
    // fp16 hi (column j) and lo (column R + j): the K operand of every block of the call
    const float cd = (float)(1.0 / __builtin_sqrt((double)FD));
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float y0 = (float)S.q2[j].x * sg0, y1 = (float)S.q2[j].y * sg1;
      wave_fwht(y0, y1, FD, lane);
      y0 *= cd;
      y1 *= cd;
      const h2 h = h2{(_Float16)y0, (_Float16)y1};
      const h2 l = h2{(_Float16)((y0 - (float)h.x) * LOK_UP), (_Float16)((y1 - (float)h.y) * LOK_UP)};
      W.x.qb[0][j][lane] = U32(h);
      W.x.qb[0][R + j][lane] = U32(l);
    }
  }

  const int nsink = __builtin_amdgcn_readfirstlane(F.nsinks);
  const int sblk = lane < nsink ? F.sinks[lane] / G : -1;  // block of sink `lane`

  if (bi < lastb) {
    while (true) {
      load_blk<FMT, KB, VB, RP>(d1, rs, rec_of(bi + NW), bo);
      block_step(S, W, Q, F.sinks, d0, blkf + bi, blo, bhi, sblk, nsink, q2k_w, F.tq_tab, lane);
      rope_next();
      bi += NW;
      if (bi >= lastb) break;
      load_blk<FMT, KB, VB, RP>(d0, rs, rec_of(bi + NW), bo);
      block_step(S, W, Q, F.sinks, d1, blkf + bi, blo, bhi, sblk, nsink, q2k_w, F.tq_tab, lane);
      rope_next();
      bi += NW;
      if (bi >= lastb) break;
    }
  }

  // ---- wave results: zero-point term, output (column j plus column R + j), (m, l) ----
  const int tp = i16;
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int jr = kg + 4 * p;
    const float lsum = row_sum16(S.l_[p]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float z;
      if constexpr (TQ) {  // cm * sum_t w (one value for every channel group)
        z = tq_c0 * row_sum16(S.zacc[p][0] * S.ifv);
      } else {
        z = row_sum16(S.zacc[p][q] * S.ifv);
        if constexpr (Q2K) z = -8.f * z;
      }
      if (jr < R && tp == 0) W.zt[jr][q] = z;
    }
    if (jr < R && tp == 0) {
      W.m[jr] = S.m_[p];
      W.l[jr] = lsum;
    }
  }
  // V codes entered as u * 2^(pv - 24), the weights carried 2^(PV - pv) (TurboQuant: +-1 planes)
  const float SV = TQ ? 1.f : ldexpf(1.f, 24 - PV);
#pragma unroll
  for (int mu = 0; mu < 8; ++mu) {
    f4 lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = __shfl(S.acc[mu][i], lane + R);
    if (i16 < R) {
      const float zt = W.zt[i16][mu >> 1];
      const f4 v = S.acc[mu] + lo * (TQ ? LO_DOWN : 1.f);
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
      if (F.w[w].m[j] != -INFINITY) v += F.w[w].x.o[j][c] * ex2(F.w[w].m[j] - M);
    st_part(&part[j * (FD + 2) + 2 + c], v);
  }
  if (tid < R) {
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, F.w[w].m[tid]);
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (F.w[w].m[tid] != -INFINITY) L += F.w[w].l[tid] * ex2(F.w[w].m[tid] - M);
    st_part(&part[tid * (FD + 2)], M);
    st_part(&part[tid * (FD + 2) + 1], L);
  }
}

// Partial of fp16 rows [64 f, 64 f + 64) of the stream's list: window rows [bulk_hi, P) (the ones
// that are committed sinks masked: the pool holds them), then the committed sinks in slot order.
// Scores: 4 lanes per row (32 channels each, packed fp16 dot products); weights per head over the
// workgroup's rows; values: one channel pair per lane, rows split over the 4 waves.  Every row load
// (the K quarter a thread scores and the V words its wave accumulates) is issued at once, right
// after the sink list is known.
template <int R, bool RP>
__device__ void fp16_partial(const DecodeArgs& a, FpSmem<R>& F, int f) {
  constexpr int VPW = FPR / NW;  // rows per wave in the values phase
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int s = blockIdx.x, b = s / sh.Hkv, g = s % sh.Hkv;
  const int64_t qrow = ((int64_t)b * sh.Hq + (int64_t)g * R) * sh.Din;  // query rows of Din channels
  constexpr int QW = (R * FD / 2 + DNT - 1) / DNT;  // query words per thread
  uint32_t qv[QW];
#pragma unroll
  for (int k = 0; k < QW; ++k) {
    const int idx = tid + k * DNT, j = idx / (FD / 2), w = idx % (FD / 2);
    qv[k] = idx < R * FD / 2 && 2 * w < sh.Din
                ? *reinterpret_cast<const uint32_t*>(static_cast<const _Float16*>(a.q) + qrow + j * sh.Din + 2 * w)
                : 0u;
  }
  stage_sinks(a, b, F.spos, F.sslot, &F.nsink);
  if (a.k1 != nullptr && f == 0) {
    // fused decode step: the stream's appended row (position P - 1) goes to the staging rows and the
    // fp16 window ring, and the block it opens gets a zero record.  Nothing in this launch reads
    // either: the row is scored from k1 / v1, its window slot held a row below the window, and an
    // open block lies inside the fp16 window.
    const int64_t p = a.P - 1;
    if (tid < FD / 2) {
      const uint32_t kw = reinterpret_cast<const uint32_t*>(a.k1)[(int64_t)s * (FD / 2) + tid];
      const uint32_t vw = reinterpret_cast<const uint32_t*>(a.v1)[(int64_t)s * (FD / 2) + tid];
      const int64_t ws = (int64_t)s * sh.R + p % sh.R;
      reinterpret_cast<uint32_t*>(lv.staging)[((int64_t)s * G + p % G) * (FD / 2) + tid] = kw;
      reinterpret_cast<uint32_t*>(lv.win_k)[ws * (FD / 2) + tid] = kw;
      reinterpret_cast<uint32_t*>(lv.win_v)[ws * (FD / 2) + tid] = vw;
    }
    if (a.open_new) {
      uint32_t* rw = reinterpret_cast<uint32_t*>(lv.bulk + ((int64_t)s * lv.cap_b + (p / G) % lv.cap_b) * lv.rec);
      for (int i = tid; i < (int)(lv.rec / 4); i += DNT) rw[i] = 0u;
    }
  }
#pragma unroll
  for (int k = 0; k < QW; ++k) {
    const int idx = tid + k * DNT;
    if (idx < R * FD / 2) F.q[idx / (FD / 2)][idx % (FD / 2)] = qv[k];
  }
  __syncthreads();
  const int nwin = (int)(a.P - a.bulk_hi);  // positions fit in int32
  const int nfp = nwin + F.nsink;
  const int r0 = f * FPR, nr = max(0, min(FPR, nfp - r0));
  const float al = a.scale * LOG2E;

  const int w0 = nwin > 0 ? (int)a.bulk_hi % sh.R : 0;  // window slot of row 0 (nwin <= R)
  auto row_ptr = [&](int i, bool v_side) -> const uint16_t* {  // fp16 row i of the list (i < nfp)
    if (i < nwin) {
      if (a.k1 != nullptr && i == nwin - 1)  // fused step: the appended row, from the input
        return static_cast<const uint16_t*>(v_side ? a.v1 : a.k1) + (int64_t)s * FD;
      const int ws = w0 + i < sh.R ? w0 + i : w0 + i - sh.R;
      return (v_side ? lv.win_v : lv.win_k) + ((int64_t)s * sh.R + ws) * FD;
    }
    return (v_side ? lv.sink_v : lv.sink_k) + ((int64_t)s * sh.n_sink + F.sslot[i - nwin]) * FD;
  };
  const int lr = tid >> 2, qq = tid & 3, i = r0 + lr;
  u4 kw[4] = {u4{0, 0, 0, 0}, u4{0, 0, 0, 0}, u4{0, 0, 0, 0}, u4{0, 0, 0, 0}};
  if (lr < nr) {
    const u4* kr = reinterpret_cast<const u4*>(row_ptr(i, false) + 32 * qq);
#pragma unroll
    for (int k = 0; k < 4; ++k) kw[k] = kr[k];
  }
  uint32_t vw[VPW];
#pragma unroll
  for (int k = 0; k < VPW; ++k) {
    const int r = wv + NW * k;
    vw[k] = r < nr ? reinterpret_cast<const uint32_t*>(row_ptr(r0 + r, true))[lane] : 0u;
  }
  // ---- scores ----
  {
    bool ok = lr < nr;
    float acc[R];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = 0.f;
    if (ok && i < nwin)
      for (int q = 0; q < F.nsink; ++q) ok = ok && F.spos[q] != a.bulk_hi + i;
    if constexpr (RP) {
      // RoPE: q(m) . k(n) = q . R((n - m) theta) k with m the query's index: the row turns by its
      // index minus the query's, the query is used as handed over.  This thread's channels 32 qq ..
      // 32 qq + 31 pair with those of thread tid ^ 2 (channels -+ 64, one DPP step): each of the two
      // computes the cos and sin of half of their 32 shared frequencies.
      const int qi = cache_index(F.spos, F.nsink, a.lo, a.P - 1);
      int dn = 0;
      if (lr < nr) dn = cache_index(F.spos, F.nsink, a.lo, i < nwin ? a.bulk_hi + i : (int64_t)F.spos[i - nwin]) - qi;
      const int f0 = 32 * (qq & 1), hsel = qq >> 1;
      float cw[16], sw[16];  // frequencies f0 + 16 hsel + k
#pragma unroll
      for (int k = 0; k < 16; ++k) rope_cs(dn, a.lv.tables->rope_inv[f0 + 16 * hsel + k], cw[k], sw[k]);
      const uint32_t xw[16] = {kw[0].x, kw[0].y, kw[0].z, kw[0].w, kw[1].x, kw[1].y, kw[1].z, kw[1].w,
                               kw[2].x, kw[2].y, kw[2].z, kw[2].w, kw[3].x, kw[3].y, kw[3].z, kw[3].w};
      uint32_t kh[16], kl[16];  // turned key, fp16 hi and lo * 2^11, channel pairs 32 qq + 2 w
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const uint32_t yw = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)xw[w], 0x4E, 0xF, 0xF, false);
        const bool mine = hsel == (w >> 3);
        float rr[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int k = 2 * (w & 7) + e;
          // the partner's values are read in every lane (a DPP read from a lane outside the active
          // mask would return 0), then selected
          const float cp = dpp<0x4E>(cw[k]), spn = dpp<0x4E>(sw[k]);
          const float cs = mine ? cw[k] : cp, sn = mine ? sw[k] : spn;
          const float x = h16(xw[w], e), y = h16(yw, e);
          rr[e] = qq < 2 ? x * cs - y * sn : x * cs + y * sn;
        }
        split16(rr[0], rr[1], LO_UP, kh[w], kl[w]);
      }
      if (ok) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          float ah = 0.f, alo = 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const u4 qw = *reinterpret_cast<const u4*>(&F.q[j][16 * qq + 4 * k]);
            const uint32_t qv[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              ah = dot2(H2(qv[t]), H2(kh[4 * k + t]), ah);
              alo = dot2(H2(qv[t]), H2(kl[4 * k + t]), alo);
            }
          }
          acc[j] = __builtin_fmaf(alo, LO_DOWN, ah);
        }
      }
    } else if (ok) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u4 qw = *reinterpret_cast<const u4*>(&F.q[j][16 * qq + 4 * k]);
          acc[j] = dot2(H2(qw.x), H2(kw[k].x), acc[j]);
          acc[j] = dot2(H2(qw.y), H2(kw[k].y), acc[j]);
          acc[j] = dot2(H2(qw.z), H2(kw[k].z), acc[j]);
          acc[j] = dot2(H2(qw.w), H2(kw[k].w), acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float v = acc[j];
      v += dpp<0xB1>(v);
      v += dpp<0x4E>(v);
      if (qq == 0) F.sc[j][lr] = ok ? v * al : -INFINITY;
    }
  }
  __syncthreads();
  // ---- weights per head ----
  for (int j = wv; j < R; j += NW) {
    const float x = F.sc[j][lane];
    float M = x;
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float p = x == -INFINITY ? 0.f : ex2(x - M);
    F.sc[j][lane] = p;
    float L = p;
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) {
      F.m[j] = M;
      F.l[j] = L;
    }
  }
  __syncthreads();
  // ---- values ----
  {
    float acc[R][2];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j][0] = acc[j][1] = 0.f;
#pragma unroll
    for (int k = 0; k < VPW; ++k) {
      const int r = wv + NW * k;
      if (r < nr) {
        const float v0 = h16(vw[k], 0), v1 = h16(vw[k], 1);
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const float p = F.sc[j][r];
          acc[j][0] = __builtin_fmaf(p, v0, acc[j][0]);
          acc[j][1] = __builtin_fmaf(p, v1, acc[j][1]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) *reinterpret_cast<f2*>(&F.red[wv][j][2 * lane]) = f2{acc[j][0], acc[j][1]};
  }
  __syncthreads();
  float* part = a.ws + ((int64_t)s * a.nparts + a.splits + f) * R * (FD + 2);
  for (int idx = tid; idx < R * FD; idx += DNT) {
    const int j = idx / FD, c = idx % FD;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += F.red[w][j][c];
    st_part(&part[j * (FD + 2) + 2 + c], v);
  }
  if (tid < R) {
    st_part(&part[tid * (FD + 2)], F.m[tid]);
    st_part(&part[tid * (FD + 2) + 1], F.l[tid]);
  }
}

// Waves per SIMD the register allocation targets.
template <int FMT, int KB, int VB, int R, bool RP>
constexpr int waves_target() {
  return (!RP && R <= 4 && (KB == 2 || FMT == KVQ_FMT_TQ)) ? 3 : 2;
}

// Online merge of partials [q0, q1) of one (stream, query head) into (M, L, v): the partials are read
// in chunks of MC, all loads of a chunk at once, with the running maximum and sums rescaled
// between chunks (one memory round trip per chunk).
template <int R>
__device__ __forceinline__ void merge_range(const float* P0, int q0, int q1, int c, float& M, float& L, float& v) {
  constexpr int MC = 16;
  for (int qb = q0; qb < q1; qb += MC) {
    float mq[MC], lq[MC], vq[MC];
#pragma unroll
    for (int k = 0; k < MC; ++k) {  // past the last part: re-read it (no branch between the loads), unused
      const bool in = qb + k < q1;
      const float* pq = P0 + (int64_t)(in ? qb + k : q1 - 1) * R * (FD + 2);
      const float m = ld_part(pq), l = ld_part(pq + 1), x = ld_part(pq + 2 + c);
      mq[k] = in ? m : -INFINITY;
      lq[k] = in ? l : 0.f;
      vq[k] = in ? x : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < MC; ++k) Mn = fmaxf(Mn, mq[k]);
    const float fo = M == -INFINITY ? 0.f : ex2(M - Mn);  // the sums so far are 0 while M = -inf
    L *= fo;
    v *= fo;
#pragma unroll
    for (int k = 0; k < MC; ++k) {
      const float w = mq[k] == -INFINITY ? 0.f : ex2(mq[k] - Mn);
      L = __builtin_fmaf(lq[k], w, L);
      v = __builtin_fmaf(vq[k], w, v);
    }
    M = Mn;
  }
}

// Fixed-order merge of every query head of stream s by its last workgroup: bulk splits, then fp16
// groups, two heads at a time (128 threads, one channel each, per head).  TurboQuant bulk partials live
// in the rotated domain: they are merged first and rotated back (sigma * (c_d * FWHT(acc));
// "TurboQuant KV Cache Compression — Spec", "Optimization: Fused dequant-dot") before the fp16
// groups, which are in the original domain, join the merge.
// The same for every head at once (no rotation): thread (half, c) merges channel c of heads half,
// half + 2, ..., with the loads of all its heads for a chunk of partials issued together, so the
// merge takes one memory round trip per chunk instead of one per head pair.
template <int R>
__device__ void merge_heads(const DecodeArgs& a, int s) {
  constexpr int NH = (R + 1) / 2, MC = NH <= 2 ? 16 : 8;
  const int tid = threadIdx.x, half = tid >> 7, c = tid & (FD - 1);
  const int b = s / a.sh.Hkv, g = s % a.sh.Hkv;
  const float* base = a.ws + (int64_t)s * a.nparts * R * (FD + 2);
  float M[NH], L[NH], v[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) M[h] = -INFINITY, L[h] = 0.f, v[h] = 0.f;
  for (int qb = 0; qb < a.nparts; qb += MC) {
    float mq[NH][MC], lq[NH][MC], vq[NH][MC];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int j = half + 2 * h, jj = j < R ? j : R - 1;
#pragma unroll
      for (int k = 0; k < MC; ++k) {  // past the last part: re-read it (no branch between the loads), unused
        const bool in = qb + k < a.nparts;
        const float* pq = base + (int64_t)(in ? qb + k : a.nparts - 1) * R * (FD + 2) + jj * (FD + 2);
        const float m = ld_part(pq), l = ld_part(pq + 1), x = ld_part(pq + 2 + c);
        mq[h][k] = in ? m : -INFINITY;
        lq[h][k] = in ? l : 0.f;
        vq[h][k] = in ? x : 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float Mn = M[h];
#pragma unroll
      for (int k = 0; k < MC; ++k) Mn = fmaxf(Mn, mq[h][k]);
      const float fo = M[h] == -INFINITY ? 0.f : ex2(M[h] - Mn);  // the sums so far are 0 while M = -inf
      L[h] *= fo;
      v[h] *= fo;
#pragma unroll
      for (int k = 0; k < MC; ++k) {
        const float w = mq[h][k] == -INFINITY ? 0.f : ex2(mq[h][k] - Mn);
        L[h] = __builtin_fmaf(lq[h][k], w, L[h]);
        v[h] = __builtin_fmaf(vq[h][k], w, v[h]);
      }
      M[h] = Mn;
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int j = half + 2 * h;
    if (j < R && c < a.sh.Din) a.out[((int64_t)b * a.sh.Hq + (int64_t)g * R + j) * a.sh.Din + c] = v[h] / L[h];
  }
}

template <int R, bool TQ>
__device__ void merge_stream(const DecodeArgs& a, int s, float (*rot)[FD]) {
  const int tid = threadIdx.x, half = tid >> 7, c = tid & (FD - 1);
  const int b = s / a.sh.Hkv, g = s % a.sh.Hkv;
  for (int j0 = 0; j0 < R; j0 += 2) {
    const int j = j0 + half, jj = j < R ? j : R - 1;
    const float* P0 = a.ws + (int64_t)s * a.nparts * R * (FD + 2) + jj * (FD + 2);
    float M = -INFINITY, L = 0.f, v = 0.f;
    if constexpr (TQ) {
      merge_range<R>(P0, 0, a.splits, c, M, L, v);
      rot[half][c] = v;
      __syncthreads();
      if (c < 64) {  // one wave per head: v = sigma * (c_d * FWHT(v))
        float y0 = rot[half][2 * c], y1 = rot[half][2 * c + 1];
        wave_fwht(y0, y1, FD, c);
        const float cd = (float)(1.0 / __builtin_sqrt((double)FD));
        rot[half][2 * c] = a.lv.tables->signs[2 * c] * (y0 * cd);
        rot[half][2 * c + 1] = a.lv.tables->signs[2 * c + 1] * (y1 * cd);
      }
      __syncthreads();
      v = rot[half][c];
      __syncthreads();
      merge_range<R>(P0, a.splits, a.nparts, c, M, L, v);
    } else {
      merge_range<R>(P0, 0, a.nparts, c, M, L, v);
    }
    if (j < R && c < a.sh.Din) a.out[((int64_t)b * a.sh.Hq + (int64_t)g * R + j) * a.sh.Din + c] = v / L;
  }
}

// RoPE workgroups: the fp16-row groups come first in the grid (each of their rows takes its own
// rotation, which makes them longer than a bulk split's share), then the bulk splits.
template <int FMT, int KB, int VB, int R, bool RP>
__global__ __launch_bounds__(DNT) __attribute__((amdgpu_waves_per_eu(waves_target<FMT, KB, VB, R, RP>())))
void k_decode_fast(DecodeArgs a) {
  __shared__ DecSmem<R, RP> S;
  __shared__ int last;
  const int y = blockIdx.y, nfp = a.nparts - a.splits;
  if (RP ? y >= nfp : y < a.splits) bulk_partial<FMT, KB, VB, R, RP>(a, S.bulk, RP ? y - nfp : y);
  else fp16_partial<R, RP>(a, S.fp, RP ? y : y - a.splits);
  // publish the partial: its stores complete before the arrival is counted
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  const int s = blockIdx.x;
  if (threadIdx.x == 0) {
    const uint32_t n = __hip_atomic_fetch_add(&a.lv.decode_sync[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = n == (uint32_t)(a.nparts - 1);
    if (last) __hip_atomic_store(&a.lv.decode_sync[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  if constexpr (FMT == KVQ_FMT_TQ) merge_stream<R, true>(a, s, S.rot);
  else merge_heads<R>(a, s);
}

template <int FMT, int KB, int VB, bool RP>
hipError_t launch_r(const DecodeArgs& a, hipStream_t st) {
  const int r = a.sh.Hq / a.sh.Hkv;
  const int S = a.sh.B * a.sh.Hkv;
  // parts vary slowest: the (short) fp16 workgroups are dispatched after every bulk split (RoPE:
  // before them)
  dim3 grid(S, a.nparts);
  switch (r) {
    case 1:
      hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 1, RP>), grid, dim3(DNT), 0, st, a);
      break;
    case 2:
      hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 2, RP>), grid, dim3(DNT), 0, st, a);
      break;
    case 4:
      hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 4, RP>), grid, dim3(DNT), 0, st, a);
      break;
    case 8:
      hipLaunchKernelGGL((k_decode_fast<FMT, KB, VB, 8, RP>), grid, dim3(DNT), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int KB, int VB, bool RP>
int slots_r(int r, int per_cu) {
  int nb = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (r) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 1, RP>, DNT, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 2, RP>, DNT, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 4, RP>, DNT, 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_decode_fast<FMT, KB, VB, 8, RP>, DNT, 0); break;
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
  if (sh.rope) {
    if (sh.fmt == KVQ_FMT_KIVI && sh.kb == sh.vb) {
      if (sh.kb == 2) return slots_r<KVQ_FMT_KIVI, 2, 2, true>(r, cus);
      if (sh.kb == 4) return slots_r<KVQ_FMT_KIVI, 4, 4, true>(r, cus);
      if (sh.kb == 8) return slots_r<KVQ_FMT_KIVI, 8, 8, true>(r, cus);
    }
    return 0;
  }
  if (sh.fmt == KVQ_FMT_Q2K) return slots_r<KVQ_FMT_Q2K, 2, 4, false>(r, cus);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 4 && sh.vb == 2) return slots_r<KVQ_FMT_TQ, 4, 2, false>(r, cus);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 4 && sh.vb == 4) return slots_r<KVQ_FMT_TQ, 4, 4, false>(r, cus);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 3 && sh.vb == 2) return slots_r<KVQ_FMT_TQ, 3, 2, false>(r, cus);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 3 && sh.vb == 4) return slots_r<KVQ_FMT_TQ, 3, 4, false>(r, cus);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 4 && sh.vb == 3) return slots_r<KVQ_FMT_TQ, 4, 3, false>(r, cus);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 3 && sh.vb == 3) return slots_r<KVQ_FMT_TQ, 3, 3, false>(r, cus);
  if (sh.fmt == KVQ_FMT_KIVI && sh.kb == sh.vb) {
    if (sh.kb == 2) return slots_r<KVQ_FMT_KIVI, 2, 2, false>(r, cus);
    if (sh.kb == 4) return slots_r<KVQ_FMT_KIVI, 4, 4, false>(r, cus);
    if (sh.kb == 8) return slots_r<KVQ_FMT_KIVI, 8, 8, false>(r, cus);
  }
  return 0;
}

// Rows of fp16 partials one fp16 workgroup of the MFMA kernel scores.
int fast_fp16_rows_per_group() { return FPR; }

// Launches the MFMA kernel and its merge; the host only sets DecodeArgs::fast for shapes it covers.
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  if (sh.D != FD || a.nparts == 0 || sh.in_f32) return hipErrorInvalidValue;
  if (sh.rope) {
    if (sh.fmt == KVQ_FMT_KIVI && sh.kb == sh.vb) {
      if (sh.kb == 2) return launch_r<KVQ_FMT_KIVI, 2, 2, true>(a, st);
      if (sh.kb == 4) return launch_r<KVQ_FMT_KIVI, 4, 4, true>(a, st);
      if (sh.kb == 8) return launch_r<KVQ_FMT_KIVI, 8, 8, true>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (sh.fmt == KVQ_FMT_Q2K) return launch_r<KVQ_FMT_Q2K, 2, 4, false>(a, st);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 4 && sh.vb == 2) return launch_r<KVQ_FMT_TQ, 4, 2, false>(a, st);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 4 && sh.vb == 4) return launch_r<KVQ_FMT_TQ, 4, 4, false>(a, st);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 3 && sh.vb == 2) return launch_r<KVQ_FMT_TQ, 3, 2, false>(a, st);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 3 && sh.vb == 4) return launch_r<KVQ_FMT_TQ, 3, 4, false>(a, st);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 4 && sh.vb == 3) return launch_r<KVQ_FMT_TQ, 4, 3, false>(a, st);
  if (sh.fmt == KVQ_FMT_TQ && sh.kb == 3 && sh.vb == 3) return launch_r<KVQ_FMT_TQ, 3, 3, false>(a, st);
  if (sh.fmt == KVQ_FMT_KIVI && sh.kb == sh.vb) {
    if (sh.kb == 2) return launch_r<KVQ_FMT_KIVI, 2, 2, false>(a, st);
    if (sh.kb == 4) return launch_r<KVQ_FMT_KIVI, 4, 4, false>(a, st);
    if (sh.kb == 8) return launch_r<KVQ_FMT_KIVI, 8, 8, false>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
