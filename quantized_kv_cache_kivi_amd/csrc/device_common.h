// Device helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kvq_internal.h"

namespace kvq {

constexpr float EPS_SCALE = 1e-5f;  // eps of the affine scale (StreamingLLM + KIVI page, "Affine quantisation formula")

__device__ __forceinline__ uint16_t f16_bits(float x) {
  const _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even, subnormals kept
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// One input element (fp16 or fp32 as the caller hands it), as fp32.
__device__ __forceinline__ float ld_in(const void* p, int64_t i, int in_f32) {
  return in_f32 ? static_cast<const float*>(p)[i] : (float)static_cast<const _Float16*>(p)[i];
}
// The fp16 bit pattern of an input element (fp16 input is copied, fp32 input rounded to nearest even).
__device__ __forceinline__ uint16_t ld_in_f16(const void* p, int64_t i, int in_f32) {
  return in_f32 ? f16_bits(static_cast<const float*>(p)[i]) : static_cast<const uint16_t*>(p)[i];
}

// Word-interleaved packing: code k of a 32-bit word of b-bit codes sits at bit 16*(k%2) + b*(k/2).
__device__ __forceinline__ int code_shift(int k, int b) { return 16 * (k & 1) + b * (k >> 1); }

// Byte offset of the word holding K code (t, c) inside the K section, and its in-word index.
__device__ __forceinline__ void k_code_pos(int t, int c, int D, int b, int* word, int* k) {
  const int per = 32 / b;
  *word = t * (D * b / 32) + c / per;
  *k = c % per;
}
// V tile order: token t, channel c -> chunk 16*kg + i, sequence index 8*mu + e.
__device__ __forceinline__ void v_code_pos(int t, int c, int D, int b, int* word, int* k) {
  const int kg = (t & 15) >> 2, e = ((t >> 4) << 2) | (t & 3);
  const int i = c & 15, mu = c >> 4;
  const int q = 16 * kg + i, s = 8 * mu + e, per = 32 / b;
  *word = q * (D * b / 64) + s / per;
  *k = s % per;
}
// Index (in fp16 units) of the V scale or zero of token t, channel group g inside its section:
// [t / 2][g][t % 2], so both tokens of a pair sit side by side for every group.
__device__ __forceinline__ int v_meta_idx(int t, int g, int ng) { return (t >> 1) * 2 * ng + 2 * g + (t & 1); }

// Dense 3-bit stream ("TurboQuant KV Cache Compression — Spec", "Step 3: Packing", 8 values in 3
// bytes): code i of a section's sequence at bits [3i, 3i + 3), least significant bit first; the K
// sequence is row-major token rows, the V sequence the 64 chunks of the tile order one after another.
__device__ __forceinline__ int k_bit3(int t, int c, int D) { return 3 * (t * D + c); }
__device__ __forceinline__ int v_bit3(int t, int c, int D) {
  const int kg = (t & 15) >> 2, e = ((t >> 4) << 2) | (t & 3);
  return 3 * ((16 * kg + (c & 15)) * (D / 2) + 8 * (c >> 4) + e);
}
// A code of a dense stream: one word, or two when it straddles a word boundary (the next word is
// inside the section: the code ends there).
__device__ __forceinline__ uint32_t code3_at(const uint8_t* sec, int bit) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(sec);
  const int wi = bit >> 5, o = bit & 31;
  uint32_t x = w[wi] >> o;
  if (o > 29) x |= w[wi + 1] << (32 - o);
  return x & 7u;
}
// Bits of code `code` (3 bits at stream bit `bit`) that fall in word `wi` of the stream, in place.
__device__ __forceinline__ uint32_t code3_in_word(uint32_t code, int bit, int wi) {
  const int s = bit - 32 * wi;  // -2 .. 31
  return s >= 0 ? code << s : code >> (-s);
}

// Token of element e of V token group kg.
__device__ __forceinline__ int v_tok(int kg, int e) { return 16 * (e >> 2) + 4 * kg + (e & 3); }

// RoPE on read ("StreamingLLM + KIVI", "RoPE caveat"): the index of position p in the compressed
// cache, i.e. the number of valid positions (committed sinks, [lo, P)) before p.
__device__ __forceinline__ int cache_index(const int* sinks, int nsinks, int64_t lo, int64_t p) {
  const int64_t lim = p < lo ? p : lo;
  int n = 0;
  for (int q = 0; q < nsinks; ++q) n += sinks[q] < lim ? 1 : 0;
  return n + (int)(p > lo ? p - lo : 0);
}

// cos and sin of the exact angle idx * th (|idx| < 2^24, so fp32(idx) is exact): a = fp32(idx * th)
// plus its exact residual e = idx * th - a (one fma); cos(a + e) and sin(a + e) from sincosf(a) and
// the Taylor terms of e (|e| < 2^-5: error below 1e-7), or sincosf(e) for larger e (angles above 2^19).
__device__ __forceinline__ void rope_cs(int idx, float th, float& cs, float& sn) {
  const float x = (float)idx, a = x * th, e = __builtin_fmaf(x, th, -a);
  float sa, ca, se, ce;
  sincosf(a, &sa, &ca);
  if (fabsf(e) < 0.03125f) {
    const float e2 = e * e;
    ce = __builtin_fmaf(-0.5f, e2, 1.f);
    se = __builtin_fmaf(e * e2, -1.f / 6.f, e);
  } else {
    sincosf(e, &se, &ce);
  }
  cs = __builtin_fmaf(ca, ce, -sa * se);
  sn = __builtin_fmaf(sa, ce, ca * se);
}

// Rotate-half RoPE of channel c given its partner channel (c +- D/2): x' = x cos - y sin for
// c < D/2, x' = x cos + y sin above, with the angle idx * theta_{c mod D/2}.
__device__ __forceinline__ float rope_val(float x, float partner, int c, int D, int idx, const float* inv) {
  const int h = D >> 1, f = c < h ? c : c - h;
  float sn, cs;
  rope_cs(idx, inv[f], cs, sn);
  return c < h ? x * cs - partner * sn : x * cs + partner * sn;
}

// Workgroup barrier that orders LDS only: outstanding global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum_xor(float a, int first_off) {
  for (int off = first_off; off >= 1; off >>= 1) a = a + __shfl_xor(a, off);
  return a;
}

// In-wave fast Walsh-Hadamard transform of a D-vector held two per lane
// (lane l holds elements 2l, 2l+1; lanes >= D/2 carry don't-care values).
// Stages len = 1, 2, ..., D/2: (u, v) -> (u + v, u - v) with u the lower element
// ("TurboQuant KV Cache Compression — Spec", "Hadamard Transform Detail").
__device__ __forceinline__ void wave_fwht(float& y0, float& y1, int D, int lane) {
  const float a = y0 + y1, b = y0 - y1;
  y0 = a;
  y1 = b;
  for (int len = 2; len < D; len <<= 1) {
    const int m = len >> 1;
    const float p0 = __shfl_xor(y0, m), p1 = __shfl_xor(y1, m);
    if (lane & m) {
      y0 = p0 - y0;
      y1 = p1 - y1;
    } else {
      y0 = y0 + p0;
      y1 = y1 + p1;
    }
  }
}

// Canonical fp32 sum of squares of a D-vector held two per lane: pair products,
// then a butterfly over lane offsets D/4, D/8, ..., 1 (every lane ends with the sum).
__device__ __forceinline__ float wave_sumsq(float y0, float y1, int D) {
  const float p = y0 * y0;
  const float q = y1 * y1;
  return wave_sum_xor(p + q, D >> 2);
}

// A row of up to MD channels (MD = 128 or 256) held by one wave, MD / 64 values per lane: y[2h + e]
// is channel 128h + 2l + e of lane l (h = 1 only for rows of 256 channels; a row of D <= 128
// channels uses y[0], y[1] of lanes l < D/2).
__device__ __forceinline__ int row_chan(int lane, int k) { return 128 * (k >> 1) + 2 * lane + (k & 1); }

// The D-point transform (D a power of two, 2 <= D <= MD) of such a row, stages len = 1, 2, ..., D/2
// as in wave_fwht.  For 256 channels the stages below 128 pair channels inside one 128-channel half
// (each half transforms alone) and the last stage pairs channel c with c + 128, in the lane.
template <int MD>
__device__ __forceinline__ void row_fwht(float (&y)[MD / 64], int D, int lane) {
  if constexpr (MD > 128) {
    if (D > 128) {
      wave_fwht(y[0], y[1], 128, lane);
      wave_fwht(y[2], y[3], 128, lane);
      const float a0 = y[0] + y[2], a1 = y[1] + y[3], b0 = y[0] - y[2], b1 = y[1] - y[3];
      y[0] = a0;
      y[1] = a1;
      y[2] = b0;
      y[3] = b1;
      return;
    }
  }
  wave_fwht(y[0], y[1], D, lane);
}

// Canonical fp32 sum of squares of such a row (the tree of wave_sumsq).  For 256 channels the pair
// sums a_l (l < 128) sit two per lane, a_l and a_{l+64}, so the first halving is the in-lane add.
template <int MD>
__device__ __forceinline__ float row_sumsq(const float (&y)[MD / 64], int D) {
  if constexpr (MD > 128) {
    if (D > 128) {
      const float p0 = y[0] * y[0], q0 = y[1] * y[1], p1 = y[2] * y[2], q1 = y[3] * y[3];
      const float lo = p0 + q0, hi = p1 + q1;
      return wave_sum_xor(lo + hi, 32);
    }
  }
  return wave_sumsq(y[0], y[1], D);
}

}  // namespace kvq
