// Append / quantize kernels: whole blocks of a chunk, one wave per (block, stream); partial
// blocks, one workgroup per (block, stream, 32-channel group); TurboQuant and other shapes, one
// workgroup per (block, stream).
//
// Follows "StreamingLLM + KIVI — long-context decode without growing the KV
// cache" ("KIVI", "Affine quantisation formula": K per channel, V per token,
// scale = max(eps, range/levels), zero = min; "Caveats": scales frozen at
// group boundaries), the q2k pull-request page ("Summary": K 2-bit per channel
// with a Gaussian Lloyd-Max grid over block RMS, V 4-bit per token with one
// fp16 scale per 32 values), the TurboQuant spec ("As-Built Notes", "Step 1",
// "Step 2", "Step 3") and "KVSink-Adapted Sink Protection" ("How it works":
// sink rows stored fp16, excluded from calibration).
//
// Every code-deciding expression is one rounded fp32 operation at a time
// (the library is built with -ffp-contract=off), with correctly rounded
// division and square root and rintf (round half to even).
#include "device_common.h"

namespace kvq {
namespace {

constexpr int NT = 256;

// min / max over the 32 lanes of a half-wave (every lane of the half ends with the result)
__device__ __forceinline__ float half_min(float x) {
  for (int off = 1; off < 32; off <<= 1) x = fminf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float half_max(float x) {
  for (int off = 1; off < 32; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Thread layout: channel c = tid % D and row group rg = tid / D hold rows t = rg + RG*i of the
// block (RG = 256 / D row groups, i < 32 / RG), in registers.  The 32 channels of a V group
// are the 32 lanes of one half-wave.  MD: the widest stored row the instance takes (128, or 256
// for TurboQuant rows of head_dim 160).
template <int MD>
__global__ __launch_bounds__(NT) void k_append(AppendArgs a) {
  constexpr int XP = MD + 1;  // padded LDS row (bank spread for per-row loops)
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int D = sh.D, tid = threadIdx.x;
  const int s = blockIdx.y, b = s / sh.Hkv, h = s % sh.Hkv;
  const int64_t beta = a.blk0 + blockIdx.x;
  const int64_t base = beta * G;
  const int tnew0 = (int)(a.P > base ? a.P - base : 0);                    // first row new in this call
  const int tend = (int)((a.P + a.n - base) < G ? (a.P + a.n - base) : G);  // rows present after it
  const bool tq = sh.fmt == KVQ_FMT_TQ;
  uint8_t* rec = lv.bulk + ((int64_t)s * lv.cap_b + beta % lv.cap_b) * lv.rec;
  const int64_t in_row0 = ((int64_t)b * sh.Hkv + h) * a.n;  // row index base of this stream in the chunk
  const int RG = NT / D, c = tid % D, rg = tid / D;

  __shared__ float xk[G][XP];          // K rows (q2k sum of squares, TurboQuant rows)
  __shared__ float xv[G][XP];          // V rows (TurboQuant rows)
  __shared__ alignas(16) uint8_t ck[G][MD];   // K codes [token][channel]
  __shared__ alignas(16) uint8_t cvt[MD][G];  // V codes [channel][token]
  __shared__ float red0[NT / 32][MD], red1[NT / 32][MD];  // per row group partials
  __shared__ int sink_slot[G];
  __shared__ uint32_t smask_s;
  __shared__ uint16_t vmeta_s[G][4], vmeta_z[G][4];
  __shared__ float knorm[G], vnorm[G];

  // Every global load of the kernel is issued before any of them is used (one memory round trip
  // instead of one per loop iteration): the committed sink list, this thread's elements of the
  // block's rows (new rows from the chunk, earlier rows of an open K block from staging) and the
  // V code words that hold bits of rows appended by earlier calls.
  constexpr int PER = G * MD / NT;  // row elements per thread (at most)
  const int nper = G * D / NT;         // row elements per thread
  const int ng = D / 32;
  const int wpc = D * sh.vb / 64;      // words per V code chunk (word-interleaved widths)
  const int nvw = D * sh.vb;           // words of the V code section
  int sp[MAX_SINK];
  int scount = 0;
  if (tid < G && sh.n_sink > 0 && sh.sink_mode == KVQ_SINK_TOPK) {
    scount = lv.sink_count[b];
#pragma unroll
    for (int i = 0; i < MAX_SINK; ++i) sp[i] = i < sh.n_sink ? lv.sink_pos[b * sh.n_sink + i] : -1;
  }
  float kx[PER], vx[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int t = rg + RG * i;
    kx[i] = 0.f;
    vx[i] = 0.f;
    if (i < nper && t < tend) {
      if (t >= tnew0) {
        if (c < sh.Din) {  // input rows hold Din channels; the rest of a padded row is zero
          const int64_t gi = (in_row0 + (base + t - a.P)) * sh.Din + c;
          kx[i] = ld_in(a.k, gi, sh.in_f32);
          vx[i] = ld_in(a.v, gi, sh.in_f32);
        }
      } else if (!tq) {
        kx[i] = ld_in(lv.staging, ((int64_t)s * G + t) * D + c, sh.in_f32);
      }
    }
  }
  constexpr int VW = 64 * (MD * 8 / 64) / NT;  // V code words per thread (at most)
  uint32_t oldv[VW];
  {
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(rec + lv.v_codes);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      const int idx = tid + i * NT;
      oldv[i] = (tnew0 > 0 && idx < nvw) ? vw[idx] : 0u;
    }
  }

  // 1. sink membership of the block's rows (slots, and a bit mask of sink rows)
  if (tid < 64) {
    int slot = -1;
    if (tid < G && tid < tend && sh.n_sink > 0) {
      const int64_t p = base + tid;
      if (sh.sink_mode == KVQ_SINK_FIRST_N) {
        if (p < sh.n_sink) slot = (int)p;
      } else if (sh.sink_mode == KVQ_SINK_TOPK) {
#pragma unroll
        for (int i = 0; i < MAX_SINK; ++i)
          if (i < scount && sp[i] == p) slot = i;
      }
    }
    const uint64_t m = __ballot(slot >= 0);
    if (tid < G) {
      sink_slot[tid] = slot;
      knorm[tid] = 0.f;
      vnorm[tid] = 0.f;
    }
    if (tid == 0) smask_s = (uint32_t)m;
  }
  // 2. rows to LDS (the formats that read them across threads), codes cleared
  if (tq || sh.fmt == KVQ_FMT_Q2K) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i < nper) {
        xk[rg + RG * i][c] = kx[i];
        xv[rg + RG * i][c] = vx[i];
      }
  }
  for (int idx = tid; idx < G * MD / 16; idx += NT) {
    reinterpret_cast<uint4*>(&ck[0][0])[idx] = uint4{0, 0, 0, 0};
    reinterpret_cast<uint4*>(&cvt[0][0])[idx] = uint4{0, 0, 0, 0};
  }
  __syncthreads();
  const uint32_t smask = smask_s;
  auto calib = [&](int t) { return t < tend && !((smask >> t) & 1u); };  // present, not a sink

  // 3. K of a block format: per channel over the block's calibration rows, codes of every row
  if (!tq) {
    uint8_t* km = rec + lv.k_meta;
    float sf = 0.f, zf = 0.f;
    if (sh.fmt == KVQ_FMT_KIVI) {
      float mn = INFINITY, mx = -INFINITY, any = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i < nper && calib(rg + RG * i)) {
          mn = fminf(mn, kx[i]);
          mx = fmaxf(mx, kx[i]);
          any = 1.f;
        }
      red0[rg][c] = mn;
      red1[rg][c] = any > 0.f ? mx : -INFINITY;
      __syncthreads();
      mn = INFINITY;
      mx = -INFINITY;
      for (int q = 0; q < RG; ++q) {
        mn = fminf(mn, red0[q][c]);
        mx = fmaxf(mx, red1[q][c]);
      }
      if (mx == -INFINITY) mn = mx = 0.f;  // no calibration row
      mn = mn + 0.0f;
      mx = mx + 0.0f;
      const float L = (float)((1 << sh.kb) - 1);
      const float s32 = fmaxf(EPS_SCALE, (mx - mn) / L);
      const uint16_t s16 = f16_bits(s32), z16 = f16_bits(mn);
      if (rg == 0) {
        reinterpret_cast<uint16_t*>(km)[c] = s16;
        reinterpret_cast<uint16_t*>(km)[D + c] = z16;
      }
      sf = f16_val(s16);
      zf = f16_val(z16);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int t = rg + RG * i;
        if (i < nper && calib(t)) {
          const float u = rintf((kx[i] - zf) / sf);
          ck[t][c] = (uint8_t)fminf(fmaxf(u, 0.f), L);
        }
      }
    } else {  // Q2K: block RMS summed in token order by one thread per channel
      if (rg == 0) {
        float ss = 0.f;
        int n = 0;
        for (int t = 0; t < tend; ++t)
          if (calib(t)) {
            ss = ss + xk[t][c] * xk[t][c];
            ++n;
          }
        const float r32 = n > 0 ? fmaxf(EPS_SCALE, sqrtf(ss / (float)n)) : EPS_SCALE;
        const uint16_t r16 = f16_bits(r32);
        reinterpret_cast<uint16_t*>(km)[c] = r16;
        red0[0][c] = f16_val(r16);
      }
      __syncthreads();
      const float rf = red0[0][c];
      const float th0 = lv.tables->q2k_thr[0], th1 = lv.tables->q2k_thr[1], th2 = lv.tables->q2k_thr[2];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int t = rg + RG * i;
        if (i < nper && calib(t)) {
          const float x = kx[i] / rf;
          ck[t][c] = (uint8_t)((x >= th0) + (x >= th1) + (x >= th2));
        }
      }
    }
    // 3b. V of the new rows: per token and 32-channel group (one half-wave per group)
    const int g = c >> 5;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = rg + RG * i;
      if (i >= nper || t < tnew0 || t >= tend) continue;  // uniform over the half-wave
      if ((smask >> t) & 1u) {
        if ((c & 31) == 0) {
          vmeta_s[t][g] = 0;
          vmeta_z[t][g] = 0;
        }
        continue;
      }
      if (sh.fmt == KVQ_FMT_KIVI) {
        const float mn = half_min(vx[i]) + 0.0f, mx = half_max(vx[i]) + 0.0f;
        const float L = (float)((1 << sh.vb) - 1);
        const float s32 = fmaxf(EPS_SCALE, (mx - mn) / L);
        const uint16_t s16 = f16_bits(s32), z16 = f16_bits(mn);
        const float vsf = f16_val(s16), vzf = f16_val(z16);
        const float u = rintf((vx[i] - vzf) / vsf);
        cvt[c][t] = (uint8_t)fminf(fmaxf(u, 0.f), L);
        if ((c & 31) == 0) {
          vmeta_s[t][g] = s16;
          vmeta_z[t][g] = z16;
        }
      } else {  // Q2K: symmetric 4-bit, s = absmax / 7
        const float am = half_max(fabsf(vx[i])) + 0.0f;
        const uint16_t s16 = f16_bits(fmaxf(EPS_SCALE, am / 7.0f));
        const float vsf = f16_val(s16);
        const float q = fminf(fmaxf(rintf(vx[i] / vsf), -8.f), 7.f);
        cvt[c][t] = (uint8_t)(q + 8.f);
        if ((c & 31) == 0) {
          vmeta_s[t][g] = s16;
          vmeta_z[t][g] = 0;
        }
      }
    }
  } else {
    // TQ rows (K and V) and the rotation: one wave per row, MD / 64 channels per lane
    constexpr int NK = MD / 64;
    const int lane = tid & 63, w = tid >> 6;
    const float cd = (float)(1.0 / __builtin_sqrt((double)D));
    const Tables* T = lv.tables;
    for (int t = tnew0 + w; t < tend; t += NT / 64) {
      if (sink_slot[t] >= 0) continue;
      for (int which = 0; which < 2; ++which) {
        float (*X)[XP] = which ? xv : xk;
        const int nb = which ? sh.vb : sh.kb;
        const float* bnd = which ? T->v_bnd : T->k_bnd;
        float y[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const int cc = row_chan(lane, k);
          y[k] = cc < D ? X[t][cc] * T->signs[cc] : 0.f;
        }
        row_fwht<MD>(y, D, lane);
#pragma unroll
        for (int k = 0; k < NK; ++k) y[k] = y[k] * cd;
        const float nrm = sqrtf(row_sumsq<MD>(y, D));
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const int cc = row_chan(lane, k);
          const float tv = nrm > 0.f ? y[k] / nrm : 0.f;
          int u = 0;
          for (int j = 0; j < (1 << nb) - 1; ++j) u += tv >= bnd[j];
          if (cc < D) {
            if (which) cvt[cc][t] = (uint8_t)u;
            else ck[t][cc] = (uint8_t)u;
          }
        }
        if (lane == 0) (which ? vnorm : knorm)[t] = nrm;
      }
    }
  }
  __syncthreads();

  // 4. K codes: token rows, word-interleaved, from one vector LDS read of the word's codes.  Block
  //    formats rewrite the whole block (rows not present are 0); TQ writes its new rows (and
  //    clears the rest of a block it opens).
  {
    const int wpr = D * sh.kb / 32, per = 32 / sh.kb;
    uint32_t* kw = reinterpret_cast<uint32_t*>(rec + lv.k_codes);
    for (int idx = tid; idx < G * wpr; idx += NT) {
      const int t = idx / wpr, w = idx % wpr;
      if (tq && !((t >= tnew0 && t < tend) || (tnew0 == 0 && t >= tend))) continue;
      if (sh.kb == 3) {  // dense 3-bit stream: rows are whole words, a word holds codes c0 .. c1 of row t
        uint32_t word = 0;
        const int c0 = (32 * w) / 3, c1 = min(D - 1, (32 * w + 31) / 3);
        for (int cc = c0; cc <= c1; ++cc) word |= code3_in_word(ck[t][cc], 3 * cc, w);
        kw[idx] = word;
        continue;
      }
      uint32_t cw[4] = {0, 0, 0, 0};  // the word's codes, one byte each
      const uint8_t* src = &ck[t][w * per];
      if (per == 16) {
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        cw[0] = x.x, cw[1] = x.y, cw[2] = x.z, cw[3] = x.w;
      } else if (per == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(src);
        cw[0] = x.x, cw[1] = x.y;
      } else {
        cw[0] = *reinterpret_cast<const uint32_t*>(src);
      }
      uint32_t word = 0;
      for (int k = 0; k < per; ++k) word |= ((cw[k >> 2] >> (8 * (k & 3))) & 0xFFu) << code_shift(k, sh.kb);
      kw[idx] = word;
    }
  }
  // 5. V codes: channel tiles; bits of rows appended earlier are kept, others rewritten.  The
  //    tokens T(kg, e) of a channel for e = 0..3 and e = 4..7 are two 4-byte runs of cvt.
  {
    const int per = 32 / sh.vb;
    uint32_t* vw = reinterpret_cast<uint32_t*>(rec + lv.v_codes);
    const uint32_t m1 = (1u << sh.vb) - 1;
#pragma unroll
    for (int ii = 0; ii < VW; ++ii) {
      const int idx = tid + ii * NT;
      if (idx >= nvw) break;
      if (sh.vb == 3) {  // dense 3-bit stream: codes g0 .. g1 of the tile sequence touch word idx
        const uint32_t old = oldv[ii];
        uint32_t word = 0;
        const int half = D / 2, g0 = (32 * idx) / 3, g1 = min(64 * half - 1, (32 * idx + 31) / 3);
        for (int g = g0; g <= g1; ++g) {
          const int q = g / half, k = g % half, kg = q >> 4, i = q & 15;
          const int t = v_tok(kg, k & 7), cc = 16 * (k >> 3) + i;
          if (t < tnew0) word |= old & code3_in_word(7u, 3 * g, idx);
          else if (t < tend) word |= code3_in_word(cvt[cc][t], 3 * g, idx);
        }
        vw[idx] = word;
        continue;
      }
      const int q = idx / wpc, w = idx % wpc, kg = q >> 4, i = q & 15;
      const uint32_t old = oldv[ii];
      uint32_t word = 0;
      uint32_t run[2] = {0, 0};
      int mu_run = -1;
      for (int k = 0; k < per; ++k) {
        const int sq = w * per + k, mu = sq >> 3, e = sq & 7;
        const int t = v_tok(kg, e), sh_ = code_shift(k, sh.vb);
        if (mu != mu_run) {
          const int cc = 16 * mu + i;
          run[0] = *reinterpret_cast<const uint32_t*>(&cvt[cc][4 * kg]);
          run[1] = *reinterpret_cast<const uint32_t*>(&cvt[cc][16 + 4 * kg]);
          mu_run = mu;
        }
        if (t < tnew0) word |= old & (m1 << sh_);
        else if (t < tend) word |= ((run[e >> 2] >> (8 * (e & 3))) & 0xFFu) << sh_;
      }
      vw[idx] = word;
    }
  }
  // 6. metadata of rows from tnew0 on (rows past tend cleared)
  {
    if (tq) {
      float* kn = reinterpret_cast<float*>(rec + lv.k_meta);
      float* vn = reinterpret_cast<float*>(rec + lv.v_meta);
      if (tid >= tnew0 && tid < G) {
        kn[tid] = tid < tend ? knorm[tid] : 0.f;
        vn[tid] = tid < tend ? vnorm[tid] : 0.f;
      }
    } else {
      uint16_t* vm = reinterpret_cast<uint16_t*>(rec + lv.v_meta);
      for (int idx = tid; idx < G * ng; idx += NT) {
        const int t = idx / ng, g = idx % ng, mi = v_meta_idx(t, g, ng);
        if (t < tnew0) continue;
        vm[mi] = t < tend ? vmeta_s[t][g] : 0;
        if (sh.fmt == KVQ_FMT_KIVI) vm[G * ng + mi] = t < tend ? vmeta_z[t][g] : 0;
      }
    }
  }
  // 7. staging of an open block (raw input rows; block formats only)
  if (!tq && tend < G) {
    for (int idx = tid; idx < (tend - tnew0) * D; idx += NT) {
      const int t = tnew0 + idx / D, cc = idx % D;
      const int64_t gi = (in_row0 + (base + t - a.P)) * D + cc;
      const int64_t so = ((int64_t)s * G + t) * D + cc;
      if (sh.in_f32) reinterpret_cast<float*>(lv.staging)[so] = static_cast<const float*>(a.k)[gi];
      else reinterpret_cast<uint16_t*>(lv.staging)[so] = static_cast<const uint16_t*>(a.k)[gi];
    }
  }
  // 8. fp16 window ring: rows p in [max(P, P+n-R), P+n)
  if (sh.R > 0) {
    const int64_t wlo = (a.P + a.n - sh.R) > a.P ? (a.P + a.n - sh.R) : a.P;
    for (int idx = tid; idx < (tend - tnew0) * D; idx += NT) {
      const int t = tnew0 + idx / D, cc = idx % D;
      const int64_t p = base + t;
      if (p < wlo) continue;
      const int64_t gi = (in_row0 + (p - a.P)) * sh.Din + cc;
      const int64_t wo = ((int64_t)s * sh.R + p % sh.R) * D + cc;
      lv.win_k[wo] = cc < sh.Din ? ld_in_f16(a.k, gi, sh.in_f32) : (uint16_t)0;
      lv.win_v[wo] = cc < sh.Din ? ld_in_f16(a.v, gi, sh.in_f32) : (uint16_t)0;
    }
  }
  // 9. fp16 sink pool
  if (sh.n_sink > 0) {
    for (int idx = tid; idx < (tend - tnew0) * D; idx += NT) {
      const int t = tnew0 + idx / D, cc = idx % D;
      const int slot = sink_slot[t];
      if (slot < 0) continue;
      const int64_t gi = (in_row0 + (base + t - a.P)) * sh.Din + cc;
      const int64_t so = ((int64_t)s * sh.n_sink + slot) * D + cc;
      lv.sink_k[so] = cc < sh.Din ? ld_in_f16(a.k, gi, sh.in_f32) : (uint16_t)0;
      lv.sink_v[so] = cc < sh.Din ? ld_in_f16(a.v, gi, sh.in_f32) : (uint16_t)0;
    }
    // first-N commits: positions and count, by one workgroup per batch element
    if (sh.sink_mode == KVQ_SINK_FIRST_N && h == 0 && blockIdx.x == 0) {
      const int64_t P1 = a.P + a.n;
      if (tid < sh.n_sink && tid < P1) lv.sink_pos[b * sh.n_sink + tid] = tid;
      if (tid == 0) lv.sink_count[b] = (int)(P1 < sh.n_sink ? P1 : sh.n_sink);
    }
  }
}

// Block formats (KIVI, q2k), one workgroup per (touched block, stream, 32-channel group).
//
// Everything these formats compute is independent across 32-channel groups: K is calibrated per
// channel, V per (token, 32-channel group), a K code word holds 32/KB channels of one row and a V
// code word holds the codes of one 32-channel group's channel tiles (the group's VB/2 words of
// every 64-byte-aligned chunk), so a group is a complete unit of work.  Four times the workgroups
// of one per (block, stream) keep a one-row append (a decode step) short.  Thread (cl, rg): channel
// 32 * group + cl, rows rg + 8 i.  Arithmetic per code is the same as in k_append.
template <int FMT, int KB, int VB>
__global__ __launch_bounds__(NT) void k_append_cs(AppendArgs a) {
  constexpr bool Q2K = FMT == KVQ_FMT_Q2K;
  constexpr int RGS = NT / 32;   // row groups
  constexpr int PR = G / RGS;    // rows per thread
  constexpr int KPW = 32 / KB;   // K codes per word
  constexpr int VPW = 32 / VB;   // V codes per word
  constexpr int VWG = VB / 2;    // V words of one group per chunk
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int D = sh.D, tid = threadIdx.x, cl = tid & 31, rg = tid >> 5;
  const int grp = blockIdx.z, c = 32 * grp + cl;
  const int s = blockIdx.y, b = s / sh.Hkv, h = s % sh.Hkv;
  const int64_t beta = a.blk0 + blockIdx.x;
  const int64_t base = beta * G;
  const int tnew0 = (int)(a.P > base ? a.P - base : 0);
  const int tend = (int)((a.P + a.n - base) < G ? (a.P + a.n - base) : G);
  uint8_t* rec = lv.bulk + ((int64_t)s * lv.cap_b + beta % lv.cap_b) * lv.rec;
  const int64_t in_row0 = ((int64_t)b * sh.Hkv + h) * a.n;
  const int wpc = D * VB / 64;  // V words per chunk
  // a.defer (block formats, fp16 input, fp16 window of >= 32 rows): a block is quantized once, when
  // its last row arrives; a block left open by this call only gets its rows copied (and a zero
  // record when this call opens it), and a block completed by this call takes the V of its earlier
  // rows from the fp16 window, where all of them still are.  Otherwise an open block is re-quantized
  // on every call and the V codes of earlier rows are kept.
  const bool open_mode = a.defer && tend < G;
  const int vt0 = a.defer ? 0 : tnew0;  // first row whose V this call quantizes

  __shared__ float xk[G][33];               // q2k: rows for the per-channel sum of squares
  __shared__ alignas(16) uint8_t ck[G][32];   // K codes [token][channel of the group]
  __shared__ alignas(16) uint8_t cvt[32][G];  // V codes [channel of the group][token]
  __shared__ float red0[RGS][32], red1[RGS][32];
  __shared__ int sink_slot[G];
  __shared__ uint32_t smask_s;
  __shared__ uint16_t vms[G], vmz[G];

  // every global load first: sink list, this thread's rows, the group's old V words
  int sp[MAX_SINK];
  int scount = 0;
  if (tid < G && sh.n_sink > 0 && sh.sink_mode == KVQ_SINK_TOPK) {
    scount = lv.sink_count[b];
#pragma unroll
    for (int i = 0; i < MAX_SINK; ++i) sp[i] = i < sh.n_sink ? lv.sink_pos[b * sh.n_sink + i] : -1;
  }
  float kx[PR], vx[PR];
#pragma unroll
  for (int i = 0; i < PR; ++i) {
    const int t = rg + RGS * i;
    kx[i] = 0.f;
    vx[i] = 0.f;
    if (t < tend) {
      if (t >= tnew0) {
        const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
        kx[i] = ld_in(a.k, gi, sh.in_f32);
        vx[i] = ld_in(a.v, gi, sh.in_f32);
      } else if (!open_mode) {
        kx[i] = ld_in(lv.staging, ((int64_t)s * G + t) * D + c, sh.in_f32);
        if (a.defer) vx[i] = f16_val(lv.win_v[((int64_t)s * sh.R + (base + t) % sh.R) * D + c]);
      }
    }
  }
  uint32_t oldv = 0;  // word (chunk tid / VWG, group word tid % VWG), for tid < 64 * VWG
  const uint32_t* vwords = reinterpret_cast<const uint32_t*>(rec + lv.v_codes);
  if (vt0 > 0 && tid < 64 * VWG) oldv = vwords[(tid / VWG) * wpc + grp * VWG + tid % VWG];

  // 1. sink membership of the block's rows
  if (tid < 64) {
    int slot = -1;
    if (tid < G && tid < tend && sh.n_sink > 0) {
      const int64_t p = base + tid;
      if (sh.sink_mode == KVQ_SINK_FIRST_N) {
        if (p < sh.n_sink) slot = (int)p;
      } else if (sh.sink_mode == KVQ_SINK_TOPK) {
#pragma unroll
        for (int i = 0; i < MAX_SINK; ++i)
          if (i < scount && sp[i] == p) slot = i;
      }
    }
    const uint64_t m = __ballot(slot >= 0);
    if (tid < G) {
      sink_slot[tid] = slot;
      vms[tid] = 0;
      vmz[tid] = 0;
    }
    if (tid == 0) smask_s = (uint32_t)m;
  }
  // 2. codes cleared; q2k rows to LDS
  reinterpret_cast<uint32_t*>(&ck[0][0])[tid] = 0u;
  reinterpret_cast<uint32_t*>(&cvt[0][0])[tid] = 0u;
  if constexpr (Q2K) {
#pragma unroll
    for (int i = 0; i < PR; ++i) xk[rg + RGS * i][cl] = kx[i];
  }
  __syncthreads();
  const uint32_t smask = smask_s;
  auto calib = [&](int t) { return t < tend && !((smask >> t) & 1u); };  // present, not a sink

  if (open_mode) {
    // a block opened by this call and left open: its record is zero until it completes (this
    // group's quarter of the record words)
    if (tnew0 == 0) {
      const int words = (int)(lv.rec / 4), per = (words + 3) / 4;
      uint32_t* rw = reinterpret_cast<uint32_t*>(rec);
      for (int i = grp * per + tid; i < min(words, (grp + 1) * per); i += NT) rw[i] = 0u;
    }
  } else {
  // 3. K: per channel over the block's calibration rows, codes of every row
  uint8_t* km = rec + lv.k_meta;
  if constexpr (!Q2K) {
    float mn = INFINITY, mx = -INFINITY, any = 0.f;
#pragma unroll
    for (int i = 0; i < PR; ++i)
      if (calib(rg + RGS * i)) {
        mn = fminf(mn, kx[i]);
        mx = fmaxf(mx, kx[i]);
        any = 1.f;
      }
    red0[rg][cl] = mn;
    red1[rg][cl] = any > 0.f ? mx : -INFINITY;
    __syncthreads();
    mn = INFINITY;
    mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < RGS; ++q) {
      mn = fminf(mn, red0[q][cl]);
      mx = fmaxf(mx, red1[q][cl]);
    }
    if (mx == -INFINITY) mn = mx = 0.f;  // no calibration row
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    constexpr float L = (float)((1 << KB) - 1);
    const float s32 = fmaxf(EPS_SCALE, (mx - mn) / L);
    const uint16_t s16 = f16_bits(s32), z16 = f16_bits(mn);
    if (rg == 0) {
      reinterpret_cast<uint16_t*>(km)[c] = s16;
      reinterpret_cast<uint16_t*>(km)[D + c] = z16;
    }
    const float sf = f16_val(s16), zf = f16_val(z16);
#pragma unroll
    for (int i = 0; i < PR; ++i) {
      const int t = rg + RGS * i;
      if (calib(t)) {
        const float u = rintf((kx[i] - zf) / sf);
        ck[t][cl] = (uint8_t)fminf(fmaxf(u, 0.f), L);
      }
    }
  } else {  // block RMS summed in token order by one thread per channel
    if (rg == 0) {
      float ss = 0.f;
      int n = 0;
      for (int t = 0; t < tend; ++t)
        if (calib(t)) {
          ss = ss + xk[t][cl] * xk[t][cl];
          ++n;
        }
      const float r32 = n > 0 ? fmaxf(EPS_SCALE, sqrtf(ss / (float)n)) : EPS_SCALE;
      const uint16_t r16 = f16_bits(r32);
      reinterpret_cast<uint16_t*>(km)[c] = r16;
      red0[0][cl] = f16_val(r16);
    }
    __syncthreads();
    const float rf = red0[0][cl];
    const float th0 = lv.tables->q2k_thr[0], th1 = lv.tables->q2k_thr[1], th2 = lv.tables->q2k_thr[2];
#pragma unroll
    for (int i = 0; i < PR; ++i) {
      const int t = rg + RGS * i;
      if (calib(t)) {
        const float x = kx[i] / rf;
        ck[t][cl] = (uint8_t)((x >= th0) + (x >= th1) + (x >= th2));
      }
    }
  }
  // 3b. V of the rows from vt0 on: the group of one row is one half-wave
#pragma unroll
  for (int i = 0; i < PR; ++i) {
    const int t = rg + RGS * i;
    if (t < vt0 || t >= tend || ((smask >> t) & 1u)) continue;  // uniform over the half-wave
    if constexpr (!Q2K) {
      const float mn = half_min(vx[i]) + 0.0f, mx = half_max(vx[i]) + 0.0f;
      constexpr float L = (float)((1 << VB) - 1);
      const float s32 = fmaxf(EPS_SCALE, (mx - mn) / L);
      const uint16_t s16 = f16_bits(s32), z16 = f16_bits(mn);
      const float vsf = f16_val(s16), vzf = f16_val(z16);
      const float u = rintf((vx[i] - vzf) / vsf);
      cvt[cl][t] = (uint8_t)fminf(fmaxf(u, 0.f), L);
      if (cl == 0) {
        vms[t] = s16;
        vmz[t] = z16;
      }
    } else {  // symmetric 4-bit, s = absmax / 7
      const float am = half_max(fabsf(vx[i])) + 0.0f;
      const uint16_t s16 = f16_bits(fmaxf(EPS_SCALE, am / 7.0f));
      const float vsf = f16_val(s16);
      const float q = fminf(fmaxf(rintf(vx[i] / vsf), -8.f), 7.f);
      cvt[cl][t] = (uint8_t)(q + 8.f);
      if (cl == 0) vms[t] = s16;
    }
  }
  __syncthreads();

  // 4. K code words of the group: row t, words KB * grp .. KB * grp + KB - 1 of the row
  if (tid < G * KB) {
    const int t = tid / KB, w = tid % KB;
    uint32_t cw[4];
    if constexpr (KPW == 16) {
      const uint4 x = *reinterpret_cast<const uint4*>(&ck[t][16 * w]);
      cw[0] = x.x, cw[1] = x.y, cw[2] = x.z, cw[3] = x.w;
    } else if constexpr (KPW == 8) {
      const uint2 x = *reinterpret_cast<const uint2*>(&ck[t][8 * w]);
      cw[0] = x.x, cw[1] = x.y, cw[2] = cw[3] = 0u;
    } else {
      cw[0] = *reinterpret_cast<const uint32_t*>(&ck[t][4 * w]);
      cw[1] = cw[2] = cw[3] = 0u;
    }
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < KPW; ++k) word |= ((cw[k >> 2] >> (8 * (k & 3))) & 0xFFu) << (16 * (k & 1) + KB * (k >> 1));
    reinterpret_cast<uint32_t*>(rec + lv.k_codes)[t * (D * KB / 32) + KB * grp + w] = word;
  }
  // 5. V code words of the group: chunk q = 16 kg + i, group word w; its codes are channels
  //    16 mu + i (mu = 2 grp, 2 grp + 1) of tokens T(kg, e); bits of rows before vt0 are kept
  if (tid < 64 * VWG) {
    const int q = tid / VWG, w = tid % VWG, kg = q >> 4, i = q & 15;
    constexpr uint32_t m1 = (1u << VB) - 1;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < VPW; ++k) {
      const int sq = (VWG * grp + w) * VPW + k, mu = sq >> 3, e = sq & 7;
      const int t = v_tok(kg, e), shf = 16 * (k & 1) + VB * (k >> 1);
      const int lc = 16 * (mu - 2 * grp) + i;
      if (t < vt0) word |= oldv & (m1 << shf);
      else if (t < tend) word |= (uint32_t)cvt[lc][t] << shf;
    }
    reinterpret_cast<uint32_t*>(rec + lv.v_codes)[q * wpc + VWG * grp + w] = word;
  }
  // 6. V metadata of rows from vt0 on (rows past tend cleared)
  if (tid >= vt0 && tid < G) {
    const int ng = D / 32, mi = v_meta_idx(tid, grp, ng);
    uint16_t* vm = reinterpret_cast<uint16_t*>(rec + lv.v_meta);
    vm[mi] = tid < tend ? vms[tid] : 0;
    if constexpr (!Q2K) vm[G * ng + mi] = tid < tend ? vmz[tid] : 0;
  }
  }  // !open_mode
  // 7-9. the new rows' raw copies, from the values this thread loaded in the first phase (its rows
  //      rg + RGS i; fp16 input round-trips through fp32 exactly): staging of an open block, the
  //      fp16 window ring (rows p in [max(P, P+n-R), P+n)) and the fp16 sink pool
  const int64_t wlo = (a.P + a.n - sh.R) > a.P ? (a.P + a.n - sh.R) : a.P;
#pragma unroll
  for (int i = 0; i < PR; ++i) {
    const int t = rg + RGS * i;
    if (t < tnew0 || t >= tend) continue;
    const int64_t p = base + t;
    const uint16_t k16 = f16_bits(kx[i]), v16 = f16_bits(vx[i]);
    if (tend < G) {
      const int64_t so = ((int64_t)s * G + t) * D + c;
      if (sh.in_f32) reinterpret_cast<float*>(lv.staging)[so] = kx[i];
      else reinterpret_cast<uint16_t*>(lv.staging)[so] = k16;
    }
    if (sh.R > 0 && p >= wlo) {
      const int64_t wo = ((int64_t)s * sh.R + p % sh.R) * D + c;
      lv.win_k[wo] = k16;
      lv.win_v[wo] = v16;
    }
    if (sh.n_sink > 0) {
      const int slot = sink_slot[t];
      if (slot >= 0) {
        const int64_t so = ((int64_t)s * sh.n_sink + slot) * D + c;
        lv.sink_k[so] = k16;
        lv.sink_v[so] = v16;
      }
    }
  }
  if (sh.n_sink > 0) {
    // first-N commits: positions and count, by one workgroup per batch element
    if (sh.sink_mode == KVQ_SINK_FIRST_N && h == 0 && blockIdx.x == 0 && grp == 0) {
      const int64_t P1 = a.P + a.n;
      if (tid < sh.n_sink && tid < P1) lv.sink_pos[b * sh.n_sink + tid] = tid;
      if (tid == 0) lv.sink_count[b] = (int)(P1 < sh.n_sink ? P1 : sh.n_sink);
    }
  }
}

template <int FMT, int KB>
hipError_t launch_cs_k(const AppendArgs& a, dim3 grid, hipStream_t st) {
  switch (a.sh.vb) {
    case 2: hipLaunchKernelGGL((k_append_cs<FMT, KB, 2>), grid, dim3(NT), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_append_cs<FMT, KB, 4>), grid, dim3(NT), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_append_cs<FMT, KB, 8>), grid, dim3(NT), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Whole blocks of a prefill chunk (fp16 input, block formats): one wave per (block, stream), four
// waves per workgroup working independently.  Lane (j, r) holds channels 8j .. 8j+7 of rows
// NI*r .. NI*r + NI-1 (one 16-byte load per row and tensor; LR = D/8 lanes per row, so one load
// instruction reads 64/LR whole rows).  K statistics per channel reduce over the lane's rows and
// then across the row groups; V statistics per (row, 32 channels) reduce over four neighbouring
// lanes.  K code words are assembled in registers; V codes pass through a wave-private LDS tile
// [token][channel] so that each lane can gather the chunk of the matrix-core tile order it writes.
// q2k's block RMS sums each channel in token order from a wave-private copy of the K rows.  The
// arithmetic that decides a code is the per-element arithmetic of k_append_cs, operation for
// operation.
constexpr int FW = 4;  // waves (blocks) per workgroup of k_append_full

template <int FMT, int D>
struct FullSmem {
  static constexpr int Q = FMT == KVQ_FMT_Q2K;
  alignas(16) uint8_t vc[FW][G][D + 8];       // V codes [token][channel] (rows padded: bank spread)
  alignas(16) _Float16 kr[Q ? FW : 1][Q ? G : 1][D + 8];  // q2k: K rows
  float rf[Q ? FW : 1][D];                    // q2k: fp16 block RMS as fp32
};

__device__ __forceinline__ void h8(const uint4& w, float (&x)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xFFFFu));
    x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
  }
}

template <int FMT, int KB, int VB, int D>
__global__ __launch_bounds__(64 * FW) void k_append_full(AppendArgs a, int64_t fb0, int nfull) {
  constexpr bool Q2K = FMT == KVQ_FMT_Q2K;
  constexpr int LR = D / 8, RPI = 64 / LR, NI = G / RPI, NG = D / 32;
  constexpr int VPW = 32 / VB, WPC = D * VB / 64;
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int fb = blockIdx.x * FW + wv;
  if (fb >= nfull) return;  // waves never meet at a barrier: an idle wave may leave
  const int s = blockIdx.y, b = s / sh.Hkv, h = s % sh.Hkv;
  const int64_t beta = fb0 + fb, base = beta * G;
  const int j = lane % LR, r = lane / LR;
  uint8_t* rec = lv.bulk + ((int64_t)s * lv.cap_b + beta % lv.cap_b) * lv.rec;
  __shared__ FullSmem<FMT, D> sm;

  // every global load first: the block's K and V rows, the sink list
  const int64_t row0 = ((int64_t)b * sh.Hkv + h) * a.n + (base - a.P);  // input row of token 0
  const uint16_t* kin = static_cast<const uint16_t*>(a.k);
  const uint16_t* vin = static_cast<const uint16_t*>(a.v);
  uint4 kw[NI], vw[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t off = (row0 + NI * r + i) * D + 8 * j;
    kw[i] = *reinterpret_cast<const uint4*>(kin + off);
    vw[i] = *reinterpret_cast<const uint4*>(vin + off);
  }
  // sink rows of the block: lane t < 32 finds the slot of position base + t
  int myslot = -1;
  if (sh.n_sink > 0) {
    const int64_t p = base + (lane & 31);
    if (sh.sink_mode == KVQ_SINK_FIRST_N) {
      if (p < sh.n_sink) myslot = (int)p;
    } else if (sh.sink_mode == KVQ_SINK_TOPK) {
      const int cnt = lv.sink_count[b];
      const int sp = lane < sh.n_sink ? lv.sink_pos[b * sh.n_sink + lane] : -1;
      for (int i = 0; i < sh.n_sink; ++i) {
        const int pi = __builtin_amdgcn_readlane(sp, i);
        if (i < cnt && pi == p) myslot = i;
      }
    }
  }
  const uint32_t smask = (uint32_t)__ballot(lane < 32 && myslot >= 0);
  auto calib = [&](int t) { return !((smask >> t) & 1u); };

  // ---- K: statistics per channel, then codes ----
  uint8_t* km = rec + lv.k_meta;
  uint32_t kcode[NI][2];  // the lane's 8 codes of each row, bytes 0..3 and 4..7
  if constexpr (!Q2K) {
    float mn[8], mx[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      mn[c] = INFINITY;
      mx[c] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (!calib(NI * r + i)) continue;
      float x[8];
      h8(kw[i], x);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        mn[c] = fminf(mn[c], x[c]);
        mx[c] = fmaxf(mx[c], x[c]);
      }
    }
#pragma unroll
    for (int off = LR; off < 64; off <<= 1)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        mn[c] = fminf(mn[c], __shfl_xor(mn[c], off));
        mx[c] = fmaxf(mx[c], __shfl_xor(mx[c], off));
      }
    constexpr float L = (float)((1 << KB) - 1);
    float sf[8], zf[8];
    uint16_t s16[8], z16[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float lo = mn[c], hi = mx[c];
      if (hi == -INFINITY) lo = hi = 0.f;  // no calibration row
      lo = lo + 0.0f;
      hi = hi + 0.0f;
      const float s32 = fmaxf(EPS_SCALE, (hi - lo) / L);
      s16[c] = f16_bits(s32);
      z16[c] = f16_bits(lo);
      sf[c] = f16_val(s16[c]);
      zf[c] = f16_val(z16[c]);
    }
    if (r == 0) {
      uint32_t sw[4], zw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sw[q] = (uint32_t)s16[2 * q] | ((uint32_t)s16[2 * q + 1] << 16);
        zw[q] = (uint32_t)z16[2 * q] | ((uint32_t)z16[2 * q + 1] << 16);
      }
      *reinterpret_cast<uint4*>(km + 2 * 8 * j) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
      *reinterpret_cast<uint4*>(km + 2 * (D + 8 * j)) = make_uint4(zw[0], zw[1], zw[2], zw[3]);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float x[8];
      h8(kw[i], x);
      const bool cal = calib(NI * r + i);
      uint32_t u8[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float u = rintf((x[c] - zf[c]) / sf[c]);
        u8[c] = cal ? (uint32_t)fminf(fmaxf(u, 0.f), L) : 0u;
      }
      kcode[i][0] = u8[0] | (u8[1] << 8) | (u8[2] << 16) | (u8[3] << 24);
      kcode[i][1] = u8[4] | (u8[5] << 8) | (u8[6] << 16) | (u8[7] << 24);
    }
  } else {
    // block RMS per channel, summed in token order over the calibration rows
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<uint4*>(&sm.kr[wv][NI * r + i][8 * j]) = kw[i];
    __builtin_amdgcn_wave_barrier();
    const int ncal = G - __popc(smask);
    if (lane < D / 2) {
      float ss0 = 0.f, ss1 = 0.f;
      for (int t = 0; t < G; ++t) {
        if (!calib(t)) continue;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&sm.kr[wv][t][2 * lane]);
        const float x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
        const float x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
        ss0 = ss0 + x0 * x0;
        ss1 = ss1 + x1 * x1;
      }
      const float r0 = ncal > 0 ? fmaxf(EPS_SCALE, sqrtf(ss0 / (float)ncal)) : EPS_SCALE;
      const float r1 = ncal > 0 ? fmaxf(EPS_SCALE, sqrtf(ss1 / (float)ncal)) : EPS_SCALE;
      const uint16_t b0 = f16_bits(r0), b1 = f16_bits(r1);
      reinterpret_cast<uint32_t*>(km)[lane] = (uint32_t)b0 | ((uint32_t)b1 << 16);
      sm.rf[wv][2 * lane] = f16_val(b0);
      sm.rf[wv][2 * lane + 1] = f16_val(b1);
    }
    __builtin_amdgcn_wave_barrier();
    float rf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) rf[c] = sm.rf[wv][8 * j + c];
    const float th0 = lv.tables->q2k_thr[0], th1 = lv.tables->q2k_thr[1], th2 = lv.tables->q2k_thr[2];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float x[8];
      h8(kw[i], x);
      const bool cal = calib(NI * r + i);
      uint32_t u8[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float y = x[c] / rf[c];
        u8[c] = cal ? (uint32_t)((y >= th0) + (y >= th1) + (y >= th2)) : 0u;
      }
      kcode[i][0] = u8[0] | (u8[1] << 8) | (u8[2] << 16) | (u8[3] << 24);
      kcode[i][1] = u8[4] | (u8[5] << 8) | (u8[6] << 16) | (u8[7] << 24);
    }
  }
  // K code words: word W of a row holds channels KPW*W .. KPW*W + KPW-1, code k at bit
  // 16*(k%2) + KB*(k/2)
  uint32_t* kdst = reinterpret_cast<uint32_t*>(rec + lv.k_codes);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = NI * r + i;
    uint32_t u[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) u[c] = (kcode[i][c >> 2] >> (8 * (c & 3))) & 0xFFu;
    if constexpr (KB == 2) {  // one word per lane pair: this lane's codes are k = 8*(j%2) + c
      uint32_t part = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) part |= u[c] << (16 * (c & 1) + 8 * (j & 1) + 2 * (c >> 1));
      part |= __shfl_xor(part, 1);
      if ((j & 1) == 0) kdst[t * (D * KB / 32) + (j >> 1)] = part;
    } else if constexpr (KB == 4) {  // one word per lane
      uint32_t wd = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) wd |= u[c] << (16 * (c & 1) + 4 * (c >> 1));
      kdst[t * (D * KB / 32) + j] = wd;
    } else {  // two words per lane
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        w0 |= u[c] << (16 * (c & 1) + 8 * (c >> 1));
        w1 |= u[4 + c] << (16 * (c & 1) + 8 * (c >> 1));
      }
      *reinterpret_cast<uint2*>(&kdst[t * (D * KB / 32) + 2 * j]) = make_uint2(w0, w1);
    }
  }

  // ---- V: statistics per (row, 32-channel group) over four neighbouring lanes, codes to LDS ----
  uint16_t* vm = reinterpret_cast<uint16_t*>(rec + lv.v_meta);
  const int g = j >> 2;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = NI * r + i;
    float x[8];
    h8(vw[i], x);
    uint32_t u8[8];
    uint16_t vs16 = 0, vz16 = 0;
    if constexpr (!Q2K) {
      float lo = x[0], hi = x[0];
#pragma unroll
      for (int c = 1; c < 8; ++c) {
        lo = fminf(lo, x[c]);
        hi = fmaxf(hi, x[c]);
      }
      lo = fminf(lo, __shfl_xor(lo, 1));
      hi = fmaxf(hi, __shfl_xor(hi, 1));
      lo = fminf(lo, __shfl_xor(lo, 2));
      hi = fmaxf(hi, __shfl_xor(hi, 2));
      lo = lo + 0.0f;
      hi = hi + 0.0f;
      constexpr float L = (float)((1 << VB) - 1);
      const float s32 = fmaxf(EPS_SCALE, (hi - lo) / L);
      vs16 = f16_bits(s32);
      vz16 = f16_bits(lo);
      const float vsf = f16_val(vs16), vzf = f16_val(vz16);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float u = rintf((x[c] - vzf) / vsf);
        u8[c] = (uint32_t)fminf(fmaxf(u, 0.f), L);
      }
    } else {  // symmetric 4-bit, s = absmax / 7
      float am = fabsf(x[0]);
#pragma unroll
      for (int c = 1; c < 8; ++c) am = fmaxf(am, fabsf(x[c]));
      am = fmaxf(am, __shfl_xor(am, 1));
      am = fmaxf(am, __shfl_xor(am, 2));
      am = am + 0.0f;
      vs16 = f16_bits(fmaxf(EPS_SCALE, am / 7.0f));
      const float vsf = f16_val(vs16);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float q = fminf(fmaxf(rintf(x[c] / vsf), -8.f), 7.f);
        u8[c] = (uint32_t)(q + 8.f);
      }
    }
    const bool cal = calib(t);  // sink rows: zero codes and zero metadata
    const uint32_t c0 = u8[0] | (u8[1] << 8) | (u8[2] << 16) | (u8[3] << 24);
    const uint32_t c1 = u8[4] | (u8[5] << 8) | (u8[6] << 16) | (u8[7] << 24);
    *reinterpret_cast<uint2*>(&sm.vc[wv][t][8 * j]) = cal ? make_uint2(c0, c1) : make_uint2(0u, 0u);
    if ((j & 3) == 0) {
      const int mi = v_meta_idx(t, g, NG);
      vm[mi] = cal ? vs16 : (uint16_t)0;
      if constexpr (!Q2K) vm[G * NG + mi] = cal ? vz16 : (uint16_t)0;
    }
  }
  __builtin_amdgcn_wave_barrier();
  // V code words in the matrix-core order: chunk q = lane (token group kg = q/16, channel i = q%16)
  // holds, for channel tile mu, codes of tokens v_tok(kg, e), e = 0..7, of channel 16*mu + i
  {
    const int kg = lane >> 4, i = lane & 15;
    uint32_t* vdst = reinterpret_cast<uint32_t*>(rec + lv.v_codes) + lane * WPC;
    uint32_t words[WPC];
#pragma unroll
    for (int w = 0; w < WPC; ++w) words[w] = 0u;
#pragma unroll
    for (int mu = 0; mu < D / 16; ++mu)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t code = sm.vc[wv][v_tok(kg, e)][16 * mu + i];
        const int sq = 8 * mu + e, w = sq / VPW, k = sq % VPW;
        words[w] |= code << (16 * (k & 1) + VB * (k >> 1));
      }
#pragma unroll
    for (int w = 0; w < WPC; ++w) vdst[w] = words[w];
  }

  // ---- fp16 window ring (rows p in [max(P, P+n-R), P+n)) and sink pool: the lanes of a row copy
  // their 16 bytes ----
  const int64_t wlo = (a.P + a.n - sh.R) > a.P ? (a.P + a.n - sh.R) : a.P;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = NI * r + i;
    const int64_t p = base + t;
    if (sh.R > 0 && p >= wlo) {
      const int64_t wo = ((int64_t)s * sh.R + p % sh.R) * D + 8 * j;
      *reinterpret_cast<uint4*>(lv.win_k + wo) = kw[i];
      *reinterpret_cast<uint4*>(lv.win_v + wo) = vw[i];
    }
    const int slot = __shfl(myslot, t);
    if (slot >= 0) {
      const int64_t so = ((int64_t)s * sh.n_sink + slot) * D + 8 * j;
      *reinterpret_cast<uint4*>(lv.sink_k + so) = kw[i];
      *reinterpret_cast<uint4*>(lv.sink_v + so) = vw[i];
    }
  }
  // first-N commits (block 0 of a chunk at P = 0): positions and count, once per batch element
  if (sh.n_sink > 0 && sh.sink_mode == KVQ_SINK_FIRST_N && h == 0 && beta == 0) {
    const int64_t P1 = a.P + a.n;
    if (lane < sh.n_sink && lane < P1) lv.sink_pos[b * sh.n_sink + lane] = lane;
    if (lane == 0) lv.sink_count[b] = (int)(P1 < sh.n_sink ? P1 : sh.n_sink);
  }
}

template <int FMT, int KB, int VB>
hipError_t launch_full_kv(const AppendArgs& a, int64_t fb0, int nfull, hipStream_t st) {
  const dim3 grid((nfull + FW - 1) / FW, a.sh.B * a.sh.Hkv);
  switch (a.sh.D) {
    case 32: hipLaunchKernelGGL((k_append_full<FMT, KB, VB, 32>), grid, dim3(64 * FW), 0, st, a, fb0, nfull); break;
    case 64: hipLaunchKernelGGL((k_append_full<FMT, KB, VB, 64>), grid, dim3(64 * FW), 0, st, a, fb0, nfull); break;
    case 128: hipLaunchKernelGGL((k_append_full<FMT, KB, VB, 128>), grid, dim3(64 * FW), 0, st, a, fb0, nfull); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB>
hipError_t launch_full_k(const AppendArgs& a, int64_t fb0, int nfull, hipStream_t st) {
  switch (a.sh.vb) {
    case 2: return launch_full_kv<KVQ_FMT_KIVI, KB, 2>(a, fb0, nfull, st);
    case 4: return launch_full_kv<KVQ_FMT_KIVI, KB, 4>(a, fb0, nfull, st);
    case 8: return launch_full_kv<KVQ_FMT_KIVI, KB, 8>(a, fb0, nfull, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_full(const AppendArgs& a, int64_t fb0, int nfull, hipStream_t st) {
  const Shape& sh = a.sh;
  if (sh.fmt == KVQ_FMT_Q2K) return launch_full_kv<KVQ_FMT_Q2K, 2, 4>(a, fb0, nfull, st);
  switch (sh.kb) {
    case 2: return launch_full_k<2>(a, fb0, nfull, st);
    case 4: return launch_full_k<4>(a, fb0, nfull, st);
    case 8: return launch_full_k<8>(a, fb0, nfull, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cs(const AppendArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  dim3 grid(a.nblk, sh.B * sh.Hkv, sh.D / 32);
  if (sh.fmt == KVQ_FMT_Q2K) return launch_cs_k<KVQ_FMT_Q2K, 2>(a, grid, st);
  switch (sh.kb) {
    case 2: return launch_cs_k<KVQ_FMT_KIVI, 2>(a, grid, st);
    case 4: return launch_cs_k<KVQ_FMT_KIVI, 4>(a, grid, st);
    case 8: return launch_cs_k<KVQ_FMT_KIVI, 8>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  if (sh.fmt != KVQ_FMT_TQ && sh.D % 32 == 0) {  // block formats
    // The block the chunk starts inside (an open block: re-quantized from its staged rows, or with
    // deferral completed from its staged K and fp16-window V rows) runs first and alone: later rows
    // of the chunk overwrite staging and window slots it reads.  Then whole blocks of fp16 input: one
    // wave per (block, stream); the block left open at the end and everything else: one workgroup
    // per (block, stream, 32-channel group).
    hipError_t e;
    const int64_t end = a.P + a.n, fb0 = (a.P + G - 1) / G, fb1 = end / G, last = (end - 1) / G;
    if (a.P % G != 0) {
      AppendArgs e0 = a;
      e0.blk0 = a.P / G;
      e0.nblk = 1;
      if ((e = launch_cs(e0, st)) != hipSuccess) return e;
      if (end <= fb0 * G) return hipSuccess;  // the chunk ends inside that block
    }
    const bool aligned = (reinterpret_cast<uintptr_t>(a.k) % 16 == 0) && (reinterpret_cast<uintptr_t>(a.v) % 16 == 0);
    if (!sh.in_f32 && aligned && fb1 > fb0) {
      if ((e = launch_full(a, fb0, (int)(fb1 - fb0), st)) != hipSuccess) return e;
      if (end % G != 0) {
        AppendArgs e1 = a;
        e1.blk0 = fb1;
        e1.nblk = 1;
        if ((e = launch_cs(e1, st)) != hipSuccess) return e;
      }
      return hipSuccess;
    }
    AppendArgs e2 = a;
    e2.blk0 = fb0;
    e2.nblk = (int)(last - fb0 + 1);
    return launch_cs(e2, st);
  }
  dim3 grid(a.nblk, sh.B * sh.Hkv);
  if (sh.D > MAX_D) hipLaunchKernelGGL(k_append<MAX_SD>, grid, dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(k_append<MAX_D>, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
