// Append / quantize kernel: one workgroup per (touched 32-token block, stream).
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
constexpr int XP = MAX_D + 1;  // padded LDS row (bank spread for per-row loops)

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
// are the 32 lanes of one half-wave.
__global__ __launch_bounds__(NT) void k_append(AppendArgs a) {
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
  __shared__ alignas(16) uint8_t ck[G][MAX_D];   // K codes [token][channel]
  __shared__ alignas(16) uint8_t cvt[MAX_D][G];  // V codes [channel][token]
  __shared__ float red0[NT / 32][MAX_D], red1[NT / 32][MAX_D];  // per row group partials
  __shared__ int sink_slot[G];
  __shared__ uint32_t smask_s;
  __shared__ uint16_t vmeta_s[G][4], vmeta_z[G][4];
  __shared__ float knorm[G], vnorm[G];

  // Every global load of the kernel is issued before any of them is used (one memory round trip
  // instead of one per loop iteration): the committed sink list, this thread's elements of the
  // block's rows (new rows from the chunk, earlier rows of an open K block from staging) and the
  // V code words that hold bits of rows appended by earlier calls.
  constexpr int PER = G * MAX_D / NT;  // row elements per thread (at most)
  const int nper = G * D / NT;         // row elements per thread
  const int ng = D / 32;
  const int wpc = D * sh.vb / 64;      // words per V code chunk
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
        const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
        kx[i] = ld_in(a.k, gi, sh.in_f32);
        vx[i] = ld_in(a.v, gi, sh.in_f32);
      } else if (!tq) {
        kx[i] = ld_in(lv.staging, ((int64_t)s * G + t) * D + c, sh.in_f32);
      }
    }
  }
  constexpr int VW = 64 * (MAX_D * 8 / 64) / NT;  // V code words per thread (at most)
  uint32_t oldv[VW];
  {
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(rec + lv.v_codes);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      const int idx = tid + i * NT;
      oldv[i] = (tnew0 > 0 && idx < 64 * wpc) ? vw[idx] : 0u;
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
  for (int idx = tid; idx < G * MAX_D / 16; idx += NT) {
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
    // TQ rows (K and V) and the rotation: one wave per row
    const int lane = tid & 63, w = tid >> 6;
    const float cd = (float)(1.0 / __builtin_sqrt((double)D));
    const Tables* T = lv.tables;
    for (int t = tnew0 + w; t < tend; t += NT / 64) {
      if (sink_slot[t] >= 0) continue;
      for (int which = 0; which < 2; ++which) {
        float (*X)[XP] = which ? xv : xk;
        const int nb = which ? sh.vb : sh.kb;
        const float* bnd = which ? T->v_bnd : T->k_bnd;
        const bool act = 2 * lane < D;
        float y0 = act ? X[t][2 * lane] * T->signs[2 * lane] : 0.f;
        float y1 = act ? X[t][2 * lane + 1] * T->signs[2 * lane + 1] : 0.f;
        wave_fwht(y0, y1, D, lane);
        y0 = y0 * cd;
        y1 = y1 * cd;
        const float nrm = sqrtf(wave_sumsq(y0, y1, D));
        const float t0 = nrm > 0.f ? y0 / nrm : 0.f, t1 = nrm > 0.f ? y1 / nrm : 0.f;
        int u0 = 0, u1 = 0;
        for (int j = 0; j < (1 << nb) - 1; ++j) {
          u0 += t0 >= bnd[j];
          u1 += t1 >= bnd[j];
        }
        if (act) {
          if (which) {
            cvt[2 * lane][t] = (uint8_t)u0;
            cvt[2 * lane + 1][t] = (uint8_t)u1;
          } else {
            ck[t][2 * lane] = (uint8_t)u0;
            ck[t][2 * lane + 1] = (uint8_t)u1;
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
      if (idx >= 64 * wpc) break;
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
      const int64_t gi = (in_row0 + (p - a.P)) * D + cc;
      const int64_t wo = ((int64_t)s * sh.R + p % sh.R) * D + cc;
      lv.win_k[wo] = ld_in_f16(a.k, gi, sh.in_f32);
      lv.win_v[wo] = ld_in_f16(a.v, gi, sh.in_f32);
    }
  }
  // 9. fp16 sink pool
  if (sh.n_sink > 0) {
    for (int idx = tid; idx < (tend - tnew0) * D; idx += NT) {
      const int t = tnew0 + idx / D, cc = idx % D;
      const int slot = sink_slot[t];
      if (slot < 0) continue;
      const int64_t gi = (in_row0 + (base + t - a.P)) * D + cc;
      const int64_t so = ((int64_t)s * sh.n_sink + slot) * D + cc;
      lv.sink_k[so] = ld_in_f16(a.k, gi, sh.in_f32);
      lv.sink_v[so] = ld_in_f16(a.v, gi, sh.in_f32);
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
      } else {
        kx[i] = ld_in(lv.staging, ((int64_t)s * G + t) * D + c, sh.in_f32);
      }
    }
  }
  uint32_t oldv = 0;  // word (chunk tid / VWG, group word tid % VWG), for tid < 64 * VWG
  const uint32_t* vwords = reinterpret_cast<const uint32_t*>(rec + lv.v_codes);
  if (tnew0 > 0 && tid < 64 * VWG) oldv = vwords[(tid / VWG) * wpc + grp * VWG + tid % VWG];

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
  // 3b. V of the new rows: the group of one row is one half-wave
#pragma unroll
  for (int i = 0; i < PR; ++i) {
    const int t = rg + RGS * i;
    if (t < tnew0 || t >= tend || ((smask >> t) & 1u)) continue;  // uniform over the half-wave
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
  //    16 mu + i (mu = 2 grp, 2 grp + 1) of tokens T(kg, e); bits of rows before tnew0 are kept
  if (tid < 64 * VWG) {
    const int q = tid / VWG, w = tid % VWG, kg = q >> 4, i = q & 15;
    constexpr uint32_t m1 = (1u << VB) - 1;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < VPW; ++k) {
      const int sq = (VWG * grp + w) * VPW + k, mu = sq >> 3, e = sq & 7;
      const int t = v_tok(kg, e), shf = 16 * (k & 1) + VB * (k >> 1);
      const int lc = 16 * (mu - 2 * grp) + i;
      if (t < tnew0) word |= oldv & (m1 << shf);
      else if (t < tend) word |= (uint32_t)cvt[lc][t] << shf;
    }
    reinterpret_cast<uint32_t*>(rec + lv.v_codes)[q * wpc + VWG * grp + w] = word;
  }
  // 6. V metadata of rows from tnew0 on (rows past tend cleared)
  if (tid >= tnew0 && tid < G) {
    const int ng = D / 32, mi = v_meta_idx(tid, grp, ng);
    uint16_t* vm = reinterpret_cast<uint16_t*>(rec + lv.v_meta);
    vm[mi] = tid < tend ? vms[tid] : 0;
    if constexpr (!Q2K) vm[G * ng + mi] = tid < tend ? vmz[tid] : 0;
  }
  // 7. staging of an open block (raw K input rows)
  if (tend < G) {
    for (int t = tnew0 + rg; t < tend; t += RGS) {
      const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
      const int64_t so = ((int64_t)s * G + t) * D + c;
      if (sh.in_f32) reinterpret_cast<float*>(lv.staging)[so] = static_cast<const float*>(a.k)[gi];
      else reinterpret_cast<uint16_t*>(lv.staging)[so] = static_cast<const uint16_t*>(a.k)[gi];
    }
  }
  // 8. fp16 window ring: rows p in [max(P, P+n-R), P+n)
  if (sh.R > 0) {
    const int64_t wlo = (a.P + a.n - sh.R) > a.P ? (a.P + a.n - sh.R) : a.P;
    for (int t = tnew0 + rg; t < tend; t += RGS) {
      const int64_t p = base + t;
      if (p < wlo) continue;
      const int64_t gi = (in_row0 + (p - a.P)) * D + c;
      const int64_t wo = ((int64_t)s * sh.R + p % sh.R) * D + c;
      lv.win_k[wo] = ld_in_f16(a.k, gi, sh.in_f32);
      lv.win_v[wo] = ld_in_f16(a.v, gi, sh.in_f32);
    }
  }
  // 9. fp16 sink pool
  if (sh.n_sink > 0) {
    for (int t = tnew0 + rg; t < tend; t += RGS) {
      const int slot = sink_slot[t];
      if (slot < 0) continue;
      const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
      const int64_t so = ((int64_t)s * sh.n_sink + slot) * D + c;
      lv.sink_k[so] = ld_in_f16(a.k, gi, sh.in_f32);
      lv.sink_v[so] = ld_in_f16(a.v, gi, sh.in_f32);
    }
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

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  if (sh.fmt != KVQ_FMT_TQ && sh.D % 32 == 0) {  // block formats: one workgroup per 32-channel group
    dim3 grid(a.nblk, sh.B * sh.Hkv, sh.D / 32);
    if (sh.fmt == KVQ_FMT_Q2K) return launch_cs_k<KVQ_FMT_Q2K, 2>(a, grid, st);
    switch (sh.kb) {
      case 2: return launch_cs_k<KVQ_FMT_KIVI, 2>(a, grid, st);
      case 4: return launch_cs_k<KVQ_FMT_KIVI, 4>(a, grid, st);
      case 8: return launch_cs_k<KVQ_FMT_KIVI, 8>(a, grid, st);
      default: return hipErrorInvalidValue;
    }
  }
  dim3 grid(a.nblk, sh.B * sh.Hkv);
  hipLaunchKernelGGL(k_append, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
