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

  __shared__ float xk[G][XP];
  __shared__ float xv[G][XP];
  __shared__ uint8_t ck[G][MAX_D];
  __shared__ uint8_t cv[G][MAX_D];
  __shared__ int sink_slot[G];
  __shared__ uint16_t vmeta_s[G][4], vmeta_z[G][4];
  __shared__ float knorm[G], vnorm[G];

  // 1. sink membership of the block's rows
  if (tid < G) {
    const int64_t p = base + tid;
    int slot = -1;
    if (tid < tend && sh.n_sink > 0) {
      if (sh.sink_mode == KVQ_SINK_FIRST_N) {
        if (p < sh.n_sink) slot = (int)p;
      } else if (sh.sink_mode == KVQ_SINK_TOPK) {
        const int cnt = lv.sink_count[b];
        for (int i = 0; i < cnt; ++i)
          if (lv.sink_pos[b * sh.n_sink + i] == p) slot = i;
      }
    }
    sink_slot[tid] = slot;
    knorm[tid] = 0.f;
    vnorm[tid] = 0.f;
  }
  // 2. rows: new rows from the chunk, earlier rows of an open K block from staging
  for (int idx = tid; idx < G * D; idx += NT) {
    const int t = idx / D, c = idx % D;
    float kx = 0.f, vx = 0.f;
    if (t < tend) {
      if (t >= tnew0) {
        const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
        kx = ld_in(a.k, gi, sh.in_f32);
        vx = ld_in(a.v, gi, sh.in_f32);
      } else if (!tq) {
        kx = ld_in(lv.staging, ((int64_t)s * G + t) * D + c, sh.in_f32);
      }
    }
    xk[t][c] = kx;
    xv[t][c] = vx;
    ck[t][c] = 0;
    cv[t][c] = 0;
  }
  __syncthreads();

  // 3. K
  if (!tq) {
    for (int c = tid; c < D; c += NT) {
      uint8_t* km = rec + lv.k_meta;
      if (sh.fmt == KVQ_FMT_KIVI) {
        float mn = INFINITY, mx = -INFINITY;
        bool any = false;
        for (int t = 0; t < tend; ++t)
          if (sink_slot[t] < 0) {
            mn = fminf(mn, xk[t][c]);
            mx = fmaxf(mx, xk[t][c]);
            any = true;
          }
        if (!any) mn = mx = 0.f;
        mn = mn + 0.0f;
        mx = mx + 0.0f;
        const float L = (float)((1 << sh.kb) - 1);
        const float s32 = fmaxf(EPS_SCALE, (mx - mn) / L);
        const uint16_t s16 = f16_bits(s32), z16 = f16_bits(mn);
        reinterpret_cast<uint16_t*>(km)[c] = s16;
        reinterpret_cast<uint16_t*>(km)[D + c] = z16;
        const float sf = f16_val(s16), zf = f16_val(z16);
        for (int t = 0; t < tend; ++t)
          if (sink_slot[t] < 0) {
            const float u = rintf((xk[t][c] - zf) / sf);
            ck[t][c] = (uint8_t)fminf(fmaxf(u, 0.f), L);
          }
      } else {  // Q2K
        float ss = 0.f;
        int n = 0;
        for (int t = 0; t < tend; ++t)
          if (sink_slot[t] < 0) {
            ss = ss + xk[t][c] * xk[t][c];
            ++n;
          }
        const float r32 = n > 0 ? fmaxf(EPS_SCALE, sqrtf(ss / (float)n)) : EPS_SCALE;
        const uint16_t r16 = f16_bits(r32);
        reinterpret_cast<uint16_t*>(km)[c] = r16;
        const float rf = f16_val(r16);
        const float th0 = lv.tables->q2k_thr[0], th1 = lv.tables->q2k_thr[1], th2 = lv.tables->q2k_thr[2];
        for (int t = 0; t < tend; ++t)
          if (sink_slot[t] < 0) {
            const float x = xk[t][c] / rf;
            ck[t][c] = (uint8_t)((x >= th0) + (x >= th1) + (x >= th2));
          }
      }
    }
  }
  // TQ rows (K and V) and the rotation: one wave per row
  if (tq) {
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
          uint8_t(*C)[MAX_D] = which ? cv : ck;
          C[t][2 * lane] = (uint8_t)u0;
          C[t][2 * lane + 1] = (uint8_t)u1;
        }
        if (lane == 0) (which ? vnorm : knorm)[t] = nrm;
      }
    }
  } else {
    // V per token and 32-channel group
    const int ng = D / 32;
    for (int idx = tid; idx < (tend - tnew0) * ng; idx += NT) {
      const int t = tnew0 + idx / ng, g = idx % ng;
      if (sink_slot[t] >= 0) {
        vmeta_s[t][g] = 0;
        vmeta_z[t][g] = 0;
        continue;
      }
      if (sh.fmt == KVQ_FMT_KIVI) {
        float mn = INFINITY, mx = -INFINITY;
        for (int c = 0; c < 32; ++c) {
          mn = fminf(mn, xv[t][32 * g + c]);
          mx = fmaxf(mx, xv[t][32 * g + c]);
        }
        mn = mn + 0.0f;
        mx = mx + 0.0f;
        const float L = (float)((1 << sh.vb) - 1);
        const float s32 = fmaxf(EPS_SCALE, (mx - mn) / L);
        const uint16_t s16 = f16_bits(s32), z16 = f16_bits(mn);
        vmeta_s[t][g] = s16;
        vmeta_z[t][g] = z16;
        const float sf = f16_val(s16), zf = f16_val(z16);
        for (int c = 0; c < 32; ++c) {
          const float u = rintf((xv[t][32 * g + c] - zf) / sf);
          cv[t][32 * g + c] = (uint8_t)fminf(fmaxf(u, 0.f), L);
        }
      } else {  // Q2K: symmetric 4-bit, s = absmax / 7
        float am = 0.f;
        for (int c = 0; c < 32; ++c) am = fmaxf(am, fabsf(xv[t][32 * g + c]));
        am = am + 0.0f;
        const uint16_t s16 = f16_bits(fmaxf(EPS_SCALE, am / 7.0f));
        vmeta_s[t][g] = s16;
        vmeta_z[t][g] = 0;
        const float sf = f16_val(s16);
        for (int c = 0; c < 32; ++c) {
          const float q = fminf(fmaxf(rintf(xv[t][32 * g + c] / sf), -8.f), 7.f);
          cv[t][32 * g + c] = (uint8_t)(q + 8.f);
        }
      }
    }
  }
  __syncthreads();

  // 4. K codes: token rows, word-interleaved.  Block formats rewrite the whole
  //    block (rows not present are 0); TQ writes its new rows (and clears the
  //    rest of a block it opens).
  {
    const int wpr = D * sh.kb / 32, per = 32 / sh.kb;
    uint32_t* kw = reinterpret_cast<uint32_t*>(rec + lv.k_codes);
    for (int idx = tid; idx < G * wpr; idx += NT) {
      const int t = idx / wpr, w = idx % wpr;
      if (tq && !((t >= tnew0 && t < tend) || (tnew0 == 0 && t >= tend))) continue;
      uint32_t word = 0;
      for (int k = 0; k < per; ++k) word |= (uint32_t)ck[t][w * per + k] << code_shift(k, sh.kb);
      kw[idx] = word;
    }
  }
  // 5. V codes: channel tiles; bits of rows appended earlier are kept, others rewritten
  {
    const int wpc = D * sh.vb / 64, per = 32 / sh.vb;
    uint32_t* vw = reinterpret_cast<uint32_t*>(rec + lv.v_codes);
    const uint32_t m1 = (1u << sh.vb) - 1;
    for (int idx = tid; idx < 64 * wpc; idx += NT) {
      const int q = idx / wpc, w = idx % wpc, kg = q >> 4, i = q & 15;
      const uint32_t old = tnew0 > 0 ? vw[idx] : 0u;
      uint32_t word = 0;
      for (int k = 0; k < per; ++k) {
        const int sq = w * per + k, mu = sq >> 3, e = sq & 7;
        const int t = v_tok(kg, e), c = 16 * mu + i, sh_ = code_shift(k, sh.vb);
        if (t < tnew0) word |= old & (m1 << sh_);
        else if (t < tend) word |= (uint32_t)cv[t][c] << sh_;
      }
      vw[idx] = word;
    }
  }
  // 6. metadata of rows from tnew0 on (rows past tend cleared)
  {
    const int ng = D / 32;
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
      const int t = tnew0 + idx / D, c = idx % D;
      const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
      const int64_t so = ((int64_t)s * G + t) * D + c;
      if (sh.in_f32) reinterpret_cast<float*>(lv.staging)[so] = static_cast<const float*>(a.k)[gi];
      else reinterpret_cast<uint16_t*>(lv.staging)[so] = static_cast<const uint16_t*>(a.k)[gi];
    }
  }
  // 8. fp16 window ring: rows p in [max(P, P+n-R), P+n)
  if (sh.R > 0) {
    const int64_t wlo = (a.P + a.n - sh.R) > a.P ? (a.P + a.n - sh.R) : a.P;
    for (int idx = tid; idx < (tend - tnew0) * D; idx += NT) {
      const int t = tnew0 + idx / D, c = idx % D;
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
    for (int idx = tid; idx < (tend - tnew0) * D; idx += NT) {
      const int t = tnew0 + idx / D, c = idx % D;
      const int slot = sink_slot[t];
      if (slot < 0) continue;
      const int64_t gi = (in_row0 + (base + t - a.P)) * D + c;
      const int64_t so = ((int64_t)s * sh.n_sink + slot) * D + c;
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

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  dim3 grid(a.nblk, a.sh.B * a.sh.Hkv);
  hipLaunchKernelGGL(k_append, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
