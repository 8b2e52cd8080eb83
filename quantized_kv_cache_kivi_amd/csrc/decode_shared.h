// Shared pieces of the decode-attention kernels: sink staging, the generic (any
// format, any head_dim) per-workgroup partial and the fixed-order merge of the
// TurboQuant split partials.
//
// Online softmax runs in the log2 domain: scores are scaled by scale*log2(e)
// and exponentiated with exp2, so a partial is (m, l, acc) with
// l = sum 2^(s - m) and acc = sum 2^(s - m) v.
#pragma once

#include "device_common.h"

namespace kvq {

constexpr float LOG2E = 1.4426950408889634f;

constexpr int DNT = 256;  // threads of a decode workgroup

// Shared memory of the generic decode kernels for rows of at most MD stored channels (128, or 256 for
// TurboQuant rows of head_dim 160).
template <int MD>
struct Smem {
  static constexpr int MAX_REC = 2 * G * MD + 4 * MD + 4 * G * 4;  // 8-bit K and V, KIVI metadata
  float q[MAX_GQA][MD];          // query (rotated for TurboQuant bulk); merged output in merge_partials()
  float sc[MAX_GQA][G];          // scores, then weights, of the current 32 rows
  float fac[MAX_GQA];            // rescale factors of the current step
  float m[MAX_GQA], l[MAX_GQA];  // running max and denominator
  float Mb[MAX_GQA], Lb[MAX_GQA];
  int sinks[MAX_SINK];      // committed sink positions (< P) of this batch element
  int sink_slot[MAX_SINK];  // their sink-pool slots
  int nsinks;
  int rk[G];                // RoPE on read: index in the compressed cache of each row of the chunk
  union {
    alignas(16) uint8_t rec[MAX_REC];                       // staged block record (bulk)
    struct { uint16_t k[G][MD], v[G][MD]; } rows;           // fp16 rows of the current chunk
    float red[DNT][MAX_GQA];                                 // cross-slice reduction (after the loop)
  } u;
};

// Committed sinks (position < P) of batch element b, compacted in slot order by wave 0:
// positions, pool slots (if `slot` is not null) and their number.  Callers synchronize.  The count
// and the position slots are loaded together (one memory round trip), then masked by the count.
__device__ inline void stage_sinks(const DecodeArgs& a, int b, int* pos, int* slot, int* count) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int ns = a.sh.n_sink;
    const int cnt = ns > 0 ? a.lv.sink_count[b] : 0;
    const int praw = lane < ns ? a.lv.sink_pos[b * ns + lane] : -1;
    const int p = lane < min(cnt, ns) ? praw : -1;
    const bool ok = p >= 0 && p < a.P;
    const uint64_t m = __ballot(ok);
    const int idx = __popcll(m & ((1ull << lane) - 1ull));
    if (ok) {
      pos[idx] = p;
      if (slot) slot[idx] = lane;
    }
    if (lane == 0) *count = __popcll(m);
  }
}

__device__ __forceinline__ uint32_t code_at(const uint8_t* sec, int word, int k, int b) {
  return (reinterpret_cast<const uint32_t*>(sec)[word] >> code_shift(k, b)) & ((1u << b) - 1u);
}

// Dequantized K value of (t, c) of the staged record; TurboQuant values are rotated-domain centroids
// (the per-token norm is applied to the score).
__device__ __forceinline__ float k_val(const Shape& sh, const uint8_t* rec, const LayerView& lv, int t, int c) {
  int w, k;
  k_code_pos(t, c, sh.D, sh.kb, &w, &k);
  const uint32_t u = sh.kb == 3 ? code3_at(rec + lv.k_codes, k_bit3(t, c, sh.D)) : code_at(rec + lv.k_codes, w, k, sh.kb);
  const uint16_t* km = reinterpret_cast<const uint16_t*>(rec + lv.k_meta);
  if (sh.fmt == KVQ_FMT_KIVI) return (float)u * f16_val(km[c]) + f16_val(km[sh.D + c]);
  if (sh.fmt == KVQ_FMT_Q2K) return lv.tables->q2k_lvl[u] * f16_val(km[c]);
  return lv.tables->k_cen[u];
}
__device__ __forceinline__ float v_val(const Shape& sh, const uint8_t* rec, const LayerView& lv, int t, int c) {
  int w, k;
  v_code_pos(t, c, sh.D, sh.vb, &w, &k);
  const uint32_t u = sh.vb == 3 ? code3_at(rec + lv.v_codes, v_bit3(t, c, sh.D)) : code_at(rec + lv.v_codes, w, k, sh.vb);
  const uint16_t* vm = reinterpret_cast<const uint16_t*>(rec + lv.v_meta);
  const int ng = sh.D / 32, g = c >> 5;
  const int mi = v_meta_idx(t, g, ng);
  if (sh.fmt == KVQ_FMT_KIVI) return (float)u * f16_val(vm[mi]) + f16_val(vm[G * ng + mi]);
  if (sh.fmt == KVQ_FMT_Q2K) return ((float)u - 8.f) * f16_val(vm[mi]);
  return lv.tables->v_cen[u];
}


// Partial of this workgroup: bulk blocks of split `sigma`, or (sigma == splits, TurboQuant and
// RoPE-on-read caches) the fp16 rows.
template <int MD>
__device__ inline void generic_partial(const DecodeArgs& a, Smem<MD>& S) {

  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int D = sh.D, r = sh.Hq / sh.Hkv, tid = threadIdx.x, lane = tid & 63;
  const int sigma = blockIdx.x, s = blockIdx.y, b = s / sh.Hkv, g = s % sh.Hkv;
  const bool tq = sh.fmt == KVQ_FMT_TQ;
  const bool fp16_split = sigma == a.splits;

  // query rows of the r heads; sinks of this batch element
  for (int idx = tid; idx < r * D; idx += DNT) {
    const int j = idx / D, c = idx % D;
    S.q[j][c] = c < sh.Din ? ld_in(a.q, ((int64_t)b * sh.Hq + g * r + j) * sh.Din + c, sh.in_f32) : 0.f;
  }
  stage_sinks(a, b, S.sinks, S.sink_slot, &S.nsinks);
  if (tid < MAX_GQA) {
    S.m[tid] = -INFINITY;
    S.l[tid] = 0.f;
  }
  __syncthreads();
  if (sh.rope) {  // the query turns by its own index: the last valid position, P - 1
    const int qi = cache_index(S.sinks, S.nsinks, a.lo, a.P - 1);
    const int h = D / 2;
    float qa[MAX_GQA * MD / 2 / DNT + 1], qb[MAX_GQA * MD / 2 / DNT + 1];
    int n = 0;
    for (int idx = tid; idx < r * h; idx += DNT, ++n) {
      const int j = idx / h, c = idx % h;
      qa[n] = rope_val(S.q[j][c], S.q[j][c + h], c, D, qi, lv.tables->rope_inv);
      qb[n] = rope_val(S.q[j][c + h], S.q[j][c], c + h, D, qi, lv.tables->rope_inv);
    }
    __syncthreads();
    n = 0;
    for (int idx = tid; idx < r * h; idx += DNT, ++n) {
      const int j = idx / h, c = idx % h;
      S.q[j][c] = qa[n];
      S.q[j][c + h] = qb[n];
    }
    __syncthreads();
  }
  if (tq && !fp16_split) {  // rotate the query: q~ = c_d * FWHT(sigma * q)
    constexpr int NK = MD / 64;
    const float cd = (float)(1.0 / __builtin_sqrt((double)D));
    for (int j = tid >> 6; j < r; j += DNT / 64) {
      float y[NK];
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int c = row_chan(lane, k);
        y[k] = c < D ? S.q[j][c] * lv.tables->signs[c] : 0.f;
      }
      row_fwht<MD>(y, D, lane);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int c = row_chan(lane, k);
        if (c < D) S.q[j][c] = y[k] * cd;
      }
    }
    __syncthreads();
  }

  // score mapping: 32 rows x 8 channel slices; value mapping: D channels x (DNT/D) row slices
  const int st = tid >> 3, sl = tid & 7, cps = D / 8;
  const int vc = tid % D, vs = tid / D, nvs = DNT / D, rps = G / nvs;
  float acc[MAX_GQA];
  for (int j = 0; j < MAX_GQA; ++j) acc[j] = 0.f;

  int nchunks;
  int64_t fp_lo = 0, n_fp = 0;
  if (fp16_split) {
    fp_lo = a.bulk_hi;  // window rows [bulk_hi, P) minus sinks, then the sinks
    n_fp = (a.P - fp_lo) + S.nsinks;
    nchunks = (int)((n_fp + G - 1) / G);
  } else {
    const int first = sigma * a.blocks_per_split;
    const int lastb = min(a.nblk, first + a.blocks_per_split);
    nchunks = lastb - first;
  }

  for (int ch = 0; ch < nchunks; ++ch) {
    int64_t blk = 0;
    // stage the chunk
    if (fp16_split) {
      for (int idx = tid; idx < G * D; idx += DNT) {
        const int t = idx / D, c = idx % D;
        const int64_t i = (int64_t)ch * G + t;
        uint16_t kx = 0, vx = 0;
        if (i < a.P - fp_lo) {
          const int64_t p = fp_lo + i;
          const int64_t wo = ((int64_t)s * sh.R + p % sh.R) * D + c;
          kx = lv.win_k[wo];
          vx = lv.win_v[wo];
        } else if (i < n_fp) {
          const int si = (int)(i - (a.P - fp_lo));
          const int64_t so = ((int64_t)s * sh.n_sink + S.sink_slot[si]) * D + c;
          kx = lv.sink_k[so];
          vx = lv.sink_v[so];
        }
        S.u.rows.k[t][c] = kx;
        S.u.rows.v[t][c] = vx;
      }
    } else {
      blk = a.blk_first + (int64_t)sigma * a.blocks_per_split + ch;
      const uint8_t* src = lv.bulk + ((int64_t)s * lv.cap_b + blk % lv.cap_b) * lv.rec;
      for (int64_t o = tid * 16; o < lv.rec; o += DNT * 16)
        *reinterpret_cast<uint4*>(S.u.rec + o) = *reinterpret_cast<const uint4*>(src + o);
    }
    if (sh.rope && tid < G) {  // index in the compressed cache of each row of the chunk
      int64_t p;
      if (fp16_split) {
        const int64_t i = (int64_t)ch * G + tid;
        p = i < a.P - fp_lo ? fp_lo + i : (i < n_fp ? S.sinks[(int)(i - (a.P - fp_lo))] : 0);
      } else {
        p = blk * G + tid;
      }
      S.rk[tid] = cache_index(S.sinks, S.nsinks, a.lo, p);
    }
    __syncthreads();

    // scores
    {
      float part[MAX_GQA];
      for (int j = 0; j < MAX_GQA; ++j) part[j] = 0.f;
      for (int cc = 0; cc < cps; ++cc) {
        const int c = sl * cps + cc;
        float kv = fp16_split ? f16_val(S.u.rows.k[st][c]) : k_val(sh, S.u.rec, lv, st, c);
        if (sh.rope) {  // the key turns by its row's index in the compressed cache
          const int pc = c < D / 2 ? c + D / 2 : c - D / 2;
          const float kp = fp16_split ? f16_val(S.u.rows.k[st][pc]) : k_val(sh, S.u.rec, lv, st, pc);
          kv = rope_val(kv, kp, c, D, S.rk[st], lv.tables->rope_inv);
        }
        for (int j = 0; j < r; ++j) part[j] = fmaf(S.q[j][c], kv, part[j]);
      }
      for (int j = 0; j < r; ++j) {
        float v = part[j];
        v = v + __shfl_xor(v, 1);
        v = v + __shfl_xor(v, 2);
        v = v + __shfl_xor(v, 4);
        part[j] = v;
      }
      if (sl == 0) {
        bool valid;
        float mult = a.scale * LOG2E;
        if (fp16_split) {
          const int64_t i = (int64_t)ch * G + st;
          valid = i < n_fp;
          if (valid && i < a.P - fp_lo) {
            const int64_t p = fp_lo + i;
            for (int q = 0; q < S.nsinks; ++q) valid = valid && S.sinks[q] != p;
          }
        } else {
          const int64_t p = blk * G + st;
          valid = p >= a.bulk_lo && p < a.bulk_hi;
          for (int q = 0; q < S.nsinks; ++q) valid = valid && S.sinks[q] != p;
          if (tq) mult = mult * reinterpret_cast<const float*>(S.u.rec + lv.k_meta)[st];
        }
        for (int j = 0; j < r; ++j) S.sc[j][st] = valid ? part[j] * mult : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax, one thread per head
    if (tid < r) {
      const int j = tid;
      float mx = -INFINITY;
      for (int t = 0; t < G; ++t) mx = fmaxf(mx, S.sc[j][t]);
      const float mold = S.m[j], mnew = fmaxf(mold, mx);
      float f = 1.f, sum = 0.f;
      if (mnew == -INFINITY) {
        for (int t = 0; t < G; ++t) S.sc[j][t] = 0.f;
      } else {
        f = mold == -INFINITY ? 0.f : exp2f(mold - mnew);
        for (int t = 0; t < G; ++t) {
          const float p = S.sc[j][t] == -INFINITY ? 0.f : exp2f(S.sc[j][t] - mnew);
          S.sc[j][t] = p;
          sum += p;
        }
        S.m[j] = mnew;
      }
      S.l[j] = S.l[j] * f + sum;
      S.fac[j] = f;
    }
    __syncthreads();
    // values
    for (int j = 0; j < r; ++j) acc[j] *= S.fac[j];
    for (int tt = 0; tt < rps; ++tt) {
      const int t = vs * rps + tt;
      float vv;
      if (fp16_split) vv = f16_val(S.u.rows.v[t][vc]);
      else {
        vv = v_val(sh, S.u.rec, lv, t, vc);
        if (tq) vv = vv * reinterpret_cast<const float*>(S.u.rec + lv.v_meta)[t];
      }
      for (int j = 0; j < r; ++j) acc[j] = fmaf(S.sc[j][t], vv, acc[j]);
    }
    __syncthreads();
  }

  // reduce the value slices and write this workgroup's partial
  for (int j = 0; j < r; ++j) S.u.red[tid][j] = acc[j];
  __syncthreads();
  float* part = a.ws + ((int64_t)s * a.nparts + sigma) * r * (D + 2);
  for (int idx = tid; idx < r * D; idx += DNT) {
    const int j = idx / D, c = idx % D;
    float v = 0.f;
    for (int q = 0; q < nvs; ++q) v += S.u.red[q * D + c][j];
    part[j * (D + 2) + 2 + c] = v;
  }
  if (tid < r) {
    part[tid * (D + 2)] = S.m[tid];
    part[tid * (D + 2) + 1] = S.l[tid];
  }
}

// Fixed-order merge of the split partials of stream blockIdx.x and the output
// (runs in its own kernel, after every split has written its partial).
template <int MD>
__device__ inline void merge_partials(const DecodeArgs& a, Smem<MD>& S) {
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int D = sh.D, r = sh.Hq / sh.Hkv, tid = threadIdx.x, lane = tid & 63;
  const int s = blockIdx.x, b = s / sh.Hkv, g = s % sh.Hkv;
  const bool tq = sh.fmt == KVQ_FMT_TQ;
  const int total = a.nparts;  // bulk splits, then the fp16 partial
  // merge in fixed order; TurboQuant merges the rotated bulk first and rotates it back
  const float* P0 = a.ws + (int64_t)s * total * r * (D + 2);
  const int nbulk = a.splits;
  float* fin = &S.q[0][0];  // reuse: merged bulk accumulator [r][D]
  if (tid < r) {
    float M = -INFINITY;
    for (int q = 0; q < (tq ? nbulk : total); ++q) M = fmaxf(M, P0[(q * r + tid) * (D + 2)]);
    float L = 0.f;
    for (int q = 0; q < (tq ? nbulk : total); ++q) {
      const float mq = P0[(q * r + tid) * (D + 2)];
      if (mq != -INFINITY) L += P0[(q * r + tid) * (D + 2) + 1] * exp2f(mq - M);
    }
    S.Mb[tid] = M;
    S.Lb[tid] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < r * D; idx += DNT) {
    const int j = idx / D, c = idx % D;
    float v = 0.f;
    for (int q = 0; q < (tq ? nbulk : total); ++q) {
      const float mq = P0[(q * r + j) * (D + 2)];
      if (mq != -INFINITY) v += P0[(q * r + j) * (D + 2) + 2 + c] * exp2f(mq - S.Mb[j]);
    }
    fin[j * MD + c] = v;
  }
  __syncthreads();
  if (tq) {
    // inverse rotation of the merged bulk accumulator: sigma * (c_d * FWHT(acc))
    constexpr int NK = MD / 64;
    const float cd = (float)(1.0 / __builtin_sqrt((double)D));
    for (int j = tid >> 6; j < r; j += DNT / 64) {
      float y[NK];
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int c = row_chan(lane, k);
        y[k] = c < D ? fin[j * MD + c] : 0.f;
      }
      row_fwht<MD>(y, D, lane);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int c = row_chan(lane, k);
        if (c < D) fin[j * MD + c] = lv.tables->signs[c] * (y[k] * cd);
      }
    }
    __syncthreads();
    // merge with the fp16 partial (original domain)
    if (tid < r) {
      const float mf = P0[(nbulk * r + tid) * (D + 2)], lf = P0[(nbulk * r + tid) * (D + 2) + 1];
      const float M = fmaxf(S.Mb[tid], mf);
      const float wb = S.Mb[tid] == -INFINITY ? 0.f : exp2f(S.Mb[tid] - M);
      const float wf = mf == -INFINITY ? 0.f : exp2f(mf - M);
      S.fac[tid] = wb;
      S.m[tid] = wf;
      S.l[tid] = S.Lb[tid] * wb + lf * wf;
    }
    __syncthreads();
    for (int idx = tid; idx < r * D; idx += DNT) {
      const int j = idx / D, c = idx % D;
      const float v = fin[j * MD + c] * S.fac[j] + P0[(nbulk * r + j) * (D + 2) + 2 + c] * S.m[j];
      if (c < sh.Din) a.out[((int64_t)b * sh.Hq + g * r + j) * sh.Din + c] = v / S.l[j];
    }
  } else {
    for (int idx = tid; idx < r * D; idx += DNT) {
      const int j = idx / D, c = idx % D;
      if (c < sh.Din) a.out[((int64_t)b * sh.Hq + g * r + j) * sh.Din + c] = fin[j * MD + c] / S.Lb[j];
    }
  }
}

}  // namespace kvq
