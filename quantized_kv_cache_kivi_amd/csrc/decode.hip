// Single-query decode attention over the packed cache.
//
// out[b][j] = sum_p softmax_p(scale * q[b][j] . k_p) v_p over the valid set of
// the layer: committed sinks (fp16 sink pool), the fp16 window and the
// quantized bulk, with k_p, v_p dequantized in registers ("StreamingLLM +
// KIVI — long-context decode without growing the KV cache", "Affine
// quantisation formula"; q2k pull-request page, "Summary": the fp16 overlay
// reads exact).  For TurboQuant the bulk is scored and accumulated in the
// rotated domain against the rotated query and the merged output is rotated
// back once ("TurboQuant KV Cache Compression — Spec", "Optimization: Fused
// dequant-dot").
//
// Two launches.  The split kernel (grid (splits, batch * n_kv_heads); the
// MFMA kernel of decode_fast.hip or the generic one here) writes one
// online-softmax partial (m, l, acc) per (bulk split, stream) for the r query
// heads of the stream.  The merge kernel (grid (batch * n_kv_heads, r)) scores
// the fp16 rows (window minus sinks, then sinks) of its head itself and merges
// them with the bulk partials in fixed order, so results do not depend on
// scheduling.  TurboQuant keeps a per-stream merge: its bulk partials live in
// the rotated domain, and its fp16 rows are one more generic partial (index
// splits).
#include "decode_shared.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(DNT) void k_decode(DecodeArgs a) {
  __shared__ Smem S;
  generic_partial(a, S);
}

__global__ __launch_bounds__(DNT) void k_decode_merge(DecodeArgs a) {
  __shared__ Smem S;
  merge_partials(a, S);
}

constexpr int MNT = 256;  // threads of a merge workgroup
constexpr int MCH = 256;  // fp16 rows per chunk of the merge kernel

// Address (in fp16 elements) of fp16 row i of stream s: window rows [bulk_hi, P) first, then
// the committed sinks in slot order.
__device__ __forceinline__ int64_t fp16_row(const DecodeArgs& a, int s, int64_t i, int64_t nwin, const int* slot,
                                            bool* is_sink) {
  const int D = a.sh.D;
  if (i < nwin) {
    *is_sink = false;
    const int64_t p = a.bulk_hi + i;
    return ((int64_t)s * a.sh.R + p % a.sh.R) * D;
  }
  *is_sink = true;
  return ((int64_t)s * a.sh.n_sink + slot[i - nwin]) * D;
}

// Merge for formats without a rotation: one workgroup per (stream, query head).  The fp16 rows
// are scored (one row per D/8 lanes, 8 channels a lane), turned into weights chunk by chunk with
// an online max, and accumulated (two channels a lane, rows strided over the row slices); the
// bulk partials of the head are then folded in, in split order.
__global__ __launch_bounds__(MNT) void k_merge_heads(DecodeArgs a) {
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int s = blockIdx.x, j = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = sh.D, r = sh.Hq / sh.Hkv, b = s / sh.Hkv, g = s % sh.Hkv;
  __shared__ float sc[MCH];
  __shared__ float red[2 * MNT];
  __shared__ float wq[65];
  __shared__ int sinks[MAX_SINK], slots[MAX_SINK], nsinks;
  __shared__ float Ls, Wf;

  stage_sinks(a, b, sinks, slots, &nsinks);
  __syncthreads();
  const int64_t nwin = a.P - a.bulk_hi;
  const int64_t n_fp = nwin + nsinks;

  // query slice of this lane for the score mapping, in log2 units
  const int lpr = D / 8, rpw = 64 / lpr, part = lane % lpr, rsub = lane / lpr;
  const float mult = a.scale * LOG2E;
  const int64_t qoff = ((int64_t)b * sh.Hq + (int64_t)g * r + j) * D + 8 * part;
  float qv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) qv[k] = ld_in(a.q, qoff + k, sh.in_f32) * mult;
  // value mapping: channel pair cp, row slice vsl
  const int ncp = D / 2, cp = tid % ncp, vsl = tid / ncp, nvsl = MNT / ncp;

  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int64_t c0 = 0; c0 < n_fp; c0 += MCH) {
    const int n = (int)min((int64_t)MCH, n_fp - c0);
    // scores of rows [c0, c0 + n)
    for (int base = wv * rpw; base < n; base += (MNT / 64) * rpw) {
      const int i = base + rsub;
      float d = 0.f;
      bool ok = i < n, snk = false;
      if (ok) {
        const int64_t off = fp16_row(a, s, c0 + i, nwin, slots, &snk) + 8 * part;
        const uint4 w = *reinterpret_cast<const uint4*>((snk ? lv.sink_k : lv.win_k) + off);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          d = fmaf(qv[2 * k], f16_val((uint16_t)(ww[k] & 0xFFFFu)), d);
          d = fmaf(qv[2 * k + 1], f16_val((uint16_t)(ww[k] >> 16)), d);
        }
        if (!snk) {
          const int64_t p = a.bulk_hi + c0 + i;
          for (int q = 0; q < nsinks; ++q) ok = ok && sinks[q] != p;
        }
      }
      for (int off = lpr / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      if (part == 0 && i < n) sc[i] = ok ? d : -INFINITY;
    }
    __syncthreads();
    // chunk maximum (every wave reduces the whole chunk: no extra barrier)
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) mx = fmaxf(mx, sc[i]);
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mnew = fmaxf(m, mx);
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - mnew);
    __syncthreads();
    if (tid < n) sc[tid] = (sc[tid] == -INFINITY) ? 0.f : exp2f(sc[tid] - mnew);
    __syncthreads();
    float sum = 0.f;
    for (int i = lane; i < n; i += 64) sum += sc[i];
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (mnew != -INFINITY) {
      l = l * f + sum;
      acc0 *= f;
      acc1 *= f;
      m = mnew;
    }
    for (int i = vsl; i < n; i += nvsl) {
      bool snk;
      const int64_t off = fp16_row(a, s, c0 + i, nwin, slots, &snk) + 2 * cp;
      const uint32_t w = *reinterpret_cast<const uint32_t*>((snk ? lv.sink_v : lv.win_v) + off);
      const float p = sc[i];
      acc0 = fmaf(p, f16_val((uint16_t)(w & 0xFFFFu)), acc0);
      acc1 = fmaf(p, f16_val((uint16_t)(w >> 16)), acc1);
    }
    __syncthreads();
  }
  red[2 * tid] = acc0;
  red[2 * tid + 1] = acc1;

  // weights of the bulk partials and of the fp16 rows
  const int np = a.nparts;
  const float* P0 = a.ws + (int64_t)s * np * r * (D + 2);
  if (tid < 64) {
    float M = m;
    for (int q = tid; q < np; q += 64) M = fmaxf(M, P0[(q * r + j) * (D + 2)]);
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    for (int q = tid; q < np; q += 64) {
      const float mq = P0[(q * r + j) * (D + 2)];
      const float w = mq == -INFINITY ? 0.f : exp2f(mq - M);
      wq[q] = w;
      L += P0[(q * r + j) * (D + 2) + 1] * w;
    }
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (tid == 0) {
      const float wf = m == -INFINITY ? 0.f : exp2f(m - M);
      Wf = wf;
      Ls = L + l * wf;
    }
  }
  __syncthreads();
  if (tid < D) {
    float v = 0.f;
#pragma unroll 4
    for (int q = 0; q < np; ++q) v += wq[q] * P0[(q * r + j) * (D + 2) + 2 + tid];
    // fp16 rows: sum the row slices of channel tid
    const int c2 = tid >> 1, hi = tid & 1;
    float fp = 0.f;
    for (int q = 0; q < nvsl; ++q) fp += red[2 * (q * ncp + c2) + hi];
    v += fp * Wf;
    a.out[((int64_t)b * sh.Hq + g * r + j) * D + tid] = v / Ls;
  }
}

}  // namespace

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t st);

// Split-K decode: one kernel writes a partial (m, l, acc) per (split, stream) into the
// workspace, a second merges them per stream in fixed order.  The kernel boundary orders the
// two across the XCDs' separate L2 caches without device-scope fences inside a kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  hipError_t e;
  if (a.fast) {
    e = launch_decode_fast(a, st);
  } else if (a.nparts > 0) {
    dim3 grid(a.nparts, a.sh.B * a.sh.Hkv);
    hipLaunchKernelGGL(k_decode, grid, dim3(DNT), 0, st, a);
    e = hipGetLastError();
  } else {
    e = hipSuccess;
  }
  if (e != hipSuccess) return e;
  if (a.sh.fmt == KVQ_FMT_TQ)
    hipLaunchKernelGGL(k_decode_merge, dim3(a.sh.B * a.sh.Hkv), dim3(DNT), 0, st, a);
  else
    hipLaunchKernelGGL(k_merge_heads, dim3(a.sh.B * a.sh.Hkv, a.sh.Hq / a.sh.Hkv), dim3(MNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
