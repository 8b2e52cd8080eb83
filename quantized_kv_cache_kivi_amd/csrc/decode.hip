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

// MD: the widest stored row the instance takes (128, or 256 for TurboQuant rows of head_dim 160).
template <int MD>
__global__ __launch_bounds__(DNT) void k_decode(DecodeArgs a) {
  __shared__ Smem<MD> S;
  generic_partial<MD>(a, S);
}

template <int MD>
__global__ __launch_bounds__(DNT) void k_decode_merge(DecodeArgs a) {
  __shared__ Smem<MD> S;
  merge_partials<MD>(a, S);
}

constexpr int MNT = 256;  // threads of a merge workgroup
constexpr int MNP = 8;    // fp16 row passes per chunk (a pass covers MNT / (D/8) rows)
constexpr int MPF = 16;   // split partials a thread fetches before the fp16 rows are scored

typedef uint32_t mu4 __attribute__((ext_vector_type(4)));

// q[0..7] . (8 fp16 values of w)
__device__ __forceinline__ float dot8(const float* q, const mu4& w) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  float d = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    d = fmaf(q[2 * k], f16_val((uint16_t)(ww[k] & 0xFFFFu)), d);
    d = fmaf(q[2 * k + 1], f16_val((uint16_t)(ww[k] >> 16)), d);
  }
  return d;
}

// Online-softmax state of the fp16 rows of one (stream, head): m is block-uniform; l and the
// 8-channel accumulator are per thread (rows of its row slot).
struct FpState {
  float m, l, acc[8];
};

// Folds a set of K scores (one per pass of this thread's row slot; -inf where masked) and their
// V rows into the state.  The block-wide maximum takes two barriers.
template <int K>
__device__ __forceinline__ void fp_update(FpState& st, const float (&sc)[K], const mu4 (&v)[K], bool counts,
                                          float* wred, int lane, int wv) {
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < K; ++k) mx = fmaxf(mx, sc[k]);
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) wred[wv] = mx;
  lds_barrier();
  float M = wred[0];
#pragma unroll
  for (int w = 1; w < MNT / 64; ++w) M = fmaxf(M, wred[w]);
  lds_barrier();
  const float mnew = fmaxf(st.m, M);
  if (mnew == -INFINITY) return;  // nothing valid yet (uniform)
  const float f = st.m == -INFINITY ? 0.f : exp2f(st.m - mnew);
  float lsum = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.acc[c] *= f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float w = sc[k] == -INFINITY ? 0.f : exp2f(sc[k] - mnew);
    lsum += w;
    const uint32_t vv[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      st.acc[2 * c] = fmaf(w, f16_val((uint16_t)(vv[c] & 0xFFFFu)), st.acc[2 * c]);
      st.acc[2 * c + 1] = fmaf(w, f16_val((uint16_t)(vv[c] >> 16)), st.acc[2 * c + 1]);
    }
  }
  st.l = st.l * f + (counts ? lsum : 0.f);  // one lane per row counts the row's weight
  st.m = mnew;
}

// Window rows [c0, c0 + MNP * rpp) of this thread's row slot (rows past the window read row 0).
__device__ __forceinline__ void load_window(mu4 (&kr)[MNP], mu4 (&vr)[MNP], const uint16_t* wk, const uint16_t* wv,
                                            int c0, int rs, int rpp, int nwin, int slot0, int R, int D) {
#pragma unroll
  for (int k = 0; k < MNP; ++k) {
    const int row = c0 + rs + k * rpp;
    const int rr = row < nwin ? row : 0;  // clamped: the load is always in bounds
    int sl = slot0 + rr;
    if (sl >= R) sl -= R;
    kr[k] = *reinterpret_cast<const mu4*>(wk + (int64_t)sl * D);
    vr[k] = *reinterpret_cast<const mu4*>(wv + (int64_t)sl * D);
  }
}

// Merge for formats without a rotation: one workgroup per (stream, query head).  Every load is
// issued before any is used (sink slots, query slice, split partials, sink-pool rows, the first
// chunk of window rows; clamped addresses instead of branches); the fp16 rows (window rows
// [bulk_hi, P) minus committed sinks, then the sink pool in slot order) are scored with D/8 lanes
// per row and folded in with an online maximum; the bulk partials of the head are then merged in
// split order.
__global__ __launch_bounds__(MNT) void k_merge_heads(DecodeArgs a) {
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int s = blockIdx.x, j = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = sh.D, r = sh.Hq / sh.Hkv, b = s / sh.Hkv, g = s % sh.Hkv, ns = sh.n_sink;
  const int lpr = D / 8, rpp = MNT / lpr, part = tid % lpr, rs = tid / lpr;
  __shared__ int spos[MAX_SINK];  // position of each sink-pool slot; -1 unless a committed sink < P
  __shared__ int wsk[MAX_SINK];   // window rows holding a committed sink (read from the pool instead)
  __shared__ int nwsk;
  __shared__ float wred[MNT / 64];
  __shared__ float red[MNT * 8];
  __shared__ float wq[65];
  __shared__ float Ls, Wf;

  const int nwin = (int)(a.P - a.bulk_hi);  // positions fit in int32
  const int np = a.nparts;
  const float* P0 = a.ws + (int64_t)s * np * r * (D + 2);

  // ---- loads (branch-free: an empty source is replaced by an always-valid one and masked later) ----
  const int cnt = lv.sink_count[b];
  const int praw = *(ns > 0 ? lv.sink_pos + b * ns + min(tid, ns - 1) : lv.sink_count + b);
  // query slice: one 16-byte load (fp16) or two (fp32)
  const int64_t qo = ((int64_t)b * sh.Hq + (int64_t)g * r + j) * sh.Din + 8 * part;  // Din = D here (not TQ)
  const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qo * (sh.in_f32 ? 4 : 2);
  const mu4 qw0 = *reinterpret_cast<const mu4*>(qp);
  const mu4 qw1 = *reinterpret_cast<const mu4*>(qp + (sh.in_f32 ? 16 : 0));
  const int npc = max(np, 1);  // the workspace always holds one partial per stream
  float pm = P0[(min(tid, npc - 1) * r + j) * (D + 2)];
  float pl = P0[(min(tid, npc - 1) * r + j) * (D + 2) + 1];
  float pv[MPF];
#pragma unroll
  for (int q = 0; q < MPF; ++q) pv[q] = P0[(min(q, npc - 1) * r + j) * (D + 2) + 2 + min(tid, D - 1)];
  const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + 8 * part;  // stand-in row source
  const uint16_t* skp = ns > 0 ? lv.sink_k + ((int64_t)s * ns + min(rs, ns - 1)) * D + 8 * part : q16;
  const uint16_t* svp = ns > 0 ? lv.sink_v + ((int64_t)s * ns + min(rs, ns - 1)) * D + 8 * part : q16;
  const mu4 sk = *reinterpret_cast<const mu4*>(skp);
  const mu4 svv = *reinterpret_cast<const mu4*>(svp);
  const int slot0 = nwin > 0 ? (int)(a.bulk_hi % sh.R) : 0;
  const int rring = max(sh.R, 1);
  const uint16_t* wk = nwin > 0 ? lv.win_k + ((int64_t)s * sh.R) * D + 8 * part : q16;
  const uint16_t* wvp = nwin > 0 ? lv.win_v + ((int64_t)s * sh.R) * D + 8 * part : q16;
  mu4 kr[MNP], vr[MNP];
  load_window(kr, vr, wk, wvp, 0, rs, rpp, nwin, slot0, rring, D);

  // ---- uses ----
  if (tid < ns) spos[tid] = (tid < min(cnt, ns) && praw >= 0 && praw < a.P) ? praw : -1;
  if (tid >= np) {
    pm = -INFINITY;
    pl = 0.f;
  }
  if (np == 0) {
#pragma unroll
    for (int q = 0; q < MPF; ++q) pv[q] = 0.f;
  }
  const float mult = a.scale * LOG2E;
  float qv[8];
  if (sh.in_f32) {
    const uint32_t ww[8] = {qw0.x, qw0.y, qw0.z, qw0.w, qw1.x, qw1.y, qw1.z, qw1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) qv[k] = __builtin_bit_cast(float, ww[k]);
  } else {
    const uint32_t ww[4] = {qw0.x, qw0.y, qw0.z, qw0.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qv[2 * k] = f16_val((uint16_t)(ww[k] & 0xFFFFu));
      qv[2 * k + 1] = f16_val((uint16_t)(ww[k] >> 16));
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) qv[k] *= mult;
  lds_barrier();
  if (tid < 64) {  // committed sinks inside the window
    const int p = lane < ns ? spos[lane] : -1;
    const bool in = p >= 0 && p >= a.bulk_hi && p < a.P;
    const uint64_t msk = __ballot(in);
    if (in) wsk[__popcll(msk & ((1ull << lane) - 1ull))] = (int)(p - a.bulk_hi);
    if (lane == 0) nwsk = __popcll(msk);
  }
  lds_barrier();
  const int nw = nwsk;

  FpState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.acc[c] = 0.f;
  // window rows, chunk by chunk
  for (int c0 = 0; c0 < nwin; c0 += MNP * rpp) {
    if (c0 > 0) load_window(kr, vr, wk, wvp, c0, rs, rpp, nwin, slot0, rring, D);
#pragma unroll
    for (int k = 0; k < MNP; ++k)
      if (c0 + rs + k * rpp >= nwin) kr[k] = vr[k] = mu4{0, 0, 0, 0};
    float sc[MNP];
#pragma unroll
    for (int k = 0; k < MNP; ++k) {
      float d = dot8(qv, kr[k]);
      for (int off = lpr / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      const int row = c0 + rs + k * rpp;
      bool ok = row < nwin;
      for (int q = 0; q < nw; ++q) ok = ok && wsk[q] != row;
      sc[k] = ok ? d : -INFINITY;
    }
    fp_update(st, sc, vr, part == 0, wred, lane, wv);
  }
  // sink pool rows (slot order), one pass
  {
    float d = dot8(qv, sk);
    for (int off = lpr / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
    const bool ok = rs < ns && spos[rs] >= 0;
    const float sc1[1] = {ok ? d : -INFINITY};
    const mu4 v1[1] = {ok ? svv : mu4{0, 0, 0, 0}};
    fp_update(st, sc1, v1, part == 0, wred, lane, wv);
  }

  // ---- reduce the fp16 state over the row slots ----
  float lt = st.l;
  for (int off = 32; off >= 1; off >>= 1) lt += __shfl_xor(lt, off);
  if (lane == 0) wred[wv] = lt;
#pragma unroll
  for (int c = 0; c < 8; ++c) red[rs * D + 8 * part + c] = st.acc[c];
  lds_barrier();
  float lfp = 0.f;
#pragma unroll
  for (int w = 0; w < MNT / 64; ++w) lfp += wred[w];
  // ---- weights of the bulk partials and of the fp16 rows ----
  if (tid < 64) {
    float M = fmaxf(st.m, pm);  // np <= 64: lane q holds split q
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = pm == -INFINITY ? 0.f : exp2f(pm - M);
    if (tid < np) wq[tid] = w;
    float L = pl * w;
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (tid == 0) {
      const float wf = st.m == -INFINITY ? 0.f : exp2f(st.m - M);
      Wf = wf;
      Ls = L + lfp * wf;
    }
  }
  lds_barrier();
  if (tid < D) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < MPF; ++q)
      if (q < np) v += wq[q] * pv[q];
    for (int q = MPF; q < np; ++q) v += wq[q] * P0[(q * r + j) * (D + 2) + 2 + tid];
    float fp = 0.f;
    for (int q = 0; q < rpp; ++q) fp += red[q * D + tid];
    v += fp * Wf;
    a.out[((int64_t)b * sh.Hq + g * r + j) * sh.Din + tid] = v / Ls;
  }
}

}  // namespace

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t st);

// Split-K decode: one kernel writes a partial (m, l, acc) per (split, stream) into the
// workspace, a second merges them per stream in fixed order.  The kernel boundary orders the
// two across the XCDs' separate L2 caches without device-scope fences inside a kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.fast) return launch_decode_fast(a, st);  // split kernel (bulk and fp16 rows) and its merge
  hipError_t e;
  if (a.nparts > 0) {
    dim3 grid(a.nparts, a.sh.B * a.sh.Hkv);
    if (a.sh.D > MAX_D) hipLaunchKernelGGL(k_decode<MAX_SD>, grid, dim3(DNT), 0, st, a);
    else hipLaunchKernelGGL(k_decode<MAX_D>, grid, dim3(DNT), 0, st, a);
    e = hipGetLastError();
  } else {
    e = hipSuccess;
  }
  if (e != hipSuccess) return e;
  if (a.sh.D > MAX_D)
    hipLaunchKernelGGL(k_decode_merge<MAX_SD>, dim3(a.sh.B * a.sh.Hkv), dim3(DNT), 0, st, a);
  else if (a.sh.fmt == KVQ_FMT_TQ || a.sh.rope)
    hipLaunchKernelGGL(k_decode_merge<MAX_D>, dim3(a.sh.B * a.sh.Hkv), dim3(DNT), 0, st, a);
  else
    hipLaunchKernelGGL(k_merge_heads, dim3(a.sh.B * a.sh.Hkv, a.sh.Hq / a.sh.Hkv), dim3(MNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
