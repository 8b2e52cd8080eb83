// Sink selection ("KVSink-Adapted Sink Protection", "How it works", step 1,
// and "Fidelity to the paper": key-norm proxy, prefill-dominant, no retroactive
// restore).  One workgroup per batch element:
//   score_t = (sum over KV heads, in order, of sqrt(canonical sumsq of K[b,h,t,:])) / Hkv
// is folded into the running top-k (rank: score descending, position
// ascending); new rows of the merged top-k join the permanent sink set while
// it has room.  While the set is not full the running top-k equals it, so the
// set and its scores are the whole state.  Sixteen waves take interleaved rows;
// each wave requests the K rows of all heads of its next rows at once (up to
// HB heads per round trip), keeps its own top-k, and thread 0 merges the wave
// lists (the rank is a total order, so the merge order does not matter).
#include "device_common.h"

namespace kvq {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int HB = 8;  // heads per round of loads
constexpr int RB = 2;  // rows per round of loads

struct Cand {
  float s;
  int p;
};
__device__ __forceinline__ bool before(const Cand& a, const Cand& b) {
  return a.s > b.s || (a.s == b.s && a.p < b.p);
}

__global__ __launch_bounds__(NT) void k_select(SelectArgs a) {
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = sh.n_sink, D = sh.D;
  __shared__ Cand top[NW][MAX_SINK];
  __shared__ int ntop[NW];
  __shared__ int full;
  if (tid == 0) full = lv.sink_count[b] >= K;
  if (tid < NW) ntop[tid] = 0;
  __syncthreads();
  if (full) return;

  // per-wave running top-K over rows w, w + NW, ...: RB rows per round trip
  const bool act = 2 * lane < D;
  for (int t0 = w; t0 < a.n; t0 += NW * RB) {
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;
    for (int h0 = 0; h0 < sh.Hkv; h0 += HB) {
      float x0[RB][HB], x1[RB][HB];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {  // every load of the round first
          const int h = h0 + hh, t = t0 + NW * r;
          const bool ok = act && h < sh.Hkv && t < a.n;
          const int64_t row = (((int64_t)b * sh.Hkv + h) * a.n + t) * D;
          x0[r][hh] = ok ? ld_in(a.k, row + 2 * lane, sh.in_f32) : 0.f;
          x1[r][hh] = ok ? ld_in(a.k, row + 2 * lane + 1, sh.in_f32) : 0.f;
        }
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh)
          if (h0 + hh < sh.Hkv) acc[r] = acc[r] + sqrtf(wave_sumsq(x0[r][hh], x1[r][hh], D));
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + NW * r;
      if (t >= a.n) break;
      const Cand c{acc[r] / (float)sh.Hkv, (int)(a.P + t)};
      if (lane == 0) {
        int n = ntop[w];
        int i = n < K ? n : K - 1;
        if (n < K || before(c, top[w][K - 1])) {
          // insertion into the sorted list
          while (i > 0 && before(c, top[w][i - 1])) {
            top[w][i] = top[w][i - 1];
            --i;
          }
          top[w][i] = c;
          if (n < K) ntop[w] = n + 1;
        }
      }
    }
  }
  __syncthreads();
  // merge: the committed set (with its scores) and the wave lists as one candidate array; every
  // candidate's rank is the number of candidates before it (the rank order is total), the first K
  // land in rank order, and thread 0 commits the new ones among them in that order
  constexpr int NC = MAX_SINK * (NW + 1);
  __shared__ Cand cand[NC];
  __shared__ Cand best[MAX_SINK];
  __shared__ int nbest;
  const int cnt = lv.sink_count[b];
  if (tid < NC) {
    const int q = tid / MAX_SINK, i = tid % MAX_SINK;
    Cand c{-INFINITY, 0x7FFFFFFF};  // empty slot: ranked after every real candidate
    if (q < NW) {
      if (i < ntop[q]) c = top[q][i];
    } else if (i < cnt) {
      c = Cand{lv.sink_score[b * K + i], lv.sink_pos[b * K + i]};
    }
    cand[tid] = c;
  }
  if (tid == 0) {
    int nv = cnt;
    for (int q = 0; q < NW; ++q) nv += ntop[q];
    nbest = nv < K ? nv : K;  // ranks 0 .. nbest - 1 are taken
  }
  __syncthreads();
  if (tid < NC && cand[tid].p != 0x7FFFFFFF) {
    const Cand c = cand[tid];
    int r = 0;
    for (int j = 0; j < NC; ++j) r += before(cand[j], c);
    if (r < K) best[r] = c;
  }
  __syncthreads();
  if (tid != 0) return;
  int m = cnt;
  const int nb = nbest;
  for (int i = 0; i < nb; ++i) {
    if (best[i].p >= a.P && m < K) {
      lv.sink_pos[b * K + m] = best[i].p;
      lv.sink_score[b * K + m] = best[i].s;
      ++m;
    }
  }
  lv.sink_count[b] = m;
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(a.sh.B), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvq
