// Sink selection ("KVSink-Adapted Sink Protection", "How it works", step 1,
// and "Fidelity to the paper": key-norm proxy, prefill-dominant, no retroactive
// restore).  One workgroup per batch element:
//   score_t = (sum over KV heads, in order, of sqrt(canonical sumsq of K[b,h,t,:])) / Hkv
// is folded into the running top-k (rank: score descending, position
// ascending); new rows of the merged top-k join the permanent sink set while
// it has room.  While the set is not full the running top-k equals it, so the
// set and its scores are the whole state.
#include "device_common.h"

namespace kvq {
namespace {

constexpr int NT = 256;
constexpr int NW = NT / 64;

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

  // per-wave running top-K over rows w, w + NW, ...
  for (int t = w; t < a.n; t += NW) {
    float acc = 0.f;
    for (int h = 0; h < sh.Hkv; ++h) {
      const int64_t row = (((int64_t)b * sh.Hkv + h) * a.n + t) * D;
      const bool act = 2 * lane < D;
      const float x0 = act ? ld_in(a.k, row + 2 * lane, sh.in_f32) : 0.f;
      const float x1 = act ? ld_in(a.k, row + 2 * lane + 1, sh.in_f32) : 0.f;
      acc = acc + sqrtf(wave_sumsq(x0, x1, D));
    }
    const Cand c{acc / (float)sh.Hkv, (int)(a.P + t)};
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
  __syncthreads();
  if (tid != 0) return;
  // merge the committed set (its scores) with the wave lists; commit new rows in rank order
  const int cnt = lv.sink_count[b];
  Cand all[MAX_SINK * (NW + 1)];
  int n = 0;
  for (int i = 0; i < cnt; ++i) all[n++] = Cand{lv.sink_score[b * K + i], lv.sink_pos[b * K + i]};
  for (int q = 0; q < NW; ++q)
    for (int i = 0; i < ntop[q]; ++i) all[n++] = top[q][i];
  for (int i = 1; i < n; ++i) {  // insertion sort by rank
    Cand c = all[i];
    int j = i;
    while (j > 0 && before(c, all[j - 1])) {
      all[j] = all[j - 1];
      --j;
    }
    all[j] = c;
  }
  int m = cnt;
  for (int i = 0; i < n && i < K; ++i) {
    if (all[i].p >= a.P && m < K) {
      lv.sink_pos[b * K + m] = all[i].p;
      lv.sink_score[b * K + m] = all[i].s;
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
