// Sink selection ("KVSink-Adapted Sink Protection", "How it works", step 1,
// and "Fidelity to the paper": key-norm proxy, prefill-dominant, no retroactive
// restore).  For each batch element b:
//   score_t = (sum over KV heads, in order, of sqrt(canonical sumsq of K[b,h,t,:])) / Hkv
// is folded into the running top-k (rank: score descending, position
// ascending); new rows of the merged top-k join the permanent sink set while
// it has room.  While the set is not full the running top-k equals it, so the
// set and its scores are the whole state.
//
// Rows are read 16 bytes per lane: one load instruction covers 64 / LR
// consecutive tokens of one head (LR lanes per row), and the canonical sum of
// squares (pair products, then halving) is formed with in-row DPP moves for the
// halvings that cross lanes and in-register adds for the rest, in exactly the
// canonical order.  Each wave keeps its own sorted top-k in registers (entry i
// in lane i; k <= 16, so the list is one DPP row), and every merge is more
// insertions into such a list.  A chunk of at most 64 rows takes one workgroup
// per batch element, whose first wave merges the other waves' lists and the
// committed set and commits; a longer chunk is split over up to 64 workgroups
// per batch element, each writing its top-k to the cache's selection work area,
// and a one-wave kernel per batch element merges those lists.  The rank is a
// total order, so the merge order never changes the result.
#include "device_common.h"

namespace kvq {
namespace {

constexpr int PNT = 256;       // threads of a row workgroup
constexpr int PNW = PNT / 64;  // its waves
constexpr int HB = 8;          // heads per round of loads
constexpr int RB = 2;          // load instructions (token groups) per head per round
constexpr int EMPTY_P = 0x7FFFFFFF;

struct Cand {
  float s;
  int p;
};
__device__ __forceinline__ bool before(float as, int ap, float bs, int bp) {
  return as > bs || (as == bs && ap < bp);
}
__device__ __forceinline__ bool before(const Cand& a, const Cand& b) { return before(a.s, a.p, b.s, b.p); }

// Value of lane (l + M) for lanes l whose partner lies in the same row group (others: don't care).
template <int M>
__device__ __forceinline__ float from_up(float v) {
  if constexpr (M < 16) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x100 + M, 0xF, 0xF,
                                                                 false));  // row_shl:M
  } else {
    return __shfl_down(v, M);
  }
}

// Cross-lane halvings: lane offsets M, M/2, ..., 1 on the Q pair sums each lane holds.
template <int M, int Q>
__device__ __forceinline__ void cross_halvings(float (&a)[Q]) {
  if constexpr (M >= 1) {
#pragma unroll
    for (int i = 0; i < Q; ++i) a[i] = a[i] + from_up<M>(a[i]);
    cross_halvings<M / 2, Q>(a);
  }
}

// Canonical sum of squares of one row held 16 bytes per lane (E elements, Q = E/2 pairs per lane,
// LR = D/E lanes per row).  Pair sums a_l for l = jQ .. jQ+Q-1 sit in lane j of the row group; the
// halving a[l] + a[l + h] pairs lane j with lane j + h/Q while h >= Q and stays in the lane after.
// Lane 0 of each row group ends with the sum.
template <int ESZ, int D>
__device__ __forceinline__ float row_sumsq(const uint4& w) {
  constexpr int E = 16 / ESZ, Q = E / 2, LR = D / E;
  float x[E];
  if constexpr (ESZ == 2) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] & 0xFFFFu));
      x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[i] >> 16));
    }
  } else {
    x[0] = __builtin_bit_cast(float, w.x);
    x[1] = __builtin_bit_cast(float, w.y);
    x[2] = __builtin_bit_cast(float, w.z);
    x[3] = __builtin_bit_cast(float, w.w);
  }
  float a[Q];
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const float p = x[2 * i] * x[2 * i];
    const float q = x[2 * i + 1] * x[2 * i + 1];
    a[i] = p + q;
  }
  cross_halvings<LR / 2, Q>(a);
#pragma unroll
  for (int hq = Q / 2; hq >= 1; hq >>= 1)
#pragma unroll
    for (int i = 0; i < hq; ++i) a[i] = a[i] + a[i + hq];
  return a[0];
}

// Sorted per-wave top-k held one entry per lane (lanes >= n hold don't-care values).
struct WaveTop {
  float s;
  int p;
  int n;              // entries held (uniform)
  float ks;           // k-th entry once n == K (uniform)
  int kp;
};

__device__ __forceinline__ float rdl(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Value of lane l - 1 in lane l of each 16-lane row (row_shr:1; lane 0 of a row keeps its own).
__device__ __forceinline__ int row_up(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x111, 0xF, 0xF, false); }
__device__ __forceinline__ float row_up(float v) { return __builtin_bit_cast(float, row_up(__builtin_bit_cast(int, v))); }

// Inserts the offered candidates (cs, cp) of the lanes with `offer` into the wave's list, in lane
// order (the result does not depend on it): a ballot keeps the ones that beat the k-th entry, and
// each is placed by one ballot (its rank) and one in-row shift of the entries behind it.
__device__ __forceinline__ void wave_insert(WaveTop& T, float cs, int cp, bool offer, int K, int lane) {
  uint64_t m = __ballot(offer && (T.n < K || before(cs, cp, T.ks, T.kp)));
  while (m) {
    const int src = __builtin_ctzll(m);
    m &= m - 1;
    const float s = rdl(cs, src);
    const int p = __builtin_amdgcn_readlane(cp, src);
    if (T.n == K && !before(s, p, T.ks, T.kp)) continue;  // the k-th entry improved meanwhile
    const int pos = __popcll(__ballot(lane < T.n && before(T.s, T.p, s, p)));
    const float us = row_up(T.s);
    const int up = row_up(T.p);
    if (lane > pos) {
      T.s = us;
      T.p = up;
    }
    if (lane == pos) {
      T.s = s;
      T.p = p;
    }
    T.n = T.n < K ? T.n + 1 : K;
    if (T.n == K) {
      T.ks = rdl(T.s, K - 1);
      T.kp = __builtin_amdgcn_readlane(T.p, K - 1);
    }
  }
}

// The new rows (p >= P) of the merged list join the set in rank order while it has room (lane 0
// stores).
__device__ __forceinline__ void commit(const LayerView& lv, int b, int K, int cnt, const WaveTop& T, int64_t P,
                                       int lane) {
  int m = cnt;
  for (int i = 0; i < T.n; ++i) {
    const float s = rdl(T.s, i);
    const int p = __builtin_amdgcn_readlane(T.p, i);
    if (p >= P && m < K) {
      if (lane == 0) {
        lv.sink_pos[b * K + m] = p;
        lv.sink_score[b * K + m] = s;
      }
      ++m;
    }
  }
  if (lane == 0) lv.sink_count[b] = m;
}

template <int ESZ, int D, bool FINAL>
__global__ __launch_bounds__(PNT) void k_select_rows(SelectArgs a) {
  constexpr int E = 16 / ESZ, LR = D / E, RPW = 64 / LR;
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int b = blockIdx.x, g = blockIdx.y, G = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = sh.n_sink, H = sh.Hkv;
  const int cnt = lv.sink_count[b];
  if (cnt >= K) return;  // the set is full: nothing more joins

  // rows [tb, te) of the chunk for this workgroup
  const int per = (a.n + G - 1) / G;
  const int tb = g * per, te = min(a.n, tb + per);
  const int j = lane % LR, rg = lane / LR;
  const char* kb = static_cast<const char*>(a.k);

  WaveTop T{-INFINITY, EMPTY_P, 0, -INFINITY, EMPTY_P};
  for (int t0 = tb + w * RPW * RB; t0 < te; t0 += PNW * RPW * RB) {
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;
    for (int h0 = 0; h0 < H; h0 += HB) {
      uint4 raw[RB][HB];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {  // every load of the round first
          const int h = h0 + hh, t = t0 + r * RPW + rg;
          raw[r][hh] = make_uint4(0u, 0u, 0u, 0u);
          if (h < H && t < te) {
            const int64_t row = ((int64_t)b * H + h) * a.n + t;
            raw[r][hh] = *reinterpret_cast<const uint4*>(kb + (row * D + j * E) * ESZ);
          }
        }
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int hh = 0; hh < HB; ++hh)
          if (h0 + hh < H) acc[r] = acc[r] + sqrtf(row_sumsq<ESZ, D>(raw[r][hh]));
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r * RPW + rg;
      wave_insert(T, acc[r] / (float)H, (int)(a.P + t), j == 0 && t < te, K, lane);
    }
  }

  // workgroup merge: the first wave inserts the other waves' lists (and, for a single workgroup, the
  // committed set) into its own
  __shared__ Cand lists[PNW - 1][MAX_SINK];
  __shared__ int nlist[PNW - 1];
  if (w > 0) {
    if (lane < T.n) lists[w - 1][lane] = Cand{T.s, T.p};
    if (lane == 0) nlist[w - 1] = T.n;
  }
  __syncthreads();
  if (w > 0) return;
  {
    const int q = lane / MAX_SINK, i = lane % MAX_SINK;  // lanes 0 .. 47: the three other lists
    const bool ok = q < PNW - 1 && i < nlist[q < PNW - 1 ? q : 0];
    const Cand c = ok ? lists[q < PNW - 1 ? q : 0][i] : Cand{-INFINITY, EMPTY_P};
    wave_insert(T, c.s, c.p, ok, K, lane);
  }
  if (FINAL) {
    const bool ok = lane < cnt;
    const float cs = ok ? lv.sink_score[b * K + lane] : -INFINITY;
    const int cp = ok ? lv.sink_pos[b * K + lane] : EMPTY_P;
    wave_insert(T, cs, cp, ok, K, lane);
    commit(lv, b, K, cnt, T, a.P, lane);
  } else if (lane < K) {
    a.work[((int64_t)b * SELECT_GMAX + g) * K + lane] =
        lane < T.n ? make_int2(__builtin_bit_cast(int, T.s), T.p)
                   : make_int2(__builtin_bit_cast(int, -INFINITY), EMPTY_P);
  }
}

// Merge of the per-workgroup lists of a split chunk with the committed set: one wave per batch
// element inserts every list entry (64 per round), then the committed set, and commits.
__global__ __launch_bounds__(64) void k_select_merge(SelectArgs a, int G) {
  const LayerView lv = a.lv;
  const int b = blockIdx.x, lane = threadIdx.x, K = a.sh.n_sink;
  const int cnt = lv.sink_count[b];
  if (cnt >= K) return;
  WaveTop T{-INFINITY, EMPTY_P, 0, -INFINITY, EMPTY_P};
  const int nc = K * G;
  for (int i0 = 0; i0 < nc; i0 += 64) {
    const int i = i0 + lane;
    int2 e = make_int2(0, EMPTY_P);
    if (i < nc) e = a.work[((int64_t)b * SELECT_GMAX + i / K) * K + i % K];
    wave_insert(T, __builtin_bit_cast(float, e.x), e.y, e.y != EMPTY_P, K, lane);
  }
  const bool ok = lane < cnt;
  const float cs = ok ? lv.sink_score[b * K + lane] : -INFINITY;
  const int cp = ok ? lv.sink_pos[b * K + lane] : EMPTY_P;
  wave_insert(T, cs, cp, ok, K, lane);
  commit(lv, b, K, cnt, T, a.P, lane);
}

template <int ESZ, int D>
hipError_t launch_rows(const SelectArgs& a, int G, hipStream_t st) {
  if (G == 1) {
    hipLaunchKernelGGL((k_select_rows<ESZ, D, true>), dim3(a.sh.B, 1), dim3(PNT), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_select_rows<ESZ, D, false>), dim3(a.sh.B, G), dim3(PNT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_select_merge, dim3(a.sh.B), dim3(64), 0, st, a, G);
  return hipGetLastError();
}

}  // namespace

int select_groups(int n) {
  const int g = (n + SELECT_MIN_ROWS - 1) / SELECT_MIN_ROWS;
  return g < 1 ? 1 : (g > SELECT_GMAX ? SELECT_GMAX : g);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const int G = select_groups(a.n);
  const int D = a.sh.D;
  if (a.sh.in_f32) {
    if (D == 32) return launch_rows<4, 32>(a, G, st);
    if (D == 64) return launch_rows<4, 64>(a, G, st);
    if (D == 128) return launch_rows<4, 128>(a, G, st);
  } else {
    if (D == 32) return launch_rows<2, 32>(a, G, st);
    if (D == 64) return launch_rows<2, 64>(a, G, st);
    if (D == 128) return launch_rows<2, 128>(a, G, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
