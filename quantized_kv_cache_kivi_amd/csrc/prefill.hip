// Causal multi-query attention of a prefill chunk over the quantized cache: the queries of the last
// n appended positions P-n .. P-1 attend the valid positions (sinks, fp16 window, quantized bulk,
// read priority as in decode attention) that are not after their own position.  Dequantization
// follows "StreamingLLM + KIVI" ("Affine quantisation formula") and the q2k page ("Summary": Gaussian
// Lloyd-Max K levels times the block RMS, symmetric 4-bit V); the attention itself is the plain
// softmax attention of decode, with a causal limit per query.
//
// One workgroup per (stream, tile of queries); its waves each own one or two tiles of 16 MFMA columns
// (16 / r queries times the r query heads of the KV head): 4 waves of 2 tiles (KIVI), 8 waves of 1
// (q2k), 4 waves of 1 (TurboQuant; RoPE and fp32 queries on short chunks).  Key/value rows are taken 32 at a time
// ("row blocks": a bulk block, or up to 32 fp16 window rows, or the sinks): the workgroup
// dequantizes a row block once into LDS (K and V as fp16 hi + lo halves whose sum is the fp32
// value, V transposed into the matrix-core token order), then every wave runs
//   scores = K . q  (v_mfma_f32_16x16x32_f16, hi and lo halves into one accumulator),
// the online softmax of its columns in registers (log2 units), and
//   acc += V^T . p  (the weights, split into fp16 hi + lo, enter as the B operand straight from the
//                    score registers: the score lane layout is the token order of the V tile;
//                    V_hi p_hi + V_hi p_lo + V_lo p_hi).
// Row blocks after a tile's last query are skipped; within a row block every column masks the rows
// after its own position.
#include "device_common.h"

namespace kvq {
constexpr int PT = 2;     // 16-column tiles per wave (block formats)
namespace {

// Waves per workgroup (a template parameter of the kernel) and 16-column tiles per wave.  KIVI: 4
// waves of 2 tiles.  With 8 waves of 2 tiles (one staged row block feeding 8 waves) the config-2
// prefill took 5.6 ms instead of 4.9: one 8-wave workgroup per CU (222 VGPRs) leaves no second
// workgroup to compute while one stages; 4 waves of 1 tile (117 VGPRs, 4 waves per SIMD) took 4.5
// ms instead of 4.3.  q2k, whose staging costs more (the level lookups): 8 waves of 1 tile (121
// VGPRs, two workgroups per CU) took its 4096 queries at P = 32768 in 101 ms instead of 117 (4 waves
// of 2 tiles) or 150 (4 waves of 1).  Queries staged through LDS (TurboQuant, RoPE, fp32) need 4
// waves: their staging tile holds 16 columns per wave.
constexpr int PNW_DIRECT = 4, PNW_LDS = 4, PNW_Q2K = 8;
constexpr float PLOG2E = 1.4426950408889634f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(const u4& a, const u4& b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ hv2 HV(uint32_t w) { return __builtin_bit_cast(hv2, w); }

// fp16 hi and lo halves of two fp32 values, packed: hi = x rounded toward zero (one packed
// conversion), lo = rn(x - hi) (x - hi is exact in fp32; one mixed-precision fma per value, written
// into its half).  hi + lo holds x to ~2^-21.  nm1 is -1 held in a register (an fma by a literal -1
// would be rewritten as a subtraction, which the mixed-precision fma does not cover).
__device__ __forceinline__ void split_pair(float a, float b, float nm1, uint32_t& hi, uint32_t& lo) {
  const hv2 h = __builtin_bit_cast(hv2, __builtin_amdgcn_cvt_pkrtz(a, b));
  hi = __builtin_bit_cast(uint32_t, h);
  const hv2 l = hv2{(_Float16)__builtin_fmaf((float)h.x, nm1, a), (_Float16)__builtin_fmaf((float)h.y, nm1, b)};
  lo = __builtin_bit_cast(uint32_t, l);
}

template <int D>
struct PfSmem {
  alignas(16) _Float16 khi[G][D + 8];  // K rows of the row block: fp16 hi halves
  alignas(16) _Float16 klo[G][D + 8];  // fp16 lo halves (value - hi)
  alignas(16) _Float16 vt[D][G + 8];   // V transposed: [channel][slot], slot 8*kq + e <-> row v_tok(kq, e)
  alignas(16) _Float16 vtl[D][G + 8];  // its fp16 lo halves
  int pos[G];                          // position of each row (-1: not attended)
  uint32_t meta[2][256];               // K and V metadata of bulk row blocks (<= 1 KB), by parity
  int spos[MAX_SINK], sslot[MAX_SINK];
  int nsink;
  float kcen[16], vcen[16];  // TurboQuant centroids (rotated domain)
};

template <int FMT, int KB, int VB, int D, bool LQ, int PTT, int PW>
__global__ __launch_bounds__(64 * PW) void k_prefill_attn(PrefillArgs a) {
  constexpr int PNW = PW, PNT = 64 * PW, SL = PNT / G;  // waves and threads per workgroup, staging threads per row
  // TurboQuant works in the rotated domain ("TurboQuant KV Cache Compression — Spec", "Optimization:
  // Fused dequant-dot"): queries rotated once (fp16 hi + lo, a third score product), bulk rows are
  // norm times centroid, fp16 window and sink rows are rotated while staged, outputs rotated back
  // RoPE on read ("StreamingLLM + KIVI", "RoPE caveat"): queries and staged keys turn by their
  // index in the compressed cache; the turned queries are fp16 hi + lo pairs like TurboQuant's.
  // LQ: queries staged through LDS as fp16 hi + lo, for RoPE (sh.rope) or fp32 queries (sh.in_f32).
  constexpr bool TQ = FMT == KVQ_FMT_TQ;
  constexpr bool SQ = TQ || LQ;            // queries split into fp16 hi + lo (third score product)
  constexpr int PT = PTT;  // column tiles per wave
  constexpr int NST = D / 32, NMU = D / 16, NG = D / 32;
  constexpr int VPW = 32 / VB, WPC = D * VB / 64;
  const Shape sh = a.sh;
  const LayerView lv = a.lv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i16 = lane & 15, kg = lane >> 4;
  const int s = blockIdx.y, b = s / sh.Hkv, g = s % sh.Hkv;
  const int R = sh.Hq / sh.Hkv, qpt = 16 / R;          // queries per 16-column tile
  const int QT = PNW * PT * qpt;                        // queries per workgroup
  const int tile = (int)gridDim.x - 1 - (int)blockIdx.x;  // the longest tiles start first
  const int q0 = tile * QT;
  const int qlast = min(a.n - 1, q0 + QT - 1);
  const int64_t pbase = a.P - a.n;  // position of query 0
  const int64_t qmax = pbase + qlast;
  __shared__ PfSmem<D> S;

  if (tid < 64) {  // committed sinks already appended, with their pool slots
    const int ns = sh.n_sink;
    const int cnt = ns > 0 ? lv.sink_count[b] : 0;
    const int praw = lane < ns ? lv.sink_pos[b * ns + lane] : -1;
    const int p = lane < min(cnt, ns) ? praw : -1;
    const bool ok = p >= 0 && p < a.P;
    const uint64_t m = __ballot(ok);
    const int idx = __popcll(m & ((1ull << lane) - 1ull));
    if (ok) {
      S.spos[idx] = p;
      S.sslot[idx] = lane;
    }
    if (lane == 0) S.nsink = __popcll(m);
  }
  __syncthreads();
  // ---- queries of this wave's columns as the B operand (K-dimension slots 8*kg .. of chunk st) ----
  u4 bq[PT][NST], bql[SQ ? PT : 1][SQ ? NST : 1];
  int qpos[PT];  // position of the lane's column query (-1: no query)
  int qidx[PT], head[PT];
  const float cd = (float)(1.0 / __builtin_sqrt((double)D));
  // rows held by one wave: lane l holds channels 128h + 2l + e in element 2h + e (row_chan)
  constexpr int RMD = D > 128 ? 256 : 128, NK = RMD / 64;
  float sg[NK];  // TurboQuant signs of the lane's channels
#pragma unroll
  for (int k = 0; k < NK; ++k) sg[k] = 0.f;
  if constexpr (TQ) {
#pragma unroll
    for (int k = 0; k < NK; ++k) sg[k] = row_chan(lane, k) < D ? lv.tables->signs[row_chan(lane, k)] : 0.f;
    if (tid < 16) S.kcen[tid] = lv.tables->k_cen[tid & ((1 << KB) - 1)];
    if (tid >= 16 && tid < 32) S.vcen[tid - 16] = lv.tables->v_cen[(tid - 16) & ((1 << VB) - 1)];
  }
  auto col_query = [&](int tt, int col, int* qq_out, int* head_out) {
    const int qi = col / R, jj = col % R;
    const int qq = q0 + (wv * PT + tt) * qpt + qi;
    *qq_out = qq;
    *head_out = g * R + jj;
    return qi < qpt && qq < a.n;
  };
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
    int qq, hd;
    const bool ok = col_query(tt, i16, &qq, &hd);
    qidx[tt] = qq;
    head[tt] = hd;
    qpos[tt] = ok ? (int)(pbase + qq) : -1;
    if constexpr (!SQ) {
      const int64_t qrow = (((int64_t)b * sh.Hq + hd) * a.n + qq) * D;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        u4 v = u4{0u, 0u, 0u, 0u};
        if (ok) v = *reinterpret_cast<const u4*>(static_cast<const _Float16*>(a.q) + qrow + 32 * st + 8 * kg);
        bq[tt][st] = v;
      }
    } else {
      // rotate the wave's 16 column queries one by one (lane l holds channels row_chan(l, k)) into
      // a wave-private LDS tile, then read each lane's B-operand slice back as fp16 hi + lo
      float* qs = reinterpret_cast<float*>(&S.khi[0][0]) + wv * 16 * D;
      for (int col = 0; col < 16; ++col) {
        int cq, ch;
        const bool cok = col_query(tt, col, &cq, &ch);
        float y[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) y[k] = 0.f;
        if (!cok) {  // a padding column (uniform over the wave): zeros, nothing to turn
#pragma unroll
          for (int k = 0; k < NK; ++k)
            if (row_chan(lane, k) < D) qs[col * D + row_chan(lane, k)] = 0.f;
          continue;
        }
        const int64_t qrow = (((int64_t)b * sh.Hq + ch) * a.n + cq) * sh.Din;
#pragma unroll
        for (int k = 0; k < NK; k += 2) {
          const int c = row_chan(lane, k);
          if (c < sh.Din) {  // query rows of Din channels (TurboQuant pads the rest with zeros)
            if (sh.in_f32) {
              const float2 w = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + qrow + c);
              y[k] = w.x;
              y[k + 1] = w.y;
            } else {
              const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const _Float16*>(a.q) + qrow + c);
              y[k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
              y[k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
            }
          }
        }
        if constexpr (TQ) {
#pragma unroll
          for (int k = 0; k < NK; ++k) y[k] *= sg[k];
          row_fwht<RMD>(y, D, lane);
#pragma unroll
          for (int k = 0; k < NK; ++k) y[k] *= cd;
        } else if (sh.rope) {  // RoPE: channel 2l pairs with 2l + D/2, held by lane l ^ (D/4)
          const float p0 = __shfl_xor(y[0], D / 4), p1 = __shfl_xor(y[1], D / 4);
          const int qi = cache_index(S.spos, S.nsink, a.lo, pbase + cq);
          const float r0 = rope_val(y[0], p0, 2 * lane, D, qi, lv.tables->rope_inv);
          const float r1 = rope_val(y[1], p1, 2 * lane + 1, D, qi, lv.tables->rope_inv);
          y[0] = r0;
          y[1] = r1;
        }
#pragma unroll
        for (int k = 0; k < NK; ++k)
          if (row_chan(lane, k) < D) qs[col * D + row_chan(lane, k)] = y[k];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float x0 = qs[i16 * D + 32 * st + 8 * kg + 2 * m], x1 = qs[i16 * D + 32 * st + 8 * kg + 2 * m + 1];
          const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
          hw[m] = (uint32_t)h16(x0) | ((uint32_t)h16(x1) << 16);
          lw[m] = (uint32_t)h16(x0 - (float)h0) | ((uint32_t)h16(x1 - (float)h1) << 16);
        }
        bq[tt][st] = u4{hw[0], hw[1], hw[2], hw[3]};
        bql[tt][st] = u4{lw[0], lw[1], lw[2], lw[3]};
      }
    }
  }
  const int nsink = S.nsink;
  auto is_sink = [&](int64_t p) {
    bool r = false;
    for (int q = 0; q < nsink; ++q) r = r || S.spos[q] == p;
    return r;
  };

  float m_[PT], l_[PT];
  f4 acc[PT][NMU];
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
    m_[tt] = -INFINITY;
    l_[tt] = 0.f;
#pragma unroll
    for (int mu = 0; mu < NMU; ++mu) acc[tt][mu] = f4{0.f, 0.f, 0.f, 0.f};
  }
  const float al = a.scale * PLOG2E;
  float nm1 = -1.f;
  asm("" : "+v"(nm1));  // -1 opaque to the optimizer (no instruction): see split_pair
  const float lv0 = FMT == KVQ_FMT_Q2K ? lv.tables->q2k_lvl[0] : 0.f;
  const float lv1 = FMT == KVQ_FMT_Q2K ? lv.tables->q2k_lvl[1] : 0.f;
  const float lv2 = FMT == KVQ_FMT_Q2K ? lv.tables->q2k_lvl[2] : 0.f;
  const float lv3 = FMT == KVQ_FMT_Q2K ? lv.tables->q2k_lvl[3] : 0.f;

  // row blocks: bulk blocks, then fp16 window rows in groups of 32, then the sinks
  const int64_t bhi = a.bulk_hi < qmax + 1 ? a.bulk_hi : qmax + 1;  // bulk rows [lo, bhi)
  const int64_t blk0 = a.lo / G;
  const int nbulk = bhi > a.lo ? (int)((bhi - 1) / G - blk0 + 1) : 0;
  const int64_t whi = a.P < qmax + 1 ? a.P : qmax + 1;  // window rows [bulk_hi, whi)
  const int nwin = whi > a.bulk_hi ? (int)(whi - a.bulk_hi) : 0;
  const int nwblk = (nwin + G - 1) / G;
  const int nrb = nbulk + nwblk + (nsink > 0 ? 1 : 0);
  const int slot0 = (int)(blk0 % lv.cap_b);                        // ring slot of the first bulk block
  const int wslot0 = nwin > 0 ? (int)(a.bulk_hi % sh.R) : 0;        // window slot of row bulk_hi
  const uint8_t* sbase = lv.bulk + (int64_t)s * lv.cap_b * lv.rec;  // this stream's ring

  // split over row blocks (decode-sized calls): this workgroup reads row blocks [rb_lo, rb_hi)
  const int split = blockIdx.z;
  const int rb_lo = (int)((int64_t)nrb * split / a.splits), rb_hi = (int)((int64_t)nrb * (split + 1) / a.splits);
  bool anyq = false;
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) anyq = anyq || qpos[tt] >= 0;
  const bool live = __any(anyq);

  // Block formats load a bulk row block one row block ahead, so the loads of the next one are in
  // flight during this one's matrix work (TurboQuant loads it when it stages it: the registers held
  // across the matrix work would cost its kernel a wave per SIMD).  Loaded: the code words of this
  // thread's K channels and V chunk words into registers, and one dword per thread of the record's
  // metadata (the K and V sections are contiguous), which is staged through LDS.  The barriers of the
  // loop order LDS only, so loads in flight stay in flight across them.
  constexpr bool PF = !TQ;
  constexpr int CPT = D / SL;  // channels per staging thread
  constexpr int KPER = KB == 3 ? 1 : 32 / KB;  // K codes per word (3-bit codes: the dense stream)
  constexpr int KWN = KB == 3 ? 1 : (CPT >= KPER ? CPT / KPER : 1);  // K code words per thread
  constexpr int NWI = (WPC + PNW - 1) / PNW;                          // V code words per thread
  constexpr int KMW = FMT == KVQ_FMT_KIVI ? D : (FMT == KVQ_FMT_Q2K ? D / 2 : G);  // K metadata dwords
  const int t = tid / SL, c0 = (tid % SL) * CPT;
  const int nmeta = (int)((lv.rec - lv.k_meta) / 4);  // <= 256 for every format
  auto rec_of = [&](int rbx) {
    int slot = slot0 + rbx;
    if (slot >= lv.cap_b) slot -= lv.cap_b;
    return sbase + (int64_t)slot * lv.rec;
  };
  uint32_t pkc[KWN], pvc[NWI], pmeta = 0u;
  auto fetch = [&](int rbx) {
    const uint8_t* r = rec_of(rbx);
    if constexpr (KB != 3) {
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(r + lv.k_codes) + t * (D * KB / 32) + c0 / KPER;
#pragma unroll
      for (int j = 0; j < KWN; ++j) pkc[j] = kw[j];
    }
    if constexpr (VB != 3 && PF) {  // (without the look-ahead the V words are read where used)
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(r + lv.v_codes);
#pragma unroll
      for (int n = 0; n < NWI; ++n) {
        const int wi = wv + n * PNW;
        pvc[n] = wi < WPC ? vw[lane * WPC + wi] : 0u;
      }
    }
    if (PF && tid < nmeta) pmeta = reinterpret_cast<const uint32_t*>(r + lv.k_meta)[tid];
  };
  if (PF && rb_lo < nbulk) fetch(rb_lo);

  for (int rb = rb_lo; rb < rb_hi; ++rb) {
    // the metadata loaded ahead goes to the buffer of this row block's parity (last read while row
    // block rb - 2 was staged, before the barrier that ended its staging)
    if (PF && rb < nbulk && tid < nmeta) S.meta[rb & 1][tid] = pmeta;
    lds_barrier();  // the previous row block is consumed; this one's metadata is visible
    // ---- stage the row block: thread (row t, channel slice) for K; chunk-wise for V ----
    if (rb < nbulk) {
      const int64_t beta = blk0 + rb;
      const uint8_t* rec = rec_of(rb);
      // metadata dword i of the record: from LDS (loaded ahead), or read in place
      const uint32_t* md = PF ? S.meta[rb & 1] : reinterpret_cast<const uint32_t*>(rec + lv.k_meta);
      if constexpr (!PF) fetch(rb);  // the code words (TurboQuant's metadata is read in place)
      {  // K: codes of row t, channels c0 .. c0 + CPT - 1, with their metadata
        constexpr int per = KPER;
        uint32_t sc[CPT / 2], zc[CPT / 2];
        float nk = 0.f;  // TurboQuant: the row's K norm
        if constexpr (TQ) {
          nk = __builtin_bit_cast(float, md[t]);
        } else {
#pragma unroll
          for (int i = 0; i < CPT / 2; ++i) {
            sc[i] = md[c0 / 2 + i];
            zc[i] = FMT == KVQ_FMT_KIVI ? md[D / 2 + c0 / 2 + i] : 0u;
          }
        }
        uint32_t hk[CPT / 2], lk[CPT / 2];  // the thread's channels as fp16 hi / lo pairs
#pragma unroll
        for (int i = 0; i < CPT / 2; ++i) {
          float x[2];
          if constexpr (KB == 3) {  // dense 3-bit stream (TurboQuant): one code at a time
#pragma unroll
            for (int h = 0; h < 2; ++h) x[h] = nk * S.kcen[code3_at(rec + lv.k_codes, k_bit3(t, c0 + 2 * i + h, D))];
          } else {
            // channels c, c + 1 (k even): codes k and k + 1 of their word sit at the same bit offset
            // of its two 16-bit halves, so one shift and one mask put both in the halves' low bytes
            const int c = c0 + 2 * i, k = c % per;
            const uint32_t uu = (pkc[c / per - c0 / per] >> (KB * (k >> 1))) & (((1u << KB) - 1u) * 0x10001u);
            const float u0 = (float)(uu & 0xFFu), u1 = (float)(uu >> 16);
            if constexpr (TQ) {
              x[0] = nk * S.kcen[uu & 0xFFFFu];
              x[1] = nk * S.kcen[uu >> 16];
            } else if constexpr (FMT == KVQ_FMT_KIVI) {  // u s + z, one rounding
              const hv2 s2 = HV(sc[i]), z2 = HV(zc[i]);
              x[0] = __builtin_fmaf(u0, (float)s2.x, (float)z2.x);
              x[1] = __builtin_fmaf(u1, (float)s2.y, (float)z2.y);
            } else {
              const hv2 s2 = HV(sc[i]);
              const uint32_t ua = uu & 0xFFFFu, ub = uu >> 16;
              const float la = ua == 0 ? lv0 : (ua == 1 ? lv1 : (ua == 2 ? lv2 : lv3));
              const float lb = ub == 0 ? lv0 : (ub == 1 ? lv1 : (ub == 2 ? lv2 : lv3));
              x[0] = la * (float)s2.x;
              x[1] = lb * (float)s2.y;
            }
          }
          split_pair(x[0], x[1], nm1, hk[i], lk[i]);
        }
        if constexpr (CPT >= 8) {  // 16-byte LDS stores of the thread's run of channels
#pragma unroll
          for (int m = 0; m < CPT / 8; ++m) {
            *reinterpret_cast<u4*>(&S.khi[t][c0 + 8 * m]) = u4{hk[4 * m], hk[4 * m + 1], hk[4 * m + 2], hk[4 * m + 3]};
            *reinterpret_cast<u4*>(&S.klo[t][c0 + 8 * m]) = u4{lk[4 * m], lk[4 * m + 1], lk[4 * m + 2], lk[4 * m + 3]};
          }
        } else if constexpr (CPT == 4) {
          *reinterpret_cast<uint2*>(&S.khi[t][c0]) = make_uint2(hk[0], hk[1]);
          *reinterpret_cast<uint2*>(&S.klo[t][c0]) = make_uint2(lk[0], lk[1]);
        } else {  // one channel pair per thread (head_dim 32 with 8 waves)
          *reinterpret_cast<uint32_t*>(&S.khi[t][c0]) = hk[0];
          *reinterpret_cast<uint32_t*>(&S.klo[t][c0]) = lk[0];
        }
        if (tid < G) {
          const int64_t p = beta * G + tid;
          S.pos[tid] = (p >= a.lo && p < bhi && !is_sink(p)) ? (int)p : -1;
        }
      }
      if constexpr (VB == 3) {  // V from the dense 3-bit stream, one element per thread and pass
        const float* vn = reinterpret_cast<const float*>(md + KMW);  // the V norms
        for (int idx = tid; idx < G * D; idx += PNT) {
          const int tv = idx % G, c = idx / G;
          const float x = vn[tv] * S.vcen[code3_at(rec + lv.v_codes, v_bit3(tv, c, D))];
          const int kq = (tv & 15) >> 2, e = ((tv >> 4) << 2) | (tv & 3);
          const _Float16 hx = (_Float16)x;
          S.vt[c][8 * kq + e] = hx;
          S.vtl[c][8 * kq + e] = (_Float16)(x - (float)hx);
        }
      } else {  // V: chunk q = 16*kq + i holds, for channel tile mu, rows v_tok(kq, e) of channel 16*mu + i
        const uint32_t* vm = md + KMW;
        const int q = tid & 63, kq = q >> 4, i = q & 15;
        constexpr int EPW = VPW < 8 ? VPW : 8;  // row slots of one channel a word covers
#pragma unroll
        for (int n = 0; n < NWI; ++n) {
          const int wi = wv + n * PNW;
          if (wi >= WPC) break;  // uniform over the wave
          const uint32_t w = PF ? pvc[n] : reinterpret_cast<const uint32_t*>(rec + lv.v_codes)[lane * WPC + wi];
#pragma unroll
          for (int k0 = 0; k0 < VPW; k0 += EPW) {
            const int sq0 = wi * VPW + k0, mu = sq0 >> 3, e0 = sq0 & 7, c = 16 * mu + i, gq = c >> 5;
            // metadata of the word's rows: token pairs (t, t+1) share a dword in each section, and
            // codes k, k + 1 (k even) of the word sit at the same bit offset of its two halves
            uint32_t ph[EPW / 2], pl[EPW / 2];
#pragma unroll
            for (int ee = 0; ee < EPW; ee += 2) {
              const int e = e0 + ee, tk = v_tok(kq, e);  // tk even, tk + 1 = v_tok(kq, e + 1)
              const int mi = v_meta_idx(tk, gq, NG) >> 1;
              const uint32_t sw = TQ ? 0u : vm[mi];
              const uint32_t zw = FMT == KVQ_FMT_KIVI ? vm[G * NG / 2 + mi] : 0u;
              const int k = k0 + ee;
              const uint32_t uu = (w >> (VB * (k >> 1))) & (((1u << VB) - 1u) * 0x10001u);
              const float u0 = (float)(uu & 0xFFu), u1 = (float)(uu >> 16);
              const hv2 s2 = HV(sw), z2 = HV(zw);
              float x0, x1;
              if constexpr (TQ) {  // V norms of rows tk, tk + 1 times their centroids
                x0 = __builtin_bit_cast(float, vm[tk]) * S.vcen[uu & 0xFFFFu];
                x1 = __builtin_bit_cast(float, vm[tk + 1]) * S.vcen[uu >> 16];
              } else if constexpr (FMT == KVQ_FMT_KIVI) {  // u s + z, one rounding
                x0 = __builtin_fmaf(u0, (float)s2.x, (float)z2.x);
                x1 = __builtin_fmaf(u1, (float)s2.y, (float)z2.y);
              } else {
                x0 = (u0 - 8.f) * (float)s2.x;
                x1 = (u1 - 8.f) * (float)s2.y;
              }
              split_pair(x0, x1, nm1, ph[ee / 2], pl[ee / 2]);
            }
            if constexpr (EPW == 8) {
              *reinterpret_cast<u4*>(&S.vt[c][8 * kq]) = u4{ph[0], ph[1], ph[2], ph[3]};
              *reinterpret_cast<u4*>(&S.vtl[c][8 * kq]) = u4{pl[0], pl[1], pl[2], pl[3]};
            } else {
              *reinterpret_cast<uint2*>(&S.vt[c][8 * kq + e0]) = make_uint2(ph[0], ph[1]);
              *reinterpret_cast<uint2*>(&S.vtl[c][8 * kq + e0]) = make_uint2(pl[0], pl[1]);
            }
          }
        }
      }
    } else {
      // fp16 rows: window rows bulk_hi + r0 + t (sinks excluded: read from the pool), or the sinks
      const bool sinks = rb >= nbulk + nwblk;
      const int r0 = (rb - nbulk) * G;
      auto row_src = [&](int tr, int64_t* pp, const uint16_t** kp, const uint16_t** vp) {
        *pp = -1;
        *kp = *vp = nullptr;
        if (!sinks) {
          if (r0 + tr < nwin) {
            *pp = a.bulk_hi + r0 + tr;
            int ws = wslot0 + r0 + tr;  // nwin <= R, so one wrap at most
            if (ws >= sh.R) ws -= sh.R;
            const int64_t wo = (int64_t)s * sh.R + ws;
            *kp = lv.win_k + wo * D;
            *vp = lv.win_v + wo * D;
            if (is_sink(*pp)) *pp = -1;
          }
        } else if (tr < nsink && S.spos[tr] <= qmax) {
          *pp = S.spos[tr];
          const int64_t so = (int64_t)s * sh.n_sink + S.sslot[tr];
          *kp = lv.sink_k + so * D;
          *vp = lv.sink_v + so * D;
        }
      };
      if constexpr (TQ) {  // one row per wave pass, rotated: lane l holds channels row_chan(l, k)
        for (int rr = 0; rr < G / PNW; ++rr) {
          const int tr = wv + PNW * rr;
          int64_t p;
          const uint16_t *kr, *vr;
          row_src(tr, &p, &kr, &vr);
          float ky[NK], vy[NK];
#pragma unroll
          for (int k = 0; k < NK; ++k) ky[k] = vy[k] = 0.f;
#pragma unroll
          for (int k = 0; k < NK; k += 2) {
            const int c = row_chan(lane, k);
            if (kr && c < D) {
              const uint32_t kw2 = *reinterpret_cast<const uint32_t*>(kr + c);
              const uint32_t vw2 = *reinterpret_cast<const uint32_t*>(vr + c);
              ky[k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(kw2 & 0xFFFFu)) * sg[k];
              ky[k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(kw2 >> 16)) * sg[k + 1];
              vy[k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw2 & 0xFFFFu)) * sg[k];
              vy[k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw2 >> 16)) * sg[k + 1];
            }
          }
          row_fwht<RMD>(ky, D, lane);
          row_fwht<RMD>(vy, D, lane);
          const int kq = (tr & 15) >> 2, e = ((tr >> 4) << 2) | (tr & 3);
#pragma unroll
          for (int k = 0; k < NK; k += 2) {
            const int c = row_chan(lane, k);
            if (c < D) {
              const float k0 = ky[k] * cd, k1 = ky[k + 1] * cd, v0 = vy[k] * cd, v1 = vy[k + 1] * cd;
              const _Float16 hk0 = (_Float16)k0, hk1 = (_Float16)k1, hv0 = (_Float16)v0, hv1 = (_Float16)v1;
              *reinterpret_cast<uint32_t*>(&S.khi[tr][c]) = (uint32_t)h16(k0) | ((uint32_t)h16(k1) << 16);
              *reinterpret_cast<uint32_t*>(&S.klo[tr][c]) =
                  (uint32_t)h16(k0 - (float)hk0) | ((uint32_t)h16(k1 - (float)hk1) << 16);
              S.vt[c][8 * kq + e] = hv0;
              S.vt[c + 1][8 * kq + e] = hv1;
              S.vtl[c][8 * kq + e] = (_Float16)(v0 - (float)hv0);
              S.vtl[c + 1][8 * kq + e] = (_Float16)(v1 - (float)hv1);
            }
          }
          if (lane == 0) S.pos[tr] = (int)p;
        }
      } else {
        int64_t p;
        const uint16_t *kr, *vr;
        row_src(t, &p, &kr, &vr);
        // rows of this thread's V transpose: row t goes to slot 8*kq + e with v_tok(kq, e) = t
        const int kq = (t & 15) >> 2, e = ((t >> 4) << 2) | (t & 3);
#pragma unroll
        for (int c = c0; c < c0 + CPT; c += 2) {
          uint32_t kw2 = 0u, vw2 = 0u;
          if (kr) {
            kw2 = *reinterpret_cast<const uint32_t*>(kr + c);
            vw2 = *reinterpret_cast<const uint32_t*>(vr + c);
          }
          *reinterpret_cast<uint32_t*>(&S.khi[t][c]) = kw2;
          *reinterpret_cast<uint32_t*>(&S.klo[t][c]) = 0u;
          S.vt[c][8 * kq + e] = __builtin_bit_cast(_Float16, (uint16_t)(vw2 & 0xFFFFu));
          S.vt[c + 1][8 * kq + e] = __builtin_bit_cast(_Float16, (uint16_t)(vw2 >> 16));
          S.vtl[c][8 * kq + e] = (_Float16)0.f;
          S.vtl[c + 1][8 * kq + e] = (_Float16)0.f;
        }
        if (tid % SL == 0) S.pos[t] = (int)p;
      }
    }
    // the next bulk row block's loads, in flight during this row block's matrix work
    if (PF && rb + 1 < rb_hi && rb + 1 < nbulk) fetch(rb + 1);
    lds_barrier();
    if (LQ && sh.rope) {  // the staged keys turn by their rows' indices in the compressed cache
      constexpr int H = D / 2;
      for (int idx = tid; idx < G * H; idx += PNT) {
        const int t = idx / H, c = idx % H;
        const int p = S.pos[t];
        if (p < 0) continue;
        const int ri = cache_index(S.spos, nsink, a.lo, p);
        const float x0 = (float)S.khi[t][c] + (float)S.klo[t][c];
        const float x1 = (float)S.khi[t][c + H] + (float)S.klo[t][c + H];
        float sn, cs;  // one angle per pair: both channels turn by idx * theta_c
        rope_cs(ri, lv.tables->rope_inv[c], cs, sn);
        const float y0 = x0 * cs - x1 * sn, y1 = x1 * cs + x0 * sn;
        const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
        S.khi[t][c] = h0;
        S.klo[t][c] = (_Float16)(y0 - (float)h0);
        S.khi[t][c + H] = h1;
        S.klo[t][c + H] = (_Float16)(y1 - (float)h1);
      }
      lds_barrier();
    }

    // ---- the wave's tiles against the row block: every LDS operand read feeds all tiles ----
    if (!live) continue;  // a wave without queries (a short chunk) only helps to stage
    f4 c[PT][2];
#pragma unroll
    for (int tt = 0; tt < PT; ++tt) c[tt][0] = c[tt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const u4 ah = *reinterpret_cast<const u4*>(&S.khi[16 * tau + i16][32 * st + 8 * kg]);
        const u4 alo = *reinterpret_cast<const u4*>(&S.klo[16 * tau + i16][32 * st + 8 * kg]);
#pragma unroll
        for (int tt = 0; tt < PT; ++tt) {
          c[tt][tau] = mfma(ah, bq[tt][st], c[tt][tau]);
          c[tt][tau] = mfma(alo, bq[tt][st], c[tt][tau]);
          if constexpr (SQ) c[tt][tau] = mfma(ah, bql[tt][st], c[tt][tau]);
        }
      }
    // lane (column i16, group kg) holds rows 16*tau + 4*kg + e
    int rp[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int e = 0; e < 4; ++e) rp[4 * tau + e] = S.pos[16 * tau + 4 * kg + e];
    u4 bph[PT], bpl[PT];
#pragma unroll
    for (int tt = 0; tt < PT; ++tt) {
      float y[8];
      float mb = -INFINITY;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = rp[4 * tau + e];
          const bool ok = p >= 0 && qpos[tt] >= 0 && p <= qpos[tt];
          y[4 * tau + e] = ok ? c[tt][tau][e] * al : -INFINITY;
          mb = fmaxf(mb, y[4 * tau + e]);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float mnew = fmaxf(m_[tt], mb);
      if (__any(mnew > m_[tt])) {
        const float f = mnew == m_[tt] ? 1.f : (m_[tt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_[tt] - mnew));
        l_[tt] *= f;
#pragma unroll
        for (int mu = 0; mu < NMU; ++mu) acc[tt][mu] *= f;
        m_[tt] = mnew;
      }
      // weights as fp16 hi + lo halves (the pair holds the weight to ~2^-21)
      float pw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pw[k] = mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(y[k] - mnew);
        l_[tt] += pw[k];
      }
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) split_pair(pw[2 * m], pw[2 * m + 1], nm1, wh[m], wl[m]);
      bph[tt] = u4{wh[0], wh[1], wh[2], wh[3]};
      bpl[tt] = u4{wl[0], wl[1], wl[2], wl[3]};
    }
#pragma unroll
    for (int mu = 0; mu < NMU; ++mu) {  // V_hi p_hi + V_hi p_lo + V_lo p_hi
      const u4 avh = *reinterpret_cast<const u4*>(&S.vt[16 * mu + i16][8 * kg]);
      const u4 avl = *reinterpret_cast<const u4*>(&S.vtl[16 * mu + i16][8 * kg]);
#pragma unroll
      for (int tt = 0; tt < PT; ++tt) {
        acc[tt][mu] = mfma(avh, bph[tt], acc[tt][mu]);
        acc[tt][mu] = mfma(avh, bpl[tt], acc[tt][mu]);
        acc[tt][mu] = mfma(avl, bph[tt], acc[tt][mu]);
      }
    }
  }

  // ---- outputs: lane (column i16, group kg) holds channels 16*mu + 4*kg .. + 3 ----
  if constexpr (TQ) __syncthreads();  // the LDS tiles become the rotation scratch
#pragma unroll
  for (int tt = 0; tt < PT; ++tt) {
    float l = l_[tt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float il = l > 0.f ? 1.f / l : 0.f;
    if (!TQ && a.splits > 1) {  // un-normalised partial (acc, m, l) of this split
      if (qpos[tt] < 0) continue;
      float* pp = a.part + ((((int64_t)b * sh.Hq + head[tt]) * a.n + qidx[tt]) * a.splits + split) * (D + 4);
#pragma unroll
      for (int mu = 0; mu < NMU; ++mu) *reinterpret_cast<f4*>(pp + 16 * mu + 4 * kg) = acc[tt][mu];
      if (kg == 0) {
        pp[D] = m_[tt];
        pp[D + 1] = l;
      }
      continue;
    }
    if constexpr (!TQ) {
      if (qpos[tt] < 0) continue;
      float* o = a.out + (((int64_t)b * sh.Hq + head[tt]) * a.n + qidx[tt]) * D;
#pragma unroll
      for (int mu = 0; mu < NMU; ++mu) *reinterpret_cast<f4*>(o + 16 * mu + 4 * kg) = acc[tt][mu] * il;
    } else {
      // rotated-domain rows to a wave-private LDS tile, then o = sigma * (c_d * FWHT(row)) per column
      float* os = reinterpret_cast<float*>(&S.khi[0][0]) + wv * 16 * D;
#pragma unroll
      for (int mu = 0; mu < NMU; ++mu) *reinterpret_cast<f4*>(os + i16 * D + 16 * mu + 4 * kg) = acc[tt][mu] * il;
      __builtin_amdgcn_wave_barrier();
      for (int col = 0; col < 16; ++col) {
        int cq, ch;
        const bool cok = col_query(tt, col, &cq, &ch);
        float y[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) y[k] = row_chan(lane, k) < D ? os[col * D + row_chan(lane, k)] : 0.f;
        row_fwht<RMD>(y, D, lane);
        float* o = a.out + (((int64_t)b * sh.Hq + ch) * a.n + cq) * sh.Din;
#pragma unroll
        for (int k = 0; k < NK; k += 2) {
          const int c = row_chan(lane, k);
          if (cok && c < sh.Din) *reinterpret_cast<float2*>(o + c) = make_float2(sg[k] * (y[k] * cd), sg[k + 1] * (y[k + 1] * cd));
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Fixed-order merge of the row-block splits of one (b, head, query): o = sum 2^(m_i - M) acc_i /
// sum 2^(m_i - M) l_i; a query without valid rows in any split gets zeros.
template <int D>
__global__ __launch_bounds__(D) void k_prefill_merge(PrefillArgs a) {
  const int64_t idx = blockIdx.x;  // (b * Hq + head) * n + query
  const int c = threadIdx.x;
  const float* base = a.part + idx * a.splits * (D + 4);
  __shared__ float sm[64], sl[64], sw[64];  // splits <= 64: every split's (m, l) loaded at once
  for (int sp = c; sp < a.splits; sp += D) {
    sm[sp] = base[sp * (D + 4) + D];
    sl[sp] = base[sp * (D + 4) + D + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, sm[sp]);
  for (int sp = c; sp < a.splits; sp += D) sw[sp] = sm[sp] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[sp] - M);
  __syncthreads();
  float av = 0.f, lv = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < a.splits; ++sp) {
    av = av + base[sp * (D + 4) + c] * sw[sp];
    lv = lv + sl[sp] * sw[sp];
  }
  a.out[idx * D + c] = lv > 0.f ? av / lv : 0.f;
}

// Column tiles per wave: TurboQuant 1 (the rotated queries' lo halves take a second tile's
// registers); queries staged through LDS (RoPE, fp32) 1 for short chunks (a decode query: fewer idle
// columns, more waves per SIMD) and 2 for long ones; otherwise 2.
int tiles_per_wave(const PrefillArgs& a) {
  if (a.sh.fmt == KVQ_FMT_TQ) return 1;
  if ((a.sh.rope || a.sh.in_f32) && a.n < 256) return 1;
  return PT;
}

template <int FMT, bool LQ>
constexpr int waves_per_wg() {
  return (FMT == KVQ_FMT_TQ || LQ) ? PNW_LDS : (FMT == KVQ_FMT_Q2K ? PNW_Q2K : PNW_DIRECT);
}

template <int FMT, int KB, int VB, bool LQ, int PTT>
hipError_t launch_drp(const PrefillArgs& a, hipStream_t st) {
  constexpr int PW = waves_per_wg<FMT, LQ>();
  const int QT = PW * PTT * (16 / (a.sh.Hq / a.sh.Hkv));
  const dim3 grid((a.n + QT - 1) / QT, a.sh.B * a.sh.Hkv, a.splits > 1 ? a.splits : 1);
  switch (a.sh.D) {
    case 32: hipLaunchKernelGGL((k_prefill_attn<FMT, KB, VB, 32, LQ, PTT, PW>), grid, dim3(64 * PW), 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_prefill_attn<FMT, KB, VB, 64, LQ, PTT, PW>), grid, dim3(64 * PW), 0, st, a); break;
    case 128: hipLaunchKernelGGL((k_prefill_attn<FMT, KB, VB, 128, LQ, PTT, PW>), grid, dim3(64 * PW), 0, st, a); break;
    case 256:  // TurboQuant rows of head_dim 160, stored at 256
      if constexpr (FMT == KVQ_FMT_TQ) {
        hipLaunchKernelGGL((k_prefill_attn<FMT, KB, VB, 256, LQ, PTT, PW>), grid, dim3(64 * PW), 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int KB, int VB, bool LQ>
hipError_t launch_dr(const PrefillArgs& a, hipStream_t st) {
  hipError_t e;
  if constexpr (FMT == KVQ_FMT_TQ) e = launch_drp<FMT, KB, VB, LQ, 1>(a, st);
  else if constexpr (LQ) e = tiles_per_wave(a) == 1 ? launch_drp<FMT, KB, VB, LQ, 1>(a, st) : launch_drp<FMT, KB, VB, LQ, PT>(a, st);
  else if constexpr (FMT == KVQ_FMT_Q2K) e = launch_drp<FMT, KB, VB, LQ, 1>(a, st);
  else e = launch_drp<FMT, KB, VB, LQ, PT>(a, st);
  if (e != hipSuccess || a.splits <= 1) return e;
  const dim3 mg((unsigned)((int64_t)a.sh.B * a.sh.Hq * a.n));
  switch (a.sh.D) {
    case 32: hipLaunchKernelGGL(k_prefill_merge<32>, mg, dim3(32), 0, st, a); break;
    case 64: hipLaunchKernelGGL(k_prefill_merge<64>, mg, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL(k_prefill_merge<128>, mg, dim3(128), 0, st, a); break;
  }
  return hipGetLastError();
}
template <int FMT, int KB, int VB>
hipError_t launch_d(const PrefillArgs& a, hipStream_t st) {
  // TurboQuant stages its queries through LDS already (and has no RoPE); the block formats take the
  // LDS query prologue for RoPE or fp32 queries
  if constexpr (FMT == KVQ_FMT_TQ) return launch_dr<FMT, KB, VB, false>(a, st);
  else return a.sh.rope || a.sh.in_f32 ? launch_dr<FMT, KB, VB, true>(a, st) : launch_dr<FMT, KB, VB, false>(a, st);
}
template <int KB>
hipError_t launch_kivi(const PrefillArgs& a, hipStream_t st) {
  switch (a.sh.vb) {
    case 2: return launch_d<KVQ_FMT_KIVI, KB, 2>(a, st);
    case 4: return launch_d<KVQ_FMT_KIVI, KB, 4>(a, st);
    case 8: return launch_d<KVQ_FMT_KIVI, KB, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_queries_per_tile(int r, int fmt, int rope) {  // (long chunks, fp16 queries)
  if (fmt == KVQ_FMT_TQ) return PNW_LDS * (16 / r);
  if (rope) return PNW_LDS * PT * (16 / r);
  return fmt == KVQ_FMT_Q2K ? PNW_Q2K * (16 / r) : PNW_DIRECT * PT * (16 / r);
}

int prefill_row_blocks(const PrefillArgs& a) {
  // the last tile's rows: every valid position (its last query is position P - 1)
  const int64_t nb = a.bulk_hi > a.lo ? (a.bulk_hi - 1) / G - a.lo / G + 1 : 0;
  const int64_t nw = a.P - a.bulk_hi;
  return (int)(nb + (nw + G - 1) / G + (a.sh.n_sink > 0 ? 1 : 0));
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const Shape& sh = a.sh;
  if (a.splits > 1 && (sh.fmt == KVQ_FMT_TQ || !a.part)) return hipErrorInvalidValue;
  if (sh.fmt == KVQ_FMT_Q2K) return launch_d<KVQ_FMT_Q2K, 2, 4>(a, st);
  if (sh.fmt == KVQ_FMT_TQ) {
    if (sh.kb == 4 && sh.vb == 2) return launch_d<KVQ_FMT_TQ, 4, 2>(a, st);
    if (sh.kb == 2 && sh.vb == 2) return launch_d<KVQ_FMT_TQ, 2, 2>(a, st);
    if (sh.kb == 4 && sh.vb == 4) return launch_d<KVQ_FMT_TQ, 4, 4>(a, st);
    if (sh.kb == 2 && sh.vb == 4) return launch_d<KVQ_FMT_TQ, 2, 4>(a, st);
    // dense 3-bit streams
    if (sh.kb == 3 && sh.vb == 2) return launch_d<KVQ_FMT_TQ, 3, 2>(a, st);
    if (sh.kb == 3 && sh.vb == 3) return launch_d<KVQ_FMT_TQ, 3, 3>(a, st);
    if (sh.kb == 3 && sh.vb == 4) return launch_d<KVQ_FMT_TQ, 3, 4>(a, st);
    if (sh.kb == 2 && sh.vb == 3) return launch_d<KVQ_FMT_TQ, 2, 3>(a, st);
    if (sh.kb == 4 && sh.vb == 3) return launch_d<KVQ_FMT_TQ, 4, 3>(a, st);
    return hipErrorInvalidValue;
  }
  if (sh.fmt != KVQ_FMT_KIVI) return hipErrorInvalidValue;
  switch (sh.kb) {
    case 2: return launch_kivi<2>(a, st);
    case 4: return launch_kivi<4>(a, st);
    case 8: return launch_kivi<8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
