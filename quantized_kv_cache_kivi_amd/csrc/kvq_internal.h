// Internal declarations shared by the host code and the HIP kernels of libkvq.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/kvq.h"

namespace kvq {

constexpr int G = 32;          // token block length and V channel-group length
constexpr int MAX_SINK = 16;   // largest n_sink
constexpr int MAX_GQA = 16;    // largest n_q_heads / n_kv_heads
constexpr int MAX_D = 128;     // largest head_dim of the block formats (and of RoPE on read)
constexpr int MAX_SD = 256;    // widest stored row: TurboQuant head_dim 160 padded to 256
constexpr int SELECT_GMAX = 64;      // most workgroups per batch element of one sink-selection call
constexpr int SELECT_MIN_ROWS = 64;  // rows a selection workgroup takes at least

// fp32 tables written once into the device buffer (tables region).
struct Tables {
  float signs[MAX_SD];  // TQ sign diagonal (+-1), one per stored coordinate
  float k_bnd[16];      // TQ K boundaries in t-space (2^k_bits - 1 used)
  float k_cen[16];      // TQ K centroids
  float v_bnd[16];      // TQ V boundaries
  float v_cen[16];      // TQ V centroids
  float q2k_thr[4];     // Gaussian 4-level Lloyd-Max thresholds (3 used)
  float q2k_lvl[4];     // Gaussian 4-level Lloyd-Max levels
  float rope_inv[MAX_D / 2];  // RoPE theta_c = base^(-2c/D), rounded to fp32 (rope mode)
  float rope_row[16][MAX_D / 2][2];  // RoPE (cos, sin) of the exact angles i * theta_c, i < 16 (rope mode)
};

// Everything a kernel needs to address one layer of the cache.
struct LayerView {
  uint8_t* bulk;        // [S][cap_b][rec]
  uint8_t* staging;     // [S][32][D] in_dtype
  uint16_t* win_k;      // [S][R][D]
  uint16_t* win_v;
  uint16_t* sink_k;     // [S][n_sink][D]
  uint16_t* sink_v;
  int32_t* sink_pos;    // [B][n_sink]
  float* sink_score;    // [B][n_sink]
  int32_t* sink_count;  // [B]
  uint32_t* decode_sync;  // [S] arrival counters of one decode call's workgroups (zero between calls)
  const Tables* tables;
  int64_t rec, k_codes, v_codes, k_meta, v_meta;  // record size and section offsets
  int cap_b;
};

struct Shape {
  int B, Hkv, Hq, D, fmt, kb, vb, sink_mode, n_sink, W, R, in_f32, rope;
  int Din;  // channels of the caller's rows (q, K, V, outputs); D is the stored and computed width
            // (TurboQuant pads a head_dim that is not a power of two to the next one, zeros in the pad)
};

struct AppendArgs {
  Shape sh;
  LayerView lv;
  const void* k;        // [B][Hkv][n][D]
  const void* v;
  int64_t P;            // rows already appended
  int n;                // rows in this call
  int64_t blk0;         // first block touched
  int nblk;             // blocks touched
  int defer;            // 1: blocks are quantized when they complete (block formats, fp16 input, residual >= 32)
};

struct SelectArgs {
  Shape sh;
  LayerView lv;
  const void* k;        // [B][Hkv][n][D] in_dtype, 16-byte aligned
  int2* work;           // [B][SELECT_GMAX][n_sink] (fp32 score bits, position): per-workgroup top-k lists
  int64_t P;
  int n;
};

struct DecodeArgs {
  Shape sh;
  LayerView lv;
  const void* q;        // [B][Hq][D]
  float* out;           // [B][Hq][D]
  float* ws;            // partials
  float scale;
  int64_t P, lo;
  int64_t bulk_lo, bulk_hi;  // bulk token range [bulk_lo, bulk_hi)
  int64_t blk_first;         // first bulk block
  int nblk;                  // bulk blocks
  int splits;                // bulk splits S (the fp16 split is index S)
  int blocks_per_split;
  int fast;                  // 1: MFMA path (head_dim 128, fp16 input, KIVI equal widths or q2k, GQA 1/2/4/8)
  int nparts;                // partials per stream in the workspace: bulk splits, then the fp16-row groups
                             // (MFMA path: ceil(rows / 64); TurboQuant: 1; other formats: 0)
  const void* k1;            // fused decode step: the row appended at P - 1, [B][Hkv][1][D] fp16 (else NULL);
  const void* v1;            // scored from here, copied to staging and window by fp16 group 0
  int open_new;              // fused step whose row opens a block: that block's record is zeroed
};

struct PrefillArgs {
  Shape sh;
  LayerView lv;
  const void* q;        // [B][Hq][n][D] fp16, 16-byte aligned: queries of positions P-n .. P-1
  float* out;           // [B][Hq][n][D]
  float scale;
  int64_t P, lo, bulk_hi;  // valid range [lo, P) (plus sinks); bulk rows below bulk_hi
  int n;
  int splits;           // row-block splits per query tile (1: outputs written directly; > 1: not TQ)
  float* part;          // splits > 1: [B][Hq][n][splits][D + 4] partials (acc[D], m, l), merged afterwards
};

struct DequantArgs {
  Shape sh;
  LayerView lv;
  int which;
  int64_t P, lo, pos0;
  int count;
  uint16_t* out;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
int select_groups(int n);  // workgroups per batch element for an n-row selection call
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
int prefill_queries_per_tile(int r, int fmt, int rope);  // queries of one prefill-attention workgroup
int prefill_row_blocks(const PrefillArgs& a);            // row blocks the last query tile reads

// Workgroups of the MFMA decode kernel for this shape that the current device holds at once
// (compute units x resident workgroups per unit); 0 if the shape has no MFMA kernel.
int fast_resident_slots(const Shape& sh);
// fp16 rows (window and sinks) one fp16 workgroup of the MFMA decode kernel takes.
int fast_fp16_rows_per_group();

// The calling thread's error text (kvq_last_error), for every entry point of the library.
kvq_status set_error(kvq_status st, const char* msg);
void clear_error();

// Host-side table generation (tables.cpp).
void make_tables(const kvq_config& cfg, Tables* t);
// Width rows are stored and computed at (TurboQuant: head_dim 96 padded to 128; else head_dim).
int stored_dim(const kvq_config& c);

// Decode attention with its split partials in ws (ws_bytes device bytes); KVQ_ECAPACITY, with nothing
// launched, when this call's partials need more.  Shared by kvq_decode_attn (caller's workspace) and
// kvq_decode_attn_nomalloc (the library's static workspace).
kvq_status decode_attn_ws(kvq_cache* c, int32_t layer, const void* q, float* out, float scale, void* ws,
                          size_t ws_bytes, void* stream, const void* k1 = nullptr, const void* v1 = nullptr,
                          int open_new = 0);
// Takes the current device's address of the static decode workspace once per device (kvq_create
// calls it so that the address is known before any allocation-free call).
kvq_status static_ws_prepare();

}  // namespace kvq
