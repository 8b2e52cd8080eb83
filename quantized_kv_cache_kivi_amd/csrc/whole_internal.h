// Internal declarations of the whole-T KIVI cache (kvq_whole.h): host code and kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/kvq_whole.h"

namespace kvqw {

constexpr int RPT = 256;           // rows per re-quantisation tile
constexpr int MAX_SPLITS = 64;     // attention splits per stream
constexpr int MIN_SPLIT_ROWS = 256;
// Appends of at most FUSE_ROWS rows to at most FUSE_TILES * RPT rows run in one launch, one workgroup
// per stream (larger caches take two launches over every tile: the extremes, then the coding).
constexpr int FUSE_ROWS = 32;
constexpr int FUSE_TILES = 4;

struct View {
  int8_t* kc;    // [S][cap][D]
  int8_t* vc;
  uint16_t* ks;  // [S][D]
  uint16_t* kz;
  uint16_t* vs;  // [S][cap]
  uint16_t* vz;
  uint32_t* sync;  // [S] arrival counters of the workgroups of one launch (zero between calls)
};

// The stored rows of a stream in order j: the nsk sink rows (slot j), then nring ring rows
// whose ring offsets start at rs0 (slot n_sink + (rs0 + j - nsk) mod ring).
struct Rows {
  int nsk, nring, rs0, ring, n_sink;
};

struct Shape {
  int B, H, Hq, D, bits, in_f32, cap;
};

struct AppendArgs {
  Shape sh;
  View v;
  Rows old;            // rows stored before the append
  const void* k;       // [B][H][n][D] in_dtype
  const void* vin;
  int n;               // new rows per stream
  int nsk_new;         // new rows at sink positions (slots old.nsk ..)
  int ps0;             // ring offset of the first new row past the sinks
  int tiles;           // RPT-row tiles over old + new rows
  float* part;         // [S][tiles][2][D] per-tile channel min, max
  uint16_t* oldm;      // [S][2][D] K scale, zero before the append
};

struct DecodeArgs {
  Shape sh;
  View v;
  Rows rows;
  const void* q;       // [B][Hq][D] in_dtype
  float* out;          // [B][Hq][D]
  float* part;         // [S][splits][r][D + 2] (acc, m, l)
  float scale;
  int splits, rows_per_split;
};

struct DequantArgs {
  Shape sh;
  View v;
  int which, count, n_sink, ring;
  int64_t pos0;
  uint16_t* out;       // [B][H][count][D]
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);

}  // namespace kvqw
