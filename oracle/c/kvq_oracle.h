/*
 * kvq_oracle.h — plain C99 CPU oracle of the quantized KV cache hot path.
 * TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline use it;
 * the HIP library never includes, links or calls it, and it shares no code with the library.
 *
 * It computes, step by step in the pages' order, what the GPU path computes:
 *   - sink selection by per-token key L2 norm averaged over KV heads, a running top-k folded per call,
 *     new members committed while the set has room ("KVSink-Adapted Sink Protection", "How it works",
 *     "Fidelity to the paper"); or the first N positions ("StreamingLLM + KIVI — long-context decode
 *     without growing the KV cache", "StreamingLLM — why softmax needs an anchor");
 *   - KIVI asymmetric min/max group quantization, K per channel over 32-token blocks, V per token over
 *     32-channel groups, sink rows excluded from calibration (StreamingLLM + KIVI page, "Affine
 *     quantisation formula", "KIVI"; kivi_sink page, "How it works" 2);
 *   - the q2k format (2-bit K on the Gaussian Lloyd-Max grid over the block RMS, symmetric 4-bit V;
 *     q2k page "Summary", "Memory math");
 *   - TurboQuant (signs, fast Walsh-Hadamard transform, 1/sqrt(d), L2 norm, Lloyd-Max Beta(d/2, d/2)
 *     codebooks; TurboQuant spec "Step 1", "Step 2", "Codebook Generation", "Hadamard Transform
 *     Detail", "As-Built Notes");
 *   - StreamingLLM eviction of [sink, P - window) as a validity range with an fp16 overlay for sinks and
 *     the recent window (StreamingLLM + KIVI page, "Implementation"; q2k page, "Summary");
 *   - the stored bytes of every ring slot in the documented storage format (include/kvq.h; block formats
 *     with fp16 input and residual >= 32 leave an open block's record zero until the block completes);
 *   - single-query decode attention in fp64 over the exactly dequantized cache (plain definition),
 *     optionally with RoPE on read: rotate-half pairs (c, c + D/2) turned by the exact angle idx * theta_c,
 *     theta_c = base^(-2c/D) rounded to fp32, idx = the number of valid positions before the row or the
 *     query's own position ("StreamingLLM + KIVI" page, "RoPE caveat"; the readings of oracle/rope.py).
 *
 * Every code-deciding expression is fp32, one rounding per operation (built with -ffp-contract=off
 * -fno-fast-math), rintf rounding half to even, min/max results canonicalised with + 0.0f; fp32 -> fp16 is
 * written here from the IEEE-754 definition (round to nearest even, subnormals kept).  The readings of
 * the pages where they are silent are the ones the numpy oracle (the Python modules of oracle/) states; the two are
 * checked bit for bit against each other by tests/test_oracle_c.py.
 *
 * Errors: every entry point returns 0 on success and a negative code on a bad argument or a call-order /
 * capacity violation (nothing is changed then).
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stdint.h>

typedef struct {
  int32_t n_layers, batch, n_kv_heads, n_q_heads, head_dim; /* head_dim 32, 64 or 128 */
  int32_t fmt;         /* 0 KIVI (bits 2/4/8 each), 1 q2k (2, 4), 2 TurboQuant (bits 2/3/4 each) */
  int32_t k_bits, v_bits;
  int32_t sink_mode;   /* 0 none, 1 first N, 2 top-k key norm */
  int32_t n_sink;      /* 0 .. 16 */
  int32_t window;      /* StreamingLLM window (0: never evict) */
  int32_t residual;    /* fp16 recent overlay */
  int32_t capacity;    /* slots per stream, a multiple of 32 */
  int32_t in_f32;      /* 0: inputs are fp16 bit patterns, 1: fp32 */
  int32_t tq_dense3;   /* TurboQuant 3-bit codes as a dense stream (else 4-bit slots) */
  uint64_t seed;       /* TurboQuant sign seed */
  int32_t rope;        /* 1: decode attention turns keys and queries by their index (not with TurboQuant) */
  float rope_base;     /* RoPE base (<= 0: 10000) */
} ko_config;

typedef struct ko_model ko_model;

/* Host model of one cache; NULL on an invalid configuration. */
ko_model* ko_create(const ko_config* cfg);
void ko_destroy(ko_model* m);

/* Format tables: TurboQuant sign vector [d] and codebook (boundaries [2^bits - 1], centroids [2^bits]) in
 * the t = 2u - 1 space; the q2k Gaussian thresholds [3] and levels [4]. */
int ko_tq_signs(uint64_t seed, int d, float* out);
int ko_tq_codebook(int d, int bits, float* bnd, float* cen);
int ko_q2k_grid(float* thresholds, float* levels);
/* fp32 -> fp16 bit pattern (round to nearest even, subnormals kept): n values. */
void ko_f32_to_f16(const float* x, uint16_t* out, int64_t n);

/* The cache calls, per layer: select (top-k mode), append n rows, evict.  k, v: [batch][n_kv_heads][n]
 * [head_dim] fp16 bit patterns or fp32 (in_f32). */
int ko_select(ko_model* m, int layer, const void* k, int n);
int ko_append(ko_model* m, int layer, const void* k, const void* v, int n);
int ko_evict(ko_model* m, int layer);
int ko_state(const ko_model* m, int layer, int64_t* P, int64_t* lo);

/* Record geometry: record bytes, section offsets (K codes, V codes, K meta, V meta), blocks per ring. */
int ko_record_layout(const ko_model* m, int32_t* out6);

/* Stored bytes of stream (layer, b, h): bulk [cap_blocks][record], fp16 window ring [residual][D] for K and
 * V, fp16 sink pool [n_sink][D] for K and V (committed order).  Any pointer may be NULL. */
int ko_stream_image(ko_model* m, int layer, int b, int h, uint8_t* bulk, uint16_t* win_k, uint16_t* win_v,
                    uint16_t* sink_k, uint16_t* sink_v);
/* Committed sinks of (layer, b): positions [n_sink] (-1 empty), scores [n_sink], count. */
int ko_sink_state(const ko_model* m, int layer, int b, int32_t* pos, float* score, int32_t* count);

/* Values read for positions pos[0..n) of stream (layer, b, h), which 0 = K, 1 = V, read priority sink >
 * window > bulk: exact fp64 (out64) and the fp32 dequant formula rounded once to fp16 (out16); either
 * pointer may be NULL.  Positions must be valid (else -2). */
int ko_values(ko_model* m, int layer, int b, int h, int which, const int64_t* pos, int n, double* out64,
              uint16_t* out16);

/* Decode attention of one query per (batch element, query head) over the valid set of `layer`, fp64:
 * out[b][j] = sum_p softmax_p(scale * q[b][j] . k_p) v_p, scale <= 0 meaning 1/sqrt(head_dim); query head
 * j reads KV head j / (n_q_heads / n_kv_heads).  q: [batch][n_q_heads][head_dim] fp16 bits or fp32; out:
 * [batch][n_q_heads][head_dim].  Streams run on `threads` OpenMP threads (<= 0: one). */
int ko_decode_attention(ko_model* m, int layer, const void* q, double scale, double* out, int threads);

/* Byte accounting of (layer, b) (kivi_sink page, "How it works" 4): n_valid, n_compressed, n_sink,
 * n_residual, current_length, compressed_bytes, sink_fp16_bytes, residual_fp16_bytes. */
int ko_account(const ko_model* m, int layer, int b, int64_t* out8);

#endif
