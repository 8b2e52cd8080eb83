/*
 * kvq_whole.h — C ABI of the whole-T KIVI cache of libkvq (AMD MI355X, gfx950).
 *
 * The cache of "StreamingLLM + KIVI — long-context decode without growing the
 * KV cache" as that page builds it ([SK] below), next to the block-grouped
 * cache of kvq.h:
 *  - K is quantised per channel with one (scale, zero) per (batch, head,
 *    channel) over every stored token; a new token can move a channel's
 *    min/max, so every append re-quantises the whole stored K ([SK] "KIVI —
 *    int8/int4 KV cache with greedy-lossless decode", "Caveats": O(T*D) per
 *    step).
 *  - V is quantised per token with one (scale, zero) per (batch, head, token)
 *    over all channels, once at append ([SK] same section).
 *  - Codes follow [SK] "Affine quantisation formula": scale = max(1e-5,
 *    (max - min)/(qMax - qMin)), zero = min, qMin/qMax = -128/127 (int8) or
 *    -8/7 (int4).  The stored byte is the signed code q = u + qMin with
 *    u = clamp(rint((x - zero)/scale), 0, qMax - qMin) computed against the
 *    stored fp16 scale and zero; int4 precision is held in int8 bytes ([SK]
 *    "Storage layout").
 *  - Re-quantisation reads the stored K: each stored row is dequantised with
 *    the previous metadata in fp32, u*scale + zero (two roundings), the
 *    per-channel min and max run over those values and the new rows, and
 *    every stored row is coded again.  Sink rows are stored and quantised
 *    like every other row (no fp16 overlay).
 *  - StreamingLLM eviction ([SK] "Implementation"): the first n_sink
 *    positions stay, and after kvqw_evict only the last `window` others.
 *    Nothing moves: position p < n_sink lives in slot p, any other position p
 *    in slot n_sink + (p - n_sink) % (capacity - n_sink).
 *
 * Conventions are those of kvq.h: device pointers owned by the caller, every
 * launch asynchronous on `stream`, validation before any launch (on error
 * nothing runs, the state is unchanged, kvq_last_error() says why), inputs
 * finite with |x| <= 32768.
 *
 * Storage, per layer (offsets from kvqw_get_layout), S = batch * n_kv_heads:
 *   k_codes, v_codes   int8 [S][capacity][head_dim]   (slot-indexed rows)
 *   k_scale, k_zero    fp16 [S][head_dim]
 *   v_scale, v_zero    fp16 [S][capacity]
 *   sync               uint32 [S]: arrival counters of the workgroups of one append or decode launch
 *                      (the last to arrive finishes the stream); zero between calls, so calls on one
 *                      cache must not overlap (calls on one stream never do)
 */
#ifndef KVQ_WHOLE_H
#define KVQ_WHOLE_H

#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvqw_cache kvqw_cache; /* opaque host handle, owned by the library */

typedef struct {
  int32_t n_layers;   /* >= 1 */
  int32_t batch;      /* >= 1 */
  int32_t n_kv_heads; /* >= 1 */
  int32_t n_q_heads;  /* n_kv_heads times 1, 2, 4 or 8 */
  int32_t head_dim;   /* 32, 64 or 128 */
  int32_t bits;       /* 8 or 4 (int4 precision in int8 storage) */
  int32_t n_sink;     /* first-N attention sinks, >= 0 */
  int32_t window;     /* StreamingLLM window; 0 = never evict */
  int32_t capacity;   /* row slots per stream, sinks included, multiple of 32; 0 = n_sink + window + 32
                         rounded up to 32 (needs window > 0); with window > 0 it must exceed
                         n_sink + window */
  int32_t in_dtype;   /* KVQ_IN_F16 or KVQ_IN_F32 for K, V and q */
} kvqw_config;

typedef struct { /* byte offsets inside the caller's device buffer */
  uint64_t layer_stride;          /* layer l's regions start at l * layer_stride */
  uint64_t k_codes, v_codes;      /* int8 [S][capacity][head_dim] */
  uint64_t k_scale, k_zero;       /* fp16 [S][head_dim] */
  uint64_t v_scale, v_zero;       /* fp16 [S][capacity] */
  uint64_t sync;                  /* uint32 [S] */
  uint64_t total;                 /* = kvqw_required_bytes */
  int32_t capacity;
  int32_t pad_;
} kvqw_layout;

typedef struct { /* one layer, summed over the batch and the KV heads */
  int64_t n_stored;        /* stored rows per (b, head) */
  int64_t current_length;  /* positions appended so far (the generation counter, [SK] "Caveats") */
  int64_t code_bytes;      /* K and V codes, one byte per element */
  int64_t meta_bytes;      /* kScales, kZeros (per channel) and vScales, vZeros (per stored row), fp16 */
  int64_t packed_int4_bytes; /* the same rows with int4 codes packed two per byte ([SK] "Storage layout") */
  int64_t bf16_bytes;      /* the same rows unquantised in a 2-byte type */
} kvqw_bytes;

/* Validates a configuration. */
kvq_status kvqw_config_check(const kvqw_config* cfg);

/* Device bytes of the cache (all layers); 0 for an invalid configuration. */
size_t kvqw_required_bytes(const kvqw_config* cfg);

/* Offsets of every region of the storage above. */
kvq_status kvqw_get_layout(const kvqw_config* cfg, kvqw_layout* out);

/* Device bytes of the workspace kvqw_append and kvqw_decode_attn need (per-tile min/max partials of
 * the re-quantisation, the previous K metadata, split partials of attention); 16-byte aligned.  Its
 * contents carry nothing between calls. */
size_t kvqw_workspace_bytes(const kvqw_config* cfg);

/* Binds the cache to dev_buf (>= kvqw_required_bytes, 256-byte aligned) and clears it on `stream`
 * (synchronised before returning). */
kvq_status kvqw_create(const kvqw_config* cfg, void* dev_buf, size_t dev_bytes, void* stream, kvqw_cache** out);

kvq_status kvqw_destroy(kvqw_cache* c);

/* Appends n rows per (b, head) at positions P .. P+n-1 ([SK] "KIVI", "Caveats"): the new V rows are
 * quantised per token, and K is re-quantised per channel over every stored row plus the new ones.
 * k, v: [batch][n_kv_heads][n][head_dim] in_dtype, 16-byte aligned.  The rows stored from
 * max(lo, n_sink) to P+n-1 must fit the capacity - n_sink ring slots (else KVQ_ECAPACITY: evict
 * first).  Two kernel launches (per-tile channel min/max, then the re-quantisation); ws as
 * kvqw_workspace_bytes. */
kvq_status kvqw_append(kvqw_cache* c, int32_t layer, const void* k, const void* v, int32_t n, void* ws,
                       size_t ws_bytes, void* stream);

/* StreamingLLM eviction ([SK] "Implementation"): lo = max(lo, P - window) when window > 0.  Host
 * state only; moves no data. */
kvq_status kvqw_evict(kvqw_cache* c, int32_t layer);

/* Single-query decode attention over the stored rows:
 * out[b][j] = sum_p softmax_p(scale * q[b][j] . k_p) v_p with k_p, v_p the dequantised rows
 * u*scale + zero.  q: [batch][n_q_heads][head_dim] in_dtype; out: fp32, same
 * shape.  scale <= 0 means 1/sqrt(head_dim).  Two launches (split partials, then a merge in fixed
 * split order); deterministic.  KVQ_ERANGE on an empty layer. */
kvq_status kvqw_decode_attn(kvqw_cache* c, int32_t layer, const void* q, float* out, float scale, void* ws,
                            size_t ws_bytes, void* stream);

/* fp16 values of positions [pos0, pos0+count) (which: 0 = K, 1 = V), computed in fp32 as
 * u*scale + zero and rounded once to fp16.  Every position must be stored (else KVQ_ERANGE).
 * out: [batch][n_kv_heads][count][head_dim]. */
kvq_status kvqw_dequant(kvqw_cache* c, int32_t layer, int32_t which, int64_t pos0, int32_t count, uint16_t* out,
                        void* stream);

/* Byte accounting of `layer` by the storage layout ([SK] "Cache-bytes table"). Host only. */
kvq_status kvqw_account(const kvqw_cache* c, int32_t layer, kvqw_bytes* out);

/* Host state of `layer`: appended length P and eviction boundary lo. */
kvq_status kvqw_get_state(const kvqw_cache* c, int32_t layer, int64_t* P, int64_t* lo);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_WHOLE_H */
