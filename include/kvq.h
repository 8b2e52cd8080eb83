/*
 * kvq.h — C ABI of the quantized KV cache library for AMD MI355X (gfx950).
 *
 * The library keeps a per-layer KV cache of fixed-size 32-token blocks in
 * HBM, quantizes keys and values on append, protects attention-sink tokens
 * and a recent window in fp16, evicts the middle of long streams in O(1), and
 * runs single-query decode attention directly over the packed cache.
 *
 * The method follows four web pages, cited by title and section:
 *   [SK]  "StreamingLLM + KIVI — long-context decode without growing the KV cache"
 *   [TQ]  "TurboQuant KV Cache Compression — Spec"
 *   [Q2K] "KV cache: FP16 sliding window + attention sinks, and an optional
 *          2-bit K / 4-bit V cache scheme (--kv q2k)"
 *   [KS]  "KVSink-Adapted Sink Protection"
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named dev_* / k / v / q / out / ws are DEVICE pointers owned by
 *    the caller.  The library never allocates or frees device memory and
 *    never synchronises, except where an entry point says so.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every launch is asynchronous on that stream; calls for one cache must be
 *    issued on one stream (or ordered by the caller).
 *  - Host-side validation runs before any launch: on error nothing is
 *    launched, the cache state is unchanged, the call returns a negative
 *    kvq_status and kvq_last_error() describes it.  Nothing aborts.
 *  - Inputs must be finite with |x| <= 32768 (fp16-representable metadata).
 *
 * Shapes (all row-major, contiguous):
 *   K, V chunk    [batch][n_kv_heads][n][head_dim]   fp16 or fp32 (in_dtype)
 *   q             [batch][n_q_heads][head_dim]       fp16 or fp32 (in_dtype)
 *   out           [batch][n_q_heads][head_dim]       fp32
 *   dequant out   [batch][n_kv_heads][count][head_dim] fp16 bit patterns
 * Query head j reads KV head j / (n_q_heads / n_kv_heads).
 *
 * Storage format (one caller buffer; offsets from kvq_get_layout)
 * ---------------------------------------------------------------
 *  Stream = (layer, b, kv head).  Positions are absolute; the bulk of each
 *  stream is a ring of cap_blocks = capacity/32 block records, block beta in
 *  slot beta % cap_blocks.  A record is
 *      [K codes | V codes | K meta | V meta]
 *  * Word-interleaved packing: a little-endian 32-bit word holds 32/b codes
 *    of b bits; code k of the word is at bit 16*(k%2) + b*(k/2).
 *  * K codes: token row t of the block at byte t*D*bK/8, channels in order.
 *  * V codes: 64 chunks of D*bV/16 bytes; chunk 16*kg + i holds, in order
 *    k = 8*mu + e, the code of channel 16*mu + i of token
 *    T(kg, e) = 16*(e/4) + 4*kg + e%4  (kg 0..3, i 0..15, mu 0..D/16-1, e 0..7).
 *  * KIVI: K meta = scale fp16[D] then zero fp16[D]; V meta = scale
 *    fp16[16][D/32][2] then zero fp16[16][D/32][2] (token t, group g at
 *    [t/2][g][t%2]: the two tokens of a pair are adjacent per group).  Codes are unsigned offsets
 *    u = rint((x - zero)/scale) clamped to [0, 2^b - 1], computed against the
 *    stored fp16 scale and zero ([SK] "Affine quantisation formula").
 *  * Q2K: K meta = block RMS fp16[D], K code = number of Gaussian Lloyd-Max
 *    thresholds <= x/rms; V meta = scale fp16[16][D/32][2], V code = q + 8 with
 *    q = clamp(rint(x/scale), -8, 7), scale = absmax/7 ([Q2K] "Summary").
 *  * TQ: K meta = fp32 norm[32], V meta = fp32 norm[32] of the rotated row;
 *    codes are Lloyd-Max Beta(D/2, D/2) indices of the rotated, normalised
 *    coordinates ([TQ] "As-Built Notes", "Step 1", "Step 2"); 3-bit codes sit
 *    in 4-bit slots (b = 4 above: two per byte, two bits unused, [TQ] "Step 3"),
 *    or with tq_dense3 form one little-endian 3-bit stream per section (K: the
 *    token rows in order; V: the 64 chunks in order; code i at bits 3i..3i+2).
 *  * Sink rows and rows not yet appended hold code 0 and V metadata 0.
 *  Per-stream extras: K staging rows of the open block (in_dtype, KIVI and
 *  Q2K), fp16 window ring [residual][D] for K and V (slot p % residual), fp16
 *  sink pool [n_sink][D] for K and V; per (layer, b): sink positions int32
 *  [n_sink] (-1 empty), sink scores fp32 [n_sink], sink count int32.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_cache kvq_cache; /* opaque host handle, owned by the library */

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,    /* bad argument, shape or configuration */
  KVQ_ERANGE = -2,    /* position range not valid (evicted, not appended, empty cache) */
  KVQ_ECAPACITY = -3, /* the append would overwrite a live block (evict first) or exceed capacity */
  KVQ_EORDER = -4,    /* call-order violation (TOPK append without select of the same chunk) */
  KVQ_EDEVICE = -5    /* a HIP call or kernel launch failed */
} kvq_status;

enum { KVQ_FMT_KIVI = 0, KVQ_FMT_Q2K = 1, KVQ_FMT_TQ = 2 };
enum { KVQ_SINK_NONE = 0, KVQ_SINK_FIRST_N = 1, KVQ_SINK_TOPK = 2 };
enum { KVQ_IN_F16 = 0, KVQ_IN_F32 = 1 };

typedef struct {
  int32_t n_layers;   /* >= 1 */
  int32_t batch;      /* >= 1 */
  int32_t n_kv_heads; /* >= 1 */
  int32_t n_q_heads;  /* multiple of n_kv_heads, ratio <= 16 */
  int32_t head_dim;   /* 32, 64 or 128; with TQ also 96 or 160, stored zero-padded to the next power of two
                         (128, 256: [TQ] "Hadamard Transform Detail", every rotated coordinate kept), so
                         every per-row width of the layout is that stored width; top-k sinks need head_dim
                         32, 64 or 128 */
  int32_t format;     /* KVQ_FMT_*: KIVI bits (k,v) each in {2,4,8}; Q2K (2,4); TQ each in {2,3,4} (3-bit codes
                         two per byte with two bits unused, [TQ] "Step 3: Packing": stored as 4-bit slots) */
  int32_t k_bits, v_bits;
  int32_t sink_mode;  /* KVQ_SINK_*; n_sink = 0 means no sinks in any mode */
  int32_t n_sink;     /* 0 .. 16 */
  int32_t window;     /* StreamingLLM window W ([SK] "Implementation"); 0 = never evict */
  int32_t residual;   /* fp16 recent overlay R ([Q2K] "Summary"); 0 allowed */
  int32_t capacity;   /* block slots * 32 per stream; 0 = library default (needs window > 0) */
  int32_t in_dtype;   /* KVQ_IN_F16 or KVQ_IN_F32 for K, V and q */
  uint64_t seed;      /* TQ sign-diagonal seed ([TQ] "Step 1") */
  int32_t rope;       /* 1: K and q are handed over before RoPE and attention turns them on read by their
                         index in the compressed cache ([SK] "RoPE caveat", "Caveats": StreamingLLM's
                         re-positioning); 0: off.  Not with TQ. */
  float rope_base;    /* RoPE base (<= 0: 10000); channel c < head_dim/2 pairs with c + head_dim/2 and turns
                         by the exact angle idx * theta_c, theta_c = base^(-2c/head_dim) rounded to fp32,
                         idx = the number of valid positions before the row (a query: before its own
                         position); capacity + n_sink must stay below 2^24.  On the matrix-core decode path
                         (head_dim 128, fp16, KIVI with k_bits = v_bits) the turned keys enter the matrix
                         cores as fp16 pairs and must stay below 65504 in magnitude. */
  int32_t tq_dense3;  /* TQ with a 3-bit side: 1 stores 3-bit codes as a dense stream, 8 codes in 3 bytes
                         ([TQ] "Step 3: Packing"; code i of a section's sequence at bits 3i .. 3i+2, LSB
                         first); 0 (default) two per byte in 4-bit slots */
} kvq_config;

typedef struct {
  int64_t n_valid, n_compressed, n_sink, n_residual, current_length;
  int64_t compressed_bytes, sink_fp16_bytes, residual_fp16_bytes;
} kvq_bytes;

typedef struct { /* byte offsets inside the caller's device buffer */
  uint64_t layer_stride;          /* layer l's regions start at l * layer_stride */
  uint64_t bulk;                  /* [batch][n_kv_heads][cap_blocks][record_bytes] */
  uint64_t record_bytes;
  uint64_t rec_k_codes, rec_v_codes, rec_k_meta, rec_v_meta; /* section offsets inside a record */
  uint64_t staging;               /* [batch][n_kv_heads][32][head_dim] in_dtype (0 if unused) */
  uint64_t win_k, win_v;          /* [batch][n_kv_heads][residual][head_dim] fp16 */
  uint64_t sink_k, sink_v;        /* [batch][n_kv_heads][n_sink][head_dim] fp16 */
  uint64_t sink_pos, sink_score, sink_count; /* [batch][n_sink] int32, fp32; [batch] int32 */
  uint64_t decode_sync;           /* [batch][n_kv_heads] uint32: arrival counters of the decode workgroups
                                     of one call (the last to arrive merges the stream); zero between calls */
  uint64_t tables;                /* once, not per layer: fp32 tables (TQ signs and codebooks, Q2K grid) */
  uint64_t select_work;           /* once, not per layer (TOPK mode): [batch][64][n_sink] (fp32 score, int32
                                     position) top-k lists of the workgroups of one sink-selection call;
                                     contents between calls carry no state */
  uint64_t total;                 /* = kvq_required_bytes */
  int32_t cap_blocks;
  int32_t capacity;
} kvq_layout;

/* Validates a configuration ([SK] "Implementation" flags; [KS] "Usage" fields). */
kvq_status kvq_config_check(const kvq_config* cfg);

/* Device bytes the cache needs (all layers); 0 for an invalid configuration. */
size_t kvq_required_bytes(const kvq_config* cfg);

/* Offsets of every region of the documented storage format. */
kvq_status kvq_get_layout(const kvq_config* cfg, kvq_layout* out);

/* Device bytes of the workspace kvq_decode_attn needs (split partials). */
size_t kvq_workspace_bytes(const kvq_config* cfg);

/* Binds a cache to the caller's device buffer dev_buf (>= kvq_required_bytes,
 * 256-byte aligned).  Clears the buffer and writes the format tables on
 * `stream` (asynchronously); the buffer must outlive the handle.  The TQ
 * sign diagonal and Lloyd-Max codebooks, and the Q2K Gaussian grid, are
 * computed here on the host ([TQ] "Codebook Generation"). */
kvq_status kvq_create(const kvq_config* cfg, void* dev_buf, size_t dev_bytes, void* stream, kvq_cache** out);

/* Frees the host handle.  Does not touch device memory. */
kvq_status kvq_destroy(kvq_cache* c);

/* Sink selection for the next chunk of n rows of `layer` ([KS] "How it
 * works", 1): per-token key L2 norm averaged over KV heads, folded into a
 * running top-k of absolute positions; new rows of that top-k join the
 * permanent sink set while it has room ([KS] "Fidelity to the paper": no
 * retroactive restore).  k: [batch][n_kv_heads][n][head_dim], 16-byte
 * aligned in TOPK mode (else KVQ_EINVAL).  Required before kvq_append in TOPK
 * mode (else KVQ_EORDER); a no-op in other modes.  Each call commits
 * min(n_sink - |C|, n) rows, so |C| = min(n_sink, P) and a call at
 * P >= n_sink launches nothing.  Uses the cache's select_work area: calls on
 * one cache must be ordered (one stream). */
kvq_status kvq_select_sinks(kvq_cache* c, int32_t layer, const void* k, int32_t n, void* stream);

/* Appends n rows of K and V at positions [P, P+n) of `layer` and quantizes
 * them ([SK] "KIVI", "Affine quantisation formula"; [Q2K]; [TQ]): V per
 * token, K per channel over its 32-token block (the open block is
 * re-quantized from its staged rows until it is complete); sink rows are
 * excluded from calibration and copied to the fp16 sink pool ([KS] 2-3); the
 * last `residual` rows are copied to the fp16 window ring.  Fails with
 * KVQ_ECAPACITY if a written block slot still holds a live block, and with
 * KVQ_ERANGE if a position would reach 2^31 (positions are int32 on the
 * device). */
kvq_status kvq_append(kvq_cache* c, int32_t layer, const void* k, const void* v, int32_t n, void* stream);

/* StreamingLLM eviction of positions [sink, P - window) ([SK]
 * "Implementation"): host-only O(1) update of the valid range, after which
 * the valid set is (sinks) U [max(lo, P - window), P).  No-op when window = 0. */
kvq_status kvq_evict(kvq_cache* c, int32_t layer);

/* Single-query decode attention over the valid set of `layer`:
 * out[b][j] = sum_p softmax_p(scale * q[b][j] . k_p) v_p, with k_p, v_p read
 * from the sink pool, else the fp16 window, else dequantized in registers
 * from the packed bulk ([SK] "Affine quantisation formula"; [TQ]
 * "Optimization: Fused dequant-dot": TQ scores and values are accumulated in
 * the rotated domain and the output is rotated back once).  scale <= 0 means
 * 1/sqrt(head_dim).  ws: >= kvq_workspace_bytes device bytes (split partials).
 * Split-K: every workgroup writes one online-softmax partial; on the matrix-core
 * path (head_dim 128, fp16 queries) the last workgroup of a stream to finish
 * merges the stream's partials in fixed order in the same launch (counters in
 * the cache's decode_sync region), elsewhere a second launch merges them;
 * results are deterministic. */
kvq_status kvq_decode_attn(kvq_cache* c, int32_t layer, const void* q, float* out, float scale, void* ws,
                           size_t ws_bytes, void* stream);

/* One decode step of `layer` for one new row: kvq_select_sinks (top-k mode), kvq_append (1 row), kvq_evict
 * and kvq_decode_attn, in this order ([SK] "Implementation": per layer and step, append, evict, attend;
 * [KS] "How it works"), with the same results, stored bytes and state as those four calls.  k, v:
 * [batch][n_kv_heads][1][head_dim] in_dtype; q, out, scale, ws, ws_bytes as in kvq_decode_attn.  When the
 * row changes no sink (the committed set already holds min(n_sink, P) rows and n_sink <= P), completes
 * no block, the cache defers open blocks (block formats, fp16 input, residual >= 32) and the shape has
 * the matrix-core decode kernel (k and v 16-byte aligned), the step is one launch: the decode kernel's
 * first fp16-row workgroup of each stream copies the row into the staging rows and the fp16 window
 * (and zeroes the record of a block the row opens) while the row is scored straight from k and v.
 * Otherwise the four calls run as separate launches.  Errors as in those calls; on an error nothing is
 * launched and the state is unchanged. */
kvq_status kvq_decode_step(kvq_cache* c, int32_t layer, const void* k, const void* v, const void* q, float* out,
                           float scale, void* ws, size_t ws_bytes, void* stream);

/* Size of the static decode workspace kvq_decode_attn_nomalloc uses: 32 MiB of device memory per GPU,
 * held from the library's first use on that GPU until the process ends. */
#define KVQ_STATIC_WS_BYTES ((size_t)32 << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): kvq_decode_attn with the split partials in a workspace the library
 * holds in static device memory (KVQ_STATIC_WS_BYTES per GPU) instead of a caller's `ws`.  Same
 * arguments, kernels and results as kvq_decode_attn; allocates nothing.  Run it with the cache's device
 * current.  Fails with KVQ_ECAPACITY, launching nothing, when the call's split partials need more than
 * KVQ_STATIC_WS_BYTES (streams x (splits + fp16-row groups) x (n_q_heads / n_kv_heads) x
 * (head_dim + 2) x 4 bytes; with RoPE on read, batch x n_q_heads x splits x (head_dim + 4) x 4).
 * Every call on one GPU shares that GPU's workspace: calls that overlap in time on one GPU (different
 * streams, or different host threads without ordering) race and give wrong results.  Nothing in it
 * needs clearing between calls (each call writes every partial it reads). */
kvq_status kvq_decode_attn_nomalloc(kvq_cache* c, int32_t layer, const void* q, float* out, float scale,
                                    void* stream);

/* Causal multi-query attention of a prefill chunk over `layer` (the "next"
 * step after append in prefill: [Q2K] "Summary" reads prefill through the
 * same q2k cache; [TQ] "API" attention over the cached rows).  q: the
 * queries of the last n appended positions P-n .. P-1, [batch][n_q_heads][n]
 * [head_dim] in_dtype, 16-byte aligned; out: [batch][n_q_heads][n][head_dim]
 * fp32, 16-byte aligned.  Query i attends the valid positions p <= P-n+i
 * (sinks, window, bulk; the same values decode attention reads) with
 * softmax(scale * q . k) weights; a query with no such position gets zeros.
 * scale <= 0 means 1/sqrt(head_dim).  Every cache format (TurboQuant in the
 * rotated domain: queries rotated once, outputs rotated back); fp32
 * queries enter the matrix cores as fp16 hi + lo pairs; head_dim 32, 64 or
 * 128, or TQ's padded 96 and 160 (else KVQ_EINVAL); 1 <= n <= P (else
 * KVQ_ERANGE).  One kernel launch, no workspace; deterministic. */
kvq_status kvq_prefill_attn(kvq_cache* c, int32_t layer, const void* q, int32_t n, float* out, float scale,
                            void* stream);

/* Materialises fp16 values of positions [pos0, pos0+count) of `layer`
 * (which: 0 = K, 1 = V), read priority sink > window > bulk, bulk values
 * computed in fp32 as the format's dequant formula and rounded once to fp16
 * ([SK] "The bug class the previous attempt hit", 2 and 4).  The range must
 * lie in [lo, P) (else KVQ_ERANGE).  out: [batch][n_kv_heads][count][head_dim]. */
kvq_status kvq_dequant(kvq_cache* c, int32_t layer, int32_t which, int64_t pos0, int32_t count, uint16_t* out,
                       void* stream);

/* Byte accounting of `layer` summed over the batch ([KS] "How it works", 4:
 * sink bytes and residual fp16 bytes separate, no double counting; [SK]
 * "Caveats": current length next to the stored count).  Synchronises
 * `stream` to read the sink counts. */
kvq_status kvq_account(kvq_cache* c, int32_t layer, kvq_bytes* out, void* stream);

/* Host state of `layer`: appended length P and eviction boundary lo. */
kvq_status kvq_get_state(const kvq_cache* c, int32_t layer, int64_t* P, int64_t* lo);

/* Host copies of the tables kvq_create writes: signs[stored width], K boundaries
 * [2^k_bits - 1], K centroids [2^k_bits], V boundaries, V centroids (TQ, in
 * the t = 2u - 1 space), and the Q2K thresholds[3] and levels[4].  Any
 * pointer may be NULL. */
kvq_status kvq_format_tables(const kvq_config* cfg, float* signs, float* k_bnd, float* k_cen, float* v_bnd,
                             float* v_cen, float* q2k_thr, float* q2k_lvl);

/* Text of the last error on the calling thread ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
