/*
 * lazy_attn.h -- C ABI of the lazy-RoPE paged attention library (liblazyattn.so)
 *
 * Attention over a paged key/value block pool whose keys are stored WITHOUT
 * positional encoding.  Rotary position embedding (RoPE) is applied inside the
 * kernels at each request's logical positions, so one physical copy of a
 * document's blocks serves any number of requests that place the document at
 * different prompt offsets, and no re-encoded copy is ever written.  This is
 * the deferred positional encoding of "LazyAttention: Efficient
 * Retrieval-Augmented Generation with Deferred Positional Encoding"
 * (§1 and §3.1 "Deferred encoding"; problem statement of §3: the same
 * document at different offsets within one batch).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All functions return la_status and never throw.  On failure
 *    lazy_attn_last_error() returns a message for the calling thread.
 *  - Pointers marked "device" are GPU memory owned by the caller; "host"
 *    pointers are CPU memory owned by the caller.  The library allocates no
 *    device memory and keeps no state besides the per-thread error message.
 *  - GPU entry points enqueue work on the caller's stream (a hipStream_t passed
 *    as void*, NULL = default stream) and return without synchronising.
 *    Scalar arguments are checked before anything is enqueued; the contents of
 *    device arrays are NOT checked on the device (use the host-side
 *    lazy_attn_pack_segments / lazy_attn_validate_table for that, or set
 *    la_params.check_tables).  Malformed device tables give undefined results.
 *  - Calls are thread-safe; concurrent calls on one stream serialise in order.
 *
 * RoPE convention (readings of the paper, stated once here)
 * ---------------------------------------------------------
 *  Feature pair (i, i + D/2), i < D/2, is rotated by angle p * theta_i with
 *  theta_i = base^(-2i/D):  y_i = x_i cos - x_{i+D/2} sin,
 *  y_{i+D/2} = x_i sin + x_{i+D/2} cos  (§3.2 "Prefilling", rotation over the
 *  two half-dimensions).  The score of a query at position m and a key at
 *  position p is scale * (R_m q)^T (R_p k) = scale * q^T R_{p-m} k (§3.2,
 *  Fact 3.2).  Query head h reads kv head h / (num_q_heads / num_kv_heads)
 *  (§3.5 "GQA/MQA").  This is the default (LA_ROPE_HALF); la_pos_encoding
 *  below selects interleaved pairs or ALiBi instead.
 *
 * Data layouts (row-major, contiguous)
 * ------------------------------------
 *  k_pool   [num_blocks][num_kv_heads][block_size][head_dim]   un-rotated K
 *           (LA_POOL_POSITION_FREE; see la_pool_mode and la_pos_encoding
 *           for the other stored forms)
 *  v_pool   [num_blocks][num_kv_heads][head_dim][block_size]   V, dim-major
 *           inside each (block, kv head) tile, so the token axis -- the
 *           contraction axis of P.V -- is contiguous.  Why: the MFMA A operand
 *           of the P.V product is 4 (decode) or 8 (prefill) consecutive keys
 *           of one dimension, which this layout makes one 8- or 16-byte load
 *           (and lets prefill copy V tiles to LDS unchanged); a token-major
 *           tile would need a transpose per operand.  lazy_attn_store_kv
 *           writes this layout from token-major [token][kv head][dim] input.
 *  cos_sin  float32 [max_pos][2][head_dim/2]: row p holds cos(p theta_i) then
 *           sin(p theta_i).  Build it with lazy_attn_rope_table or
 *           lazy_attn_rope_table_scaled (float64 arithmetic, rounded once to
 *           float32).  Always float32.  With LA_ALIBI this argument carries
 *           the per-head slopes instead.
 *  q / out  decode:  [batch][num_q_heads][head_dim]
 *           prefill: [total_q][num_q_heads][head_dim], rows cu_q[r] ..
 *           cu_q[r+1]-1 are request r's new tokens.
 *           Element type is bf16 (LA_BF16) or float32 (LA_FP32, test mode) for
 *           q, out, k_pool and v_pool alike.
 *  lse      float32, [batch][num_q_heads] or [total_q][num_q_heads], natural
 *           log of the softmax denominator including the max; nullable.
 *
 * Block table (per request, CSR)
 * ------------------------------
 *  blk_words[req_blk_start[r] .. req_blk_start[r+1]-1] describe request r's
 *  blocks, in any order.  Each 64-bit word packs (§3.2 "Decoding": block id,
 *  offset and mask bit-packed into one 64-bit register):
 *     bits  0..31  physical block id
 *     bits 32..55  pos0: logical position of the block's slot 0 (cached
 *                  blocks of a LA_POOL_DOC_LOCAL pool: the segment start)
 *     bits 56..62  n_valid - 1: slots 0 .. n_valid-1 hold tokens
 *     bit  63      causal: the block holds new prompt tokens of a prefill
 *                  request; its key at position p is visible to a query at
 *                  position m only when p <= m.  Ignored by decode.
 *  Slot i of a block is the token at logical position pos0 + i (position-free
 *  pools).
 */
#ifndef LAZY_ATTN_H
#define LAZY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define LA_API __attribute__((visibility("default")))
#else
#define LA_API
#endif

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1,         /* null pointer, bad size, malformed table */
  LA_ERR_UNSUPPORTED = 2,         /* head_dim / block_size / dtype / group not built */
  LA_ERR_WORKSPACE_TOO_SMALL = 3, /* decode workspace below the queried size */
  LA_ERR_HIP = 4                  /* HIP runtime error (incl. no device) */
} la_status;

typedef enum la_dtype { LA_BF16 = 0, LA_FP32 = 1 } la_dtype;

/*
 * What k_pool holds.
 *  LA_POOL_POSITION_FREE (default): keys without positional encoding; the
 *    kernels rotate every key at its logical position (deferred encoding,
 *    §3.1).  Block words carry pos0 = logical position of slot 0.
 *  LA_POOL_DOC_LOCAL: each key stored pre-rotated by its index t within its
 *    segment (R_t k: each document's cache numbered from position 0, §3.2
 *    "Prefilling" and Example 3.1).  Words of cached (non-causal) blocks carry pos0 = the
 *    segment's logical start s for every block of the segment, and the score
 *    (R_m q)^T (R_{s+t} k) is computed as (R_{m-s} q)^T (R_t k) in decode --
 *    one rotation of q per segment, none of the keys (§3.2 "Decoding",
 *    Eq. 6) -- and as (R_m q)^T (R_s (R_t k)) in prefill -- one relative
 *    rotation per key, with one cos/sin row per segment (§3.2 "Prefilling").
 *    The new tokens of a prefill request form one causal segment starting at
 *    q_pos0, stored as R_t k with t counted from q_pos0; its words keep slot
 *    0's logical position (the causal mask needs it) and are rotated by
 *    q_pos0.  Decode tables must not flag blocks causal in this mode.  A pool
 *    pre-rotated at absolute positions is the special case s = 0.
 *    Tables whose rows carry an amplitude a (cos and sin both times a, as
 *    lazy_attn_rope_table_scaled writes for YaRN) give every score a^2 in
 *    every mode: stored keys written with such a table carry a once, decode
 *    rotates q with the table (a), and prefill divides its relative key
 *    rotation by a, read as row 0's first cosine (a * cos 0).
 */
typedef enum la_pool_mode { LA_POOL_POSITION_FREE = 0, LA_POOL_DOC_LOCAL = 1 } la_pool_mode;

/*
 * Positional encoding applied inside the kernels (§3.5 "Generalization Beyond
 * Standard RoPE": the score stays q^T R_{n-m} k for RoPE-family variants, or
 * gets a position-dependent bias for score-space methods).
 *  LA_ROPE_HALF (default): RoPE on feature pairs (i, i + D/2).
 *  LA_ROPE_INTERLEAVED: RoPE on adjacent pairs (2i, 2i + 1) of q and k.
 *    lazy_attn_store_kv stores such keys with their dimensions reordered to
 *    (even dims, odd dims), which turns every pair into (i, i + D/2); k_pool
 *    then holds keys in that order (write it with lazy_attn_store_kv, or apply
 *    the same reordering).  q, v and out keep the model's order.
 *  LA_ALIBI: no rotation; the score of a key at position p for a query at m
 *    gets slope_h * (p - m) (-slope_h times the distance for keys at or
 *    before the query).  The cos_sin argument of decode/prefill then points
 *    to the per-query-head slopes, float32 [num_q_heads]
 *    (lazy_attn_alibi_slopes gives the standard ones).  Position-free pools
 *    only.
 * Scaled / NTK / YaRN RoPE variants change only the cos/sin table.
 */
typedef enum la_pos_encoding {
  LA_ROPE_HALF = 0,
  LA_ROPE_INTERLEAVED = 1,
  LA_ALIBI = 2
} la_pos_encoding;

/* Packing limits of the 64-bit block word. */
#define LA_MAX_POSITION ((int64_t)1 << 24) /* positions must be < 2^24 */
#define LA_MAX_BLOCK_ID ((int64_t)1 << 32)

typedef struct la_params {
  int32_t num_q_heads;   /* Hq; a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* D: 128 (bf16 and fp32) or 64 (fp32 only) */
  int32_t block_size;    /* tokens per block: 16 */
  int64_t num_blocks;    /* blocks in the pool */
  int32_t dtype;         /* la_dtype of q, out, k_pool, v_pool */
  float scale;           /* multiplies q.k; usually 1/sqrt(head_dim) */
  int32_t max_pos;       /* rows of cos_sin; every position must be < max_pos */
  int32_t split_blocks;  /* decode: blocks per split group, 0 = automatic */
  int32_t target_workgroups; /* decode split heuristic, 0 = 512 (256 CUs x 2) */
  int32_t pool_mode;     /* la_pool_mode of k_pool (above) */
  int32_t pos_encoding;  /* la_pos_encoding (above) */
  int32_t check_tables;  /* nonzero: GPU entry points check their tables first (below) */
  int32_t reserved[2];   /* must be zero */
} la_params;

/*
 * check_tables (debugging).  When nonzero, every GPU entry point -- decode,
 * decode_noalloc, decode_shared, prefill, store_kv -- first waits for its
 * stream (hipStreamSynchronize), copies the tables it would read to the host
 * and checks them: the block words, req_blk_start, q_pos and cu_q with the
 * checks of lazy_attn_validate_table (with the call's max_blocks_per_req /
 * max_q_per_req); a shared-decode plan against the batch (item, member and
 * word ranges, every partial slot written exactly once and inside its
 * request's range, block ids inside the pool, every table row the kernel
 * reads -- |m - s|, t0 and the keys' positions -- inside max_pos); the cache
 * write's slots (inside the pool, distinct) and rotation positions.  A table
 * that fails returns LA_ERR_INVALID_ARG and nothing is enqueued.  Each call
 * then costs a device synchronisation and a copy of its tables; with 0 (the
 * default) the contents of device arrays are not checked at all.
 */

/* Human-readable name of a status code (static string). */
LA_API const char* lazy_attn_status_string(la_status s);

/* Message describing the last failure on the calling thread ("" if none). */
LA_API const char* lazy_attn_last_error(void);

/*
 * Fill a host cos/sin table: out[p][0][i] = cos(p theta_i),
 * out[p][1][i] = sin(p theta_i), theta_i = base^(-2i/head_dim), computed in
 * float64 and rounded once to float32 (stateless per row: no incremental
 * rotation updates, so no error accumulates along positions -- App. C.4).
 *   base      RoPE base (> 1), e.g. 10000 or 500000
 *   head_dim  even, 2 .. 1024
 *   rows      number of positions (>= 1)
 *   out       host, rows * head_dim floats
 */
LA_API la_status lazy_attn_rope_table(double base, int32_t head_dim, int32_t rows, float* out);

/*
 * Scaled RoPE variants (§3.5: scaled / NTK / YaRN keep the score
 * q^T R_{n-m} k; only the cos/sin table changes).  The published variants:
 *  LA_SCALING_LINEAR  position interpolation: theta_i / factor
 *  LA_SCALING_NTK     NTK-aware: base * factor^(D / (D - 2))
 *  LA_SCALING_YARN    per pair, theta_i for pairs that turn more than
 *                     beta_fast times over original_max_pos, theta_i / factor
 *                     for pairs that turn less than beta_slow times, a linear
 *                     ramp over the pair index in between (ramp ends: the
 *                     fractional pair indices of beta_fast rounded down and of
 *                     beta_slow rounded up, clamped to [0, head_dim - 1] as in
 *                     the published correction range); cos and sin are
 *                     multiplied by attn_factor (0 = 0.1 ln(factor) + 1)
 *  LA_SCALING_LLAMA3  wavelength 2 pi / theta_i below original_max_pos /
 *                     high_freq_factor kept, above original_max_pos /
 *                     low_freq_factor divided by factor, smooth in between
 */
typedef enum la_rope_scaling_type {
  LA_SCALING_NONE = 0,
  LA_SCALING_LINEAR = 1,
  LA_SCALING_NTK = 2,
  LA_SCALING_YARN = 3,
  LA_SCALING_LLAMA3 = 4
} la_rope_scaling_type;

typedef struct la_rope_scaling {
  int32_t type;              /* la_rope_scaling_type */
  int32_t original_max_pos;  /* YARN, LLAMA3: pre-training context length */
  double factor;             /* > 0 (1 = no scaling) */
  double low_freq_factor;    /* LLAMA3 */
  double high_freq_factor;   /* LLAMA3, > low_freq_factor */
  double beta_fast;          /* YARN, e.g. 32 */
  double beta_slow;          /* YARN, e.g. 1 */
  double attn_factor;        /* YARN, 0 = default */
} la_rope_scaling;

/*
 * lazy_attn_rope_table with a scaled variant (NULL or LA_SCALING_NONE: the
 * plain table).  Same layout, float64 arithmetic, one rounding to float32.
 */
LA_API la_status lazy_attn_rope_table_scaled(double base, int32_t head_dim, int32_t rows,
                                             const la_rope_scaling* scaling, float* out);

/*
 * Standard ALiBi slopes for num_heads heads (host): 2^(-8/n), 2^(-16/n), ...
 * for n a power of two; otherwise the nearest lower power of two's sequence
 * followed by every other slope of the next power of two's sequence.
 *   out  host, num_heads floats
 */
LA_API la_status lazy_attn_alibi_slopes(int32_t num_heads, float* out);

/*
 * Pack per-request segment lists into block words (host only).
 * A segment is a run of n tokens at logical positions start .. start+n-1 whose
 * token t lives in block blocks[t / block_size], slot t % block_size.
 *   batch           number of requests (>= 1)
 *   req_seg_start   host [batch+1]: request r owns segments req_seg_start[r] ..
 *   seg_start       host [S] logical position of each segment's token 0
 *   seg_len         host [S] tokens per segment (>= 1)
 *   seg_is_new      host [S] 1 = new prompt tokens (causal), 0 = cached
 *   seg_blk_start   host [S+1]: segment s owns seg_blocks[seg_blk_start[s] ..]
 *   seg_blocks      host block ids; a segment needs ceil(len/block_size) of them
 *   blk_words       host out [capacity]
 *   req_blk_start   host out [batch+1]
 *   max_blocks_per_req  host out (nullable): largest per-request block count
 * Checks block ids < num_blocks, positions < min(max_pos, 2^24), block counts,
 * and that every request has at least one token.  Returns LA_ERR_INVALID_ARG
 * (nothing written beyond what was checked) on violation.  With
 * LA_POOL_DOC_LOCAL the position field of every word of a cached segment is
 * the segment start (new-token segments keep per-block positions).
 */
LA_API la_status lazy_attn_pack_segments(const la_params* p, int32_t batch, const int64_t* req_seg_start,
                                  const int64_t* seg_start, const int64_t* seg_len,
                                  const uint8_t* seg_is_new, const int64_t* seg_blk_start,
                                  const int64_t* seg_blocks, uint64_t* blk_words,
                                  int64_t capacity, int32_t* req_blk_start,
                                  int32_t* max_blocks_per_req);

/*
 * Check a packed table against the pool and position limits (debug helper).
 * Arrays may be host or device memory (device ones are copied synchronously).
 *   blk_words      rows 0 .. req_blk_start[batch]-1 are read; row b is
 *                  blk_words[b] (the absolute index the kernels use, also when
 *                  req_blk_start[0] > 0)
 *   q_pos   decode: query position per request; prefill: position of the
 *           first new token per request
 *   cu_q    prefill: [batch+1] query row offsets; NULL for decode
 *   max_blocks_per_req  the value that will be passed to lazy_attn_decode
 *           (0 = not checked): a request with more blocks fails validation
 *   max_q_per_req       the value that will be passed to lazy_attn_prefill
 *           (0 = not checked): a request with more query rows fails
 * Decode requires every key position < max_pos and q_pos < max_pos; prefill
 * requires q_pos + (cu_q[r+1]-cu_q[r]) - 1 < max_pos and that each new-token
 * row sees at least one key.  With LA_POOL_DOC_LOCAL, decode tables may not
 * hold causal words and a prefill causal word must start a block of the
 * new-token segment (pos0 - q_pos a multiple of block_size, >= 0).
 */
LA_API la_status lazy_attn_validate_table(const la_params* p, int32_t batch, const uint64_t* blk_words,
                                   const int32_t* req_blk_start, const int32_t* q_pos,
                                   const int32_t* cu_q, int32_t max_blocks_per_req,
                                   int32_t max_q_per_req);

/*
 * Bytes of device workspace lazy_attn_decode needs for this shape (0 when the
 * split heuristic keeps one split group per (request, kv head)).  Depends only
 * on the arguments, not on the device.
 */
LA_API la_status lazy_attn_decode_workspace_size(const la_params* p, int32_t batch,
                                          int32_t max_blocks_per_req, size_t* bytes);

/*
 * Write n_tokens keys and values into pool slots (the cache write that
 * precedes attention; keys are stored once and never re-encoded).  With
 * LA_ROPE_INTERLEAVED keys are rotated on pairs (2i, 2i + 1) and stored in
 * (even dims, odd dims) order.
 *   k, v       device [n_tokens][num_kv_heads][head_dim], pool dtype
 *   slots      device int64 [n_tokens]: block_id * block_size + slot
 *   rope_pos   device int32 [n_tokens] or NULL.  NULL stores keys as given
 *              (position-free pool); otherwise key t is stored rotated,
 *              R_{rope_pos[t]} k, computed in fp32 and rounded once -- e.g.
 *              its index within its document for a LA_POOL_DOC_LOCAL pool
 *   cos_sin    device [max_pos][2][head_dim/2] float32; rope_pos < max_pos
 *              (may be NULL when rope_pos is NULL)
 *   k_pool, v_pool  device, layouts above; V is written dim-major
 * Slots must be distinct and < num_blocks * block_size (not checked on the
 * device).  k, v, k_pool and v_pool must be 16-byte aligned.  Asynchronous on
 * stream.
 */
LA_API la_status lazy_attn_store_kv(const la_params* p, const void* k, const void* v,
                                    int64_t n_tokens, const int64_t* slots,
                                    const int32_t* rope_pos, const float* cos_sin, void* k_pool,
                                    void* v_pool, void* stream);

/*
 * Decode: one new query token per request attends exactly the request's
 * listed keys (§3.2 "Decoding"; §3.4 decode roofline: only K and V are read).
 *   q              device [batch][Hq][D]
 *   k_pool/v_pool  device, layouts above
 *   blk_words      device packed words; req_blk_start device [batch+1]
 *   q_pos          device [batch] logical position m of each query
 *   cos_sin        device [max_pos][2][D/2] float32 (LA_ALIBI: the slopes,
 *                  float32 [num_q_heads])
 *   max_blocks_per_req  host scalar: upper bound of per-request block counts.
 *                  The grid (split groups x blocks per group) is sized from
 *                  it, so a request with more blocks has its trailing blocks
 *                  silently ignored (a wrong result with LA_OK); pass it to
 *                  lazy_attn_validate_table to have that checked
 *   out            device [batch][Hq][D] (same dtype as q)
 *   lse            device [batch][Hq] float32 or NULL
 *   workspace      device, >= lazy_attn_decode_workspace_size bytes (may be
 *                  NULL when that size is 0); clobbered
 * Requires every key position p and m in [0, max_pos) and every request
 * non-empty.  bf16 mode needs head_dim 128, block_size 16 and a group size
 * Hq/Hkv in {1, 2, 4, 8, 16}; fp32 mode needs head_dim 64 or 128.
 */
LA_API la_status lazy_attn_decode(const la_params* p, const void* q, const void* k_pool,
                           const void* v_pool, const uint64_t* blk_words,
                           const int32_t* req_blk_start, const int32_t* q_pos,
                           const float* cos_sin, int32_t batch, int32_t max_blocks_per_req,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory or
 * hand the library a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, semantics and
 * kernels as lazy_attn_decode without the workspace pair: the split-group
 * partials live in a fixed device array inside the library,
 * LA_DECODE_NOALLOC_SCRATCH_BYTES per GPU (one copy on each GPU the library
 * runs on, held until the process ends; its address is resolved on the first
 * call on each device).  Shapes whose partials would exceed it (those for
 * which lazy_attn_decode_workspace_size returns more) are rejected with
 * LA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  The call allocates
 * nothing.  Every call on one GPU shares that GPU's array; each launch writes
 * every partial it later reads, so nothing needs clearing between calls, but
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it and must be serialised by the caller.
 */
#define LA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

LA_API la_status lazy_attn_decode_noalloc(const la_params* p, const void* q, const void* k_pool,
                                          const void* v_pool, const uint64_t* blk_words,
                                          const int32_t* req_blk_start, const int32_t* q_pos,
                                          const float* cos_sin, int32_t batch,
                                          int32_t max_blocks_per_req, void* out, float* lse,
                                          void* stream);

/*
 * Shared-segment decode (document-major split-KV).  A position-free pool lets
 * one physical copy of a document serve every request that lists it, at any
 * offset (§1; the same document at different offsets within one batch, §3).
 * This decode also READS each such copy once per launch for all of them: a
 * work item is a chunk of one unit -- a run of blocks, each with the index t0
 * of its slot 0 -- together with up to 32 / G members (request r, start s)
 * that read it; slot i of a block holds the key at logical position
 * s + t0 + i.  A segment several requests list identically is one unit (t0
 * counted inside the segment, s its start in each request).  In a
 * LA_POOL_POSITION_FREE pool the segments only one request lists form that
 * request's private run (t0 absolute, s = 0); in a LA_POOL_DOC_LOCAL pool
 * every segment is a unit of its own.  Keys are rotated by t0 + i, each
 * member's query once per item by m - s (score = (R_{m-s} q)^T (R_t k), the
 * per-document query rotation of §3.2 "Decoding", Eq. 6); a LA_POOL_DOC_LOCAL
 * pool already stores R_t k and is read as stored.  Every (member, chunk)
 * writes one fp32 partial (o, m, l) per query head; a second kernel merges
 * each request's partials.  Same results as lazy_attn_decode (the softmax
 * over exactly the listed keys) up to rounding order.
 *
 * lazy_attn_plan_shared_decode (host) builds the plan from the segment lists
 * lazy_attn_pack_segments takes.  Two segments are the same when they have
 * the same length and block list; their logical starts may differ.  The plan
 * is a flat blob the caller copies to device memory as is:
 *     int32x4 items[n_items]        {first word, blocks, first member, members}
 *     int32x4 members[n_members]    {request, start s, partial slot, 0}
 *     int32   req_part_start[batch + 1], padded to 16 bytes: request r owns
 *                                   partial slots req_part_start[r] ..
 *     uint64  words[n_words]        per chunk block: block id (bits 0..31),
 *                                   t0 (bits 32..55), n_valid - 1 (bits 56..62)
 * It depends on the segments only (not on q_pos), so it can be reused while
 * the tables do not change.
 *   max_item_blocks  longest chunk L, in blocks: a unit of nb blocks is cut
 *                    into ceil(nb / L) chunks of nearly equal length.  0 =
 *                    automatic: the L in 16, 24, .., 96 with the shortest
 *                    launch time under a fluid model of the kernel (tasks =
 *                    items x kv heads, started longest first on the wave slots
 *                    of p->target_workgroups workgroups of four waves, 0 = 512;
 *                    each block step bounded by latency or shared bandwidth;
 *                    plus the partials' write and merge)
 *   info             out: the sizes below, and the L used (passing it back
 *                    as max_item_blocks gives the same plan without the
 *                    search: a caller sizing the blob first, or reusing L
 *                    across steps, pays for the search once)
 *   plan             host out, info->plan_bytes bytes; NULL = sizes only
 *   plan_capacity    bytes available at plan
 * seg_is_new is accepted for symmetry with lazy_attn_pack_segments and not
 * read: a decode query attends every listed key, so no block is causal (in a
 * LA_POOL_DOC_LOCAL pool a new-token segment is read like any other segment,
 * its keys indexed from its own start).
 * bf16 only (LA_ERR_UNSUPPORTED for LA_FP32 and LA_ALIBI); the same checks
 * as lazy_attn_pack_segments.
 */
typedef struct la_shared_plan_info {
  int32_t batch;            /* requests the plan covers */
  int32_t n_items;          /* work items; the launch runs n_items x num_kv_heads workgroups */
  int32_t n_members;        /* (member, chunk) pairs = partial slots */
  int32_t n_words;          /* block words of the distinct chunks */
  int32_t members_per_item; /* at most 32 / (num_q_heads / num_kv_heads) */
  int32_t max_item_blocks;  /* longest chunk allowed, in blocks (the L used) */
  int64_t plan_bytes;       /* size of the plan blob */
  int64_t workspace_bytes;  /* device workspace lazy_attn_decode_shared needs */
} la_shared_plan_info;

LA_API la_status lazy_attn_plan_shared_decode(
    const la_params* p, int32_t batch, const int64_t* req_seg_start, const int64_t* seg_start,
    const int64_t* seg_len, const uint8_t* seg_is_new, const int64_t* seg_blk_start,
    const int64_t* seg_blocks, int32_t max_item_blocks, la_shared_plan_info* info, void* plan,
    int64_t plan_capacity);

/*
 * Decode with a shared-segment plan (see above).
 *   info       host: the plan's sizes, as lazy_attn_plan_shared_decode wrote them
 *   plan       device copy of the plan blob, 16-byte aligned
 *   q, k_pool, v_pool, q_pos, cos_sin, out, lse: as for lazy_attn_decode
 *   workspace  device, >= info->workspace_bytes (the partials); clobbered
 * Requires 0 <= s + t < max_pos for every key, m < max_pos, and a plan built
 * for the same params and batch (not checked on the device; check_tables in
 * la_params checks it on the host).
 */
LA_API la_status lazy_attn_decode_shared(const la_params* p, const la_shared_plan_info* info,
                                         const void* plan, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* q_pos,
                                         const float* cos_sin, int32_t batch, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * Prefill: the new prompt tokens of each request attend every cached key of
 * the request and, among the new tokens, causally (§3.2 "Prefilling"; §3.4
 * Eq. 7 TTFT model: attention of the L' new tokens against all L keys).
 *   q          device [total_q][Hq][D]; cu_q device [batch+1]
 *   q_pos0     device [batch]: logical position of request r's first new
 *              token; new token j sits at q_pos0[r] + j
 *   max_q_per_req  host scalar: upper bound of cu_q[r+1] - cu_q[r].  The
 *              grid's q tiles are sized from it: rows of a longer request
 *              beyond it are never written (lazy_attn_validate_table checks)
 *   out        device [total_q][Hq][D]; lse device [total_q][Hq] or NULL
 * The new tokens' own K/V must already be in the pool, in blocks flagged
 * causal.  Every query row must see at least one key.  bf16 mode needs
 * head_dim 128, block_size 16, group size in {1, 2, 4, 8, 16}.
 */
LA_API la_status lazy_attn_prefill(const la_params* p, const void* q, const void* k_pool,
                            const void* v_pool, const uint64_t* blk_words,
                            const int32_t* req_blk_start, const int32_t* cu_q,
                            const int32_t* q_pos0, const float* cos_sin, int32_t batch,
                            int32_t max_q_per_req, void* out, float* lse, void* stream);

/*
 * Document-cache simulator (host only; the hit-ratio model of §2, Eqs. 1-3
 * and Table 1).  Replays n accesses (docs[i], pos[i]) -- document ids numbered
 * by popularity rank (0 = most popular), prompt positions in
 * [0, num_positions) -- against a cache of `capacity` entries and writes the
 * number of hits to *hits.
 *   policy    LA_CACHE_POSITION_AGNOSTIC: one entry per document (this
 *             library's pool); LA_CACHE_POSITION_AWARE: one entry per
 *             (document, position), as a position-encoded cache needs
 *   eviction  LA_EVICT_LRU: least recently used entry evicted on a miss;
 *             LA_EVICT_STATIC_TOP: the cache holds the most popular entries
 *             and never changes (documents < capacity, or all positions of
 *             documents < capacity / num_positions) -- Eqs. 1 and 2
 * docs/pos are host arrays; pos may be NULL for the agnostic policy.
 */
typedef enum la_cache_policy {
  LA_CACHE_POSITION_AGNOSTIC = 0,
  LA_CACHE_POSITION_AWARE = 1
} la_cache_policy;
typedef enum la_cache_eviction { LA_EVICT_LRU = 0, LA_EVICT_STATIC_TOP = 1 } la_cache_eviction;

LA_API la_status lazy_attn_cache_simulate(int64_t n, const int64_t* docs, const int32_t* pos,
                                          int32_t num_positions, int64_t capacity,
                                          int32_t policy, int32_t eviction, int64_t* hits);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* LAZY_ATTN_H */
