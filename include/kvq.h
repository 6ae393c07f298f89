/*
 * libkvq -- KIVI-style asymmetric-axis quantized KV cache for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no C++ types and no exceptions cross
 * this boundary.  Device pointers are caller-owned (allocated however the
 * caller likes, e.g. through torch); the library never allocates, frees or
 * synchronizes.  Every call validates all arguments before it enqueues any
 * work; on error it returns a status, enqueues nothing and leaves the
 * caller's kvq_state unchanged.  KVQ_EDEVICE reports a failed launch of the
 * call's own kernels: an entry point clears the calling thread's HIP
 * last-error slot (left over from earlier, unrelated HIP calls) before it
 * launches.  All device work is enqueued on the caller's
 * HIP stream (passed as an opaque hipStream_t, NULL = the null stream) and
 * is asynchronous.
 *
 * The method ("KV Cache Quantization Strategies", Steps 2-4):
 *   - Keys are quantized per channel: absmax over the token axis, one scale
 *     per channel per segment ([..., 1, head_dim]).
 *   - Values are quantized per token: absmax over head_dim, one scale per
 *     token ([..., tokens, 1]).
 *   - scale = qmax / max(absmax, eps) (an inverse step, computed in fp32,
 *     stored as fp16 clamped to 65504); code = clamp(round_half_even(
 *     fp32(x) * scale), -qmax, qmax); restore = code / max(scale, eps).
 *   - The newest tokens stay in a high-precision residual window of
 *     ``residual`` tokens; only tokens that overflow it are quantized, as new
 *     segments appended after the existing ones, which are never rewritten.
 *
 * Data layout in device memory (per (batch b, KV head h) "stream"; all
 * arrays are dense, row-major, in the order given):
 *   W = head_dim * code_bits / 8 bytes per token row; C = capacity.
 *   k_codes : uint8 [batch, kv_heads, C * W].  Token t, channel c: byte
 *             (t/64)*64*W + (r/16)*1024 + (t%64)*16 + r%16, r = c*bits/8,
 *             field at bit (c*bits)%8.
 *   v_codes : uint8 [batch, kv_heads, C * W].  Token t, channel c: byte
 *             (t/64)*64*W + c*8*bits + ((t%64)*bits)/8, field at bit
 *             ((t%64)*bits)%8.
 *             Fields are ``bits``-bit two's complement (int8 for bits = 8).
 *   k_scale : fp16 [batch, kv_heads, max_segments, head_dim], one row per
 *             segment.  With group G > 0 segment s holds tokens [sG, (s+1)G).
 *   v_scale : fp16 [batch, kv_heads, C], one per quantized token.
 *   Same-axis caches (scheme KVQ_SAME_AXIS) keep one scale per run of 64
 *   channels of every quantized token, for Keys and Values alike:
 *   k_scale and v_scale are fp16 [batch, kv_heads, C, head_dim / 64].
 *   k_tail, v_tail : kv_dtype [batch, kv_heads, ring, head_dim]; the tail
 *             token at absolute position p sits in slot p % ring, with
 *             ring = residual + group (group > 0) or residual (group == 0).
 *   seg_index : int32 [C]; with group == 0 the segment id of each quantized
 *             token (shared by all batch rows / heads); unused when group > 0.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,     /* bad argument, shape or configuration            */
  KVQ_ECAPACITY = 2,  /* append would exceed capacity or max_segments     */
  KVQ_EWORKSPACE = 3, /* workspace missing or smaller than required       */
  KVQ_EDEVICE = 4     /* a HIP launch or device query failed              */
} kvq_status;

typedef enum kvq_dtype {
  KVQ_BF16 = 0,  /* bfloat16 K/V/Q                                         */
  KVQ_F32 = 1    /* float32 K/V/Q (the exercise's teaching case)          */
} kvq_dtype;

/* Which axes the scales run along ("KV Cache Quantization Strategies",
 * Step 2 table).  KVQ_KIVI is the method: Keys per channel over a segment,
 * Values per token.  KVQ_SAME_AXIS is the table's fixed local group in the
 * setting of that page's section 5.1: Keys and Values both per token, one
 * scale per run of 64 consecutive channels; it exists to compare the two
 * and is supported by kvq_append, kvq_decode_attn(_noalloc) and
 * kvq_decode_step on uniform caches with head_dim 64 or 128 and group > 0
 * (every other entry point returns KVQ_EINVAL for it). */
typedef enum kvq_scheme {
  KVQ_KIVI = 0,
  KVQ_SAME_AXIS = 1
} kvq_scheme;

/* Decode kernel choice.  KVQ_KERNEL_AUTO runs the int8 matrix-core kernel
 * for the shapes it covers (bf16, int4 / int2 codes, head_dim 64 / 128,
 * group > 0, KIVI) and the vector-ALU kernel otherwise; KVQ_KERNEL_VALU runs
 * the vector-ALU kernel for every shape (same results within the attention
 * tolerance; for comparing the two). */
typedef enum kvq_decode_kernel {
  KVQ_KERNEL_AUTO = 0,
  KVQ_KERNEL_VALU = 1
} kvq_decode_kernel;

/* Static description of one cache (one layer).  Source: the exercise's
 * class constructor (qmax, eps) and ``append_and_partition``'s
 * residual_length; ``group`` and ``code_bits`` are the library's storage
 * choices (whole-group flushes; packed fields). */
typedef struct kvq_config {
  int32_t batch;        /* >= 1                                                   */
  int32_t kv_heads;     /* >= 1                                                   */
  int32_t head_dim;     /* 16, 32, 64 or 128; head_dim * code_bits % 128 == 0     */
  int32_t capacity;     /* max quantized tokens per sequence; multiple of 64      */
  int32_t code_bits;    /* 8, 4 or 2                                              */
  int32_t qmax;         /* 1 .. 2^(code_bits-1) - 1 (e.g. 127, 7, 1)              */
  int32_t residual;     /* residual window R > 0                                  */
  int32_t group;        /* G: 0 = one segment per flush (the exercise's rule),    */
                        /*    else a multiple of 64: flush whole groups of G      */
  int32_t max_segments; /* rows of k_scale; >= capacity / group when group > 0    */
  int32_t kv_dtype;     /* kvq_dtype of appended K/V, of the tail and of queries  */
  float eps;            /* range floor, 1e-8 in the exercise                      */
  int32_t scheme;       /* kvq_scheme (0 = KIVI)                                  */
  int32_t decode_kernel;/* kvq_decode_kernel (0 = automatic)                      */
} kvq_config;

/* Host-side token accounting, owned by the caller and updated by kvq_append
 * only when it returns KVQ_OK.  Mirrors the counters returned by the
 * exercise's ``append_and_partition``.  Zero-initialise for an empty cache. */
typedef struct kvq_state {
  int64_t quantized;    /* tokens in the quantized prefix                        */
  int64_t tail;         /* tokens in the high-precision tail                      */
  int64_t total;        /* quantized + tail                                       */
  int64_t flushed_last; /* tokens flushed by the most recent append               */
  int64_t segments;     /* quantized segments (rows of k_scale in use)            */
} kvq_state;

/* Caller-owned device buffers of one cache; sizes from kvq_buffer_sizes. */
typedef struct kvq_cache {
  void* k_codes;
  void* v_codes;
  void* k_scale;
  void* v_scale;
  void* k_tail;
  void* v_tail;
  void* seg_index;      /* may be NULL when group > 0                             */
} kvq_cache;

typedef struct kvq_sizes {
  size_t k_codes, v_codes, k_scale, v_scale, k_tail, v_tail, seg_index; /* bytes */
  int32_t ring;         /* tail ring slots                                        */
  int32_t row_bytes;    /* W                                                      */
} kvq_sizes;

/* Validate a configuration and report the byte size of every buffer.
 * Errors: KVQ_EINVAL for an unsupported configuration. */
kvq_status kvq_buffer_sizes(const kvq_config* cfg, kvq_sizes* out);

/* Pure host planning of one append (no device work): the state the cache
 * would have after appending n_new tokens.  Token accounting of the
 * exercise's Step 4 (TODO 3): overflow = max(tail + n_new - residual, 0);
 * flushed = overflow (group == 0) or (overflow / group) * group; quantized
 * += flushed; tail = tail + n_new - flushed; segments += 1 (group == 0,
 * flushed > 0) or flushed / group.
 * Errors: KVQ_EINVAL (n_new < 0, bad state), KVQ_ECAPACITY. */
kvq_status kvq_plan_append(const kvq_config* cfg, const kvq_state* st, int64_t n_new,
                           kvq_state* next);

/* Append n_new tokens (the exercise's ``append_and_partition``, and the
 * "encode, then cache.append" write of "KV Cache quantization and
 * compression", section 02).
 *   k_new, v_new : device, kv_dtype [batch, kv_heads, n_new, head_dim].
 * Tokens that overflow the residual window are quantized in place into the
 * next segment(s) (Keys per channel, Values per token; same-axis caches: both
 * per token in runs of 64 channels) straight from the old
 * tail and from k_new / v_new, with no concatenation; the tokens that remain
 * in the window are copied into the tail ring.  Earlier segments, their
 * scales and the surviving tail slots are never written.  n_new == 0 is a
 * valid no-op.  On KVQ_OK *st is advanced exactly as kvq_plan_append says.
 * Errors: KVQ_EINVAL, KVQ_ECAPACITY, KVQ_EDEVICE. */
kvq_status kvq_append(const kvq_config* cfg, kvq_state* st, const kvq_cache* cache,
                      const void* k_new, const void* v_new, int64_t n_new, void* stream);

/* Restore of the quantized prefix into dense arrays: for every quantized
 * token t and channel c, k = code / max(kscale[segment(t)][c], eps) and
 * v = code / max(vscale[t], eps) ("KV Cache Quantization Strategies",
 * Step 4 restore), computed as an IEEE fp32 division and stored as fp32 or
 * rounded once to bf16.  This is the first half of the "restore the whole
 * history to HBM, then ordinary attention" read path ("KV Cache
 * quantization and compression", section 06); the attention calls of this
 * library restore inside their kernels instead.
 *   k_out, v_out : device, out_dtype [batch, kv_heads, ld, head_dim]; rows
 *                  0 .. quantized - 1 of each (batch, head) are written
 *   out_dtype    : KVQ_F32 or KVQ_BF16
 *   ld           : rows per (batch, head) of the outputs, >= st->quantized
 * The tail is not touched (it is stored as given).  An empty prefix is a
 * valid no-op.  Errors: KVQ_EINVAL, KVQ_EDEVICE. */
kvq_status kvq_restore(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                       void* k_out, void* v_out, int32_t out_dtype, int64_t ld, void* stream);

/* Bytes of device workspace needed by kvq_decode_attn (tq = 1) or
 * kvq_block_attn (tq = query block length) for q_heads query heads.
 * Errors: KVQ_EINVAL. */
kvq_status kvq_workspace_size(const kvq_config* cfg, int32_t q_heads, int32_t tq,
                              size_t* bytes);

/* Prepare a freshly allocated workspace (clears its arrival counters with a
 * fill kernel; no memset node).  Call once per workspace before first use;
 * the attention kernels leave the counters cleared when they finish.
 * Errors: KVQ_EINVAL, KVQ_EDEVICE. */
kvq_status kvq_workspace_init(void* workspace, size_t bytes, void* stream);

/* Single-query grouped-query decode attention over the whole cache
 * ("KV Cache and autoregressive video generation", section 3.1, incremental
 * decode o_t = sum_j softmax_j(q_t k_j^T sigma) v_j; query head h reads KV
 * head h / (q_heads / kv_heads), section 04).  Keys and Values of the
 * quantized prefix are restored inside the kernel (read path "decode inside
 * the kernel", "KV Cache quantization and compression", section 06); the
 * tail is read as stored.  The sequence axis is split across workgroups and
 * the partial softmax states are merged (flash-decoding split, the former
 * page, section 05) by the last workgroup of each (batch, KV head) to
 * finish, in the same kernel; with more than 64 splits by a second, small
 * kernel.
 *   q   : device, kv_dtype [batch, q_heads, head_dim]
 *   out : device, float32 [batch, q_heads, head_dim]
 *   softmax_scale : sigma (1/sqrt(head_dim) for standard attention)
 *   num_splits : sequence splits per (batch, KV head); 0 = library's choice
 *   workspace : from kvq_workspace_size(cfg, q_heads, 1), initialised once
 * The cache must hold at least one token.  Calls that share a workspace
 * must be ordered (same stream).
 * Errors: KVQ_EINVAL, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                           const void* q, int32_t q_heads, float softmax_scale,
                           int32_t num_splits, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* kvq_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, computation and errors as kvq_decode_attn, without the
 * workspace: the split partials and arrival counters live in a device array
 * of 8 MiB inside the library, one per GPU, held until the process ends
 * (its address is looked up on the first call on each device).  Calls whose
 * partials need more than that -- batch * q_heads * splits * (head_dim + 4)
 * floats plus the counters -- return KVQ_EWORKSPACE.  The counters start at
 * zero and every call leaves them at zero.  All calls on one GPU share the
 * array: calls that overlap on one GPU (different streams, or threads) race
 * and must be ordered by the caller.  Nothing is allocated or freed.
 * Errors: KVQ_EINVAL, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_decode_attn_noalloc(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                   const void* q, int32_t q_heads, float softmax_scale,
                                   int32_t num_splits, float* out, void* stream);

/* One decode step: append n_new tokens, then attend with q over the whole
 * cache including them -- the per-step order encode, append, attend of
 * "KV Cache quantization and compression", section 02.  The result is that
 * of kvq_append(cfg, st, cache, k_new, v_new, n_new, stream) followed by
 * kvq_decode_attn(cfg, st, cache, q, ...): the same cache bytes and state,
 * and attention outputs equal within float rounding.  When the append
 * flushes nothing (1 <= n_new <= 16, kv_dtype bf16, a non-empty cache) the
 * step is one kernel launch: attention runs over the cache as it was, and
 * the workgroup that merges a (batch, KV head)'s splits adds the new tokens
 * as further softmax terms and writes them into their window slots
 * (cutting the per-step kernel launches, "KV Cache and autoregressive video
 * generation", section 05).  Otherwise it runs kvq_append, then
 * kvq_decode_attn.
 *   st           : host, advanced as kvq_plan_append says on KVQ_OK
 *   k_new, v_new : device, kv_dtype [batch, kv_heads, n_new, head_dim]
 *   q, out, softmax_scale, num_splits, workspace : as for kvq_decode_attn
 * Every precondition of both calls is checked before anything is enqueued;
 * on error *st is unchanged.
 * Errors: KVQ_EINVAL, KVQ_ECAPACITY, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_decode_step(const kvq_config* cfg, kvq_state* st, const kvq_cache* cache,
                           const void* k_new, const void* v_new, int64_t n_new,
                           const void* q, int32_t q_heads, float softmax_scale,
                           int32_t num_splits, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Attention of a block of tq new queries against the cache plus the
 * block's own keys/values (Attn = softmax(Q K^T sigma + M) V, "KV Cache and
 * autoregressive video generation", section 3.1).  Query i sits at absolute
 * position N + i after the N cached tokens: it sees all N cached tokens and
 * the block tokens j in frames no later than its own, i.e.
 * floor((N + j) / F) <= floor((N + i) / F) for frame_tokens = F --
 * bidirectional inside a frame, causal across frames (section 6.3);
 * F = 1 is the token-causal mask M_ij = -inf for j > i.  The block's own
 * K/V are read as given and are not appended.  Matrix products run on the
 * MFMA units over tiles restored into LDS.  Supported: kv_dtype bf16 and
 * head_dim 64 or 128 (other configurations return KVQ_EINVAL).
 *   q            : device, kv_dtype [batch, tq, q_heads, head_dim]
 *   k_blk, v_blk : device, kv_dtype [batch, tq, kv_heads, head_dim]
 *   frame_tokens : F >= 1 (N + tq + F below 2^31)
 *   out          : device, float32 [batch, tq, q_heads, head_dim]
 *   softmax_scale: sigma > 0 (1/sqrt(head_dim) for standard attention)
 *   num_splits   : splits of the cached sequence, at most 8; 0 = library's choice
 *   workspace    : from kvq_workspace_size(cfg, q_heads, tq), initialised once
 * Errors: KVQ_EINVAL, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_block_attn(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                          const void* q, const void* k_blk, const void* v_blk, int32_t tq,
                          int32_t q_heads, int32_t frame_tokens, float softmax_scale,
                          int32_t num_splits, float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- Paged caches: per-sequence lengths and a block table -----------------
 * The step after uniform lengths ("KV Cache quantization and compression",
 * section 02: appending also means maintaining valid lengths and paged
 * addresses; section 07: paging must cover the low-bit data and its
 * metadata together; "KV Cache and autoregressive video generation",
 * section 05: a block table maps each request's logical blocks to physical
 * blocks).  The quantized prefix of every sequence lives in pages of 64
 * tokens taken from one pool.  A page holds, for each KV head, in order:
 *   Key codes   64 * W bytes (the tile layout of the dense cache)
 *   Value codes 64 * W bytes
 *   Value scales 64 fp16 (one per token)
 *   Key scales   head_dim fp16 (the row of the segment the tile belongs to;
 *                every page of a segment holds the same row)
 * so kvq_paged_page_bytes = kv_heads * (128 * W + 128 + 2 * head_dim).
 * Logical tile j of sequence b (tokens 64 j .. 64 j + 63 of its prefix) is
 * page block_table[b * table_stride + j].  The bf16/fp32 window stays dense
 * per sequence: k_tail / v_tail as sized by kvq_buffer_sizes.  Every
 * sequence has its own kvq_state.  Supported: group > 0 (whole pages per
 * segment), batch <= 64; cfg->capacity is the per-sequence limit of the
 * prefix and must not exceed 64 * table_stride.
 * The caller owns the pool and the table (device memory) and maps the tiles
 * a call may write: those below ceil(quantized / 64) after it.  Page numbers
 * outside 0 .. n_pages - 1 are clamped (wrong results, no access outside
 * the pool). */
typedef struct kvq_paged_cache {
  void* pool;                 /* n_pages * kvq_paged_page_bytes bytes           */
  int64_t n_pages;
  const int32_t* block_table; /* device, int32 [batch, table_stride]             */
  int32_t table_stride;
  void* k_tail;               /* dense window, as in kvq_cache                   */
  void* v_tail;
} kvq_paged_cache;

/* Bytes of one page.  Errors: KVQ_EINVAL. */
kvq_status kvq_paged_page_bytes(const kvq_config* cfg, size_t* bytes);

/* Append n_new[b] tokens to sequence b (host array of batch counts, each
 * >= 0) with the same accounting as kvq_append, per sequence: each
 * sequence flushes its own overflow into its own pages.
 *   st           : host, kvq_state[batch], each advanced on KVQ_OK
 *   k_new, v_new : device, kv_dtype [batch, kv_heads, max_n, head_dim],
 *                  max_n = max(n_new); sequence b uses its first n_new[b] rows
 * Errors: KVQ_EINVAL, KVQ_ECAPACITY, KVQ_EDEVICE; on error no state changes. */
kvq_status kvq_paged_append(const kvq_config* cfg, kvq_state* st, const kvq_paged_cache* cache,
                            const void* k_new, const void* v_new, const int64_t* n_new,
                            void* stream);

/* Decode attention of every sequence over its own paged cache (the same
 * computation as kvq_decode_attn, with per-sequence lengths).  Every
 * sequence must hold at least one token.  Arguments as kvq_decode_attn; st
 * is kvq_state[batch]; the workspace is kvq_workspace_size(cfg, q_heads, 1).
 * Splits follow the work: a sequence takes splits in proportion to its
 * length; num_splits = 0 chooses the size of a split, num_splits > 0 is the
 * split count of the longest sequence.
 * Errors: KVQ_EINVAL, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_paged_decode_attn(const kvq_config* cfg, const kvq_state* st, const kvq_paged_cache* cache,
                                 const void* q, int32_t q_heads, float softmax_scale, int32_t num_splits,
                                 float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Block attention over paged caches (kvq_block_attn with per-sequence
 * lengths): every sequence b gets a block of tq queries at positions
 * N_b .. N_b + tq - 1 after its own N_b cached tokens, with the same
 * frame mask.  Arguments as kvq_block_attn; st is kvq_state[batch] and the
 * cache a kvq_paged_cache.  Every sequence uses the same split count (the
 * longest sets it).  Supported: kv_dtype bf16, head_dim 64 or 128,
 * group > 0, batch <= 64.
 * Errors: KVQ_EINVAL, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_paged_block_attn(const kvq_config* cfg, const kvq_state* st, const kvq_paged_cache* cache,
                                const void* q, const void* k_blk, const void* v_blk, int32_t tq,
                                int32_t q_heads, int32_t frame_tokens, float softmax_scale,
                                int32_t num_splits, float* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Restore of every sequence's quantized prefix from a paged cache
 * (kvq_restore for paged caches): sequence b's rows 0 .. quantized_b - 1 of
 * k_out / v_out [batch, kv_heads, ld, head_dim] are written, ld >= the
 * longest prefix; other rows are not touched.  group > 0, batch <= 64.
 * Errors: KVQ_EINVAL, KVQ_EDEVICE. */
kvq_status kvq_paged_restore(const kvq_config* cfg, const kvq_state* st, const kvq_paged_cache* cache,
                             void* k_out, void* v_out, int32_t out_dtype, int64_t ld, void* stream);

/* One decode step of every sequence of a paged cache: append n_new[b]
 * tokens to sequence b, then attend with q over each whole cache including
 * them (kvq_decode_step for paged caches).  The result is that of
 * kvq_paged_append followed by kvq_paged_decode_attn: the same pages,
 * windows and states, and outputs equal within float rounding.  When no
 * sequence flushes, every sequence already holds a token, each n_new[b] is
 * at most 16 (at least one above 0) and kv_dtype is bf16, the step runs
 * without the append's kernels: attention over the caches as they were,
 * and the merge adds each sequence's new tokens as further softmax terms
 * and writes them into its window.  Otherwise it runs the two calls.
 *   st, k_new, v_new, n_new : as for kvq_paged_append
 *   q, q_heads, softmax_scale, num_splits, out, workspace : as for
 *                 kvq_paged_decode_attn
 * Every precondition of both calls is checked before anything is enqueued;
 * on error no state changes.
 * Errors: KVQ_EINVAL, KVQ_ECAPACITY, KVQ_EWORKSPACE, KVQ_EDEVICE. */
kvq_status kvq_paged_decode_step(const kvq_config* cfg, kvq_state* st, const kvq_paged_cache* cache,
                                 const void* k_new, const void* v_new, const int64_t* n_new,
                                 const void* q, int32_t q_heads, float softmax_scale,
                                 int32_t num_splits, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Static string naming a status code. */
const char* kvq_status_str(kvq_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
