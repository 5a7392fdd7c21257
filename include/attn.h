/*
 * attn.h -- C ABI of the MI355X (gfx950) fused-attention library, libattn.so.
 *
 * What every call computes is scaled-dot-product attention,
 *
 *     O = softmax(scale * Q K^T) V,        lse_i = ln sum_j exp(scale * q_i . k_j),
 *
 * as defined in "FlashInfer kernel library: accelerating cascade-inference
 * attention with CUDA warp-level primitives" (zyxy.net/archives/24491),
 * section 1: similarity of Q and K, softmax into a probability distribution,
 * weighted sum with V.  The kernels compute it tile by tile with an online or
 * partial softmax so the score matrix never reaches device memory (the tiled
 * FlashAttention scheme in the xhh.club summary "fast attention kernels and
 * operator fusion", section "FlashAttention and paged attention").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them.  Scratch space (where needed)
 *    is passed in by the caller as `workspace`.
 *  - Alignment: q, k, v, o, the page pools and the workspace are accessed
 *    with 16-byte vector loads and stores and must be 16-byte aligned; lse,
 *    block tables, page lists, kv_lens and counters must be 4-byte aligned
 *    (hipMalloc and torch allocations are 256-byte aligned).  A misaligned
 *    pointer returns ATTN_E_ARG.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream).  Results are valid once the stream has
 *    synchronised.  Nothing is launched when a call returns an error.
 *  - Element types: ATTN_BF16 (bfloat16) or ATTN_F32 (IEEE float).  Scores,
 *    softmax statistics and accumulators are always fp32.  lse is always
 *    fp32, natural log of the scaled scores.
 *  - Dense layouts are row-major with the last dimension contiguous.
 *  - Grouped heads: query head h reads key/value head h / (heads_q / heads_kv)
 *    (heads_q must be a multiple of heads_kv).
 *  - Calls return an attn_status (0 = success).  No call prints, throws or
 *    aborts.  Device-side data (block tables, kv_lens) is NOT validated: the
 *    caller guarantees the preconditions stated per call.
 *  - Supported: head_dim 64 or 128; page_size 16; scale finite and > 0
 *    (ATTN_E_ARG otherwise).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_E_NULL = 1,        /* a required pointer is NULL                       */
    ATTN_E_SHAPE = 2,       /* a size is negative or sizes are inconsistent     */
    ATTN_E_UNSUPPORTED = 3, /* well-formed but not implemented (head_dim, ...)  */
    ATTN_E_WORKSPACE = 4,   /* workspace missing or smaller than required       */
    ATTN_E_HIP = 5,         /* the HIP runtime reported an error on launch      */
    ATTN_E_ARG = 6,         /* a value outside its domain (scale <= 0 or NaN,
                               a misaligned pointer)                            */
    ATTN_E_SCRATCH = 7      /* attn_decode_paged_noalloc: the call needs more
                               scratch than the library's fixed array holds     */
} attn_status;

/* ATTN_FP8_E4M3 names an FP8 KV cache (OCP E4M3 bytes); it is accepted only
 * by attn_decode_paged_fp8, whose queries and outputs are bf16 / fp32. */
typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1, ATTN_FP8_E4M3 = 2 } attn_dtype;

/* Text for a status code (static storage; never NULL). */
const char *attn_status_str(int status);

/*
 * attn_prefill -- fused multi-head attention over dense Q, K, V.
 *
 * The FMHA of "TensorRT-LLM deep optimization: FMHA kernels on Hopper"
 * (zyxy.net/?p=24414), section 2: score, softmax and weighted sum in one
 * kernel, K/V tiles staged on chip, numerically stable softmax.
 *
 *   q, o : [batch, heads_q,  seq_q,  head_dim]   element type `dtype`
 *   k, v : [batch, heads_kv, seq_kv, head_dim]   element type `dtype`
 *   lse  : [batch, heads_q, seq_q] fp32, or NULL to skip it
 *   causal != 0 masks key j for query i when j > i + (seq_kv - seq_q)
 *            (bottom-right aligned; the usual mask when seq_q == seq_kv).
 *            A query row with no visible key gets O = 0 and lse = -inf.
 *   scale : multiplies Q K^T (1/sqrt(head_dim) for standard attention).
 *
 * Any of batch, seq_q, seq_kv may be 0 (nothing to do, or O = 0 rows).
 * Errors: ATTN_E_NULL (q/k/v/o NULL with work to do), ATTN_E_SHAPE (negative
 * sizes, heads_q % heads_kv != 0), ATTN_E_UNSUPPORTED (head_dim not 64/128,
 * unknown dtype), ATTN_E_HIP.
 */
int attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse,
                 int batch, int heads_q, int heads_kv, int seq_q, int seq_kv,
                 int head_dim, int dtype, int causal, float scale, void *stream);

/*
 * attn_prefill_paged -- prefill of a chunk of new tokens against a paged KV
 * cache (chunked prefill).
 *
 * The tiled fused kernel of attn_prefill with its keys and values read
 * through a block table, the two used together as the xhh.club summary
 * ("fast attention kernels and operator fusion", section "FlashAttention and
 * paged attention") describes.  Sequence b holds kv_lens[b] tokens in the
 * cache, the chunk's own tokens included (their K/V are written before the
 * call); the seq_q queries of the chunk are its last seq_q positions, so
 * query i sits at position kv_lens[b] - seq_q + i.
 *
 *   q, o        : [batch, heads_q, seq_q, head_dim] bf16 (dtype ATTN_BF16)
 *   k_pages,
 *   v_pages     : [num_pages, heads_kv, page_size, head_dim] bf16
 *   block_table : int32 [batch, max_pages_per_seq] (device)
 *   kv_lens     : int32 [batch] (device)
 *   lse         : [batch, heads_q, seq_q] fp32, or NULL
 *   causal != 0 masks key j for query i when j > i + kv_lens[b] - seq_q;
 *            a query with no visible key (kv_lens[b] < seq_q) gets O = 0 and
 *            lse = -inf.
 *
 * Device-side preconditions (not checked): 0 <= kv_lens[b] <=
 * page_size * max_pages_per_seq; block_table[b][p] a valid page for
 * p < ceil(kv_lens[b] / page_size).  Entries past that are never read, and
 * slots past kv_lens[b] in the last page are never read.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_UNSUPPORTED (dtype other than
 * bf16, head_dim not 64/128, page_size != 16), ATTN_E_ARG (scale,
 * alignment), ATTN_E_HIP.
 */
int attn_prefill_paged(const void *q, const void *k_pages, const void *v_pages,
                       const int32_t *block_table, const int32_t *kv_lens, void *o, float *lse,
                       int batch, int heads_q, int heads_kv, int seq_q, int head_dim,
                       int page_size, int max_pages_per_seq, int dtype, int causal, float scale,
                       void *stream);

/*
 * Split-KV planning for paged decode.
 *
 * FlashDecoding splits the key/value length into independent partial
 * softmax results that are combined at the end (FlashDecoding++ summary,
 * wenjunhu.com/d/2311396.html, section 1); the chunk size is chosen from the
 * batch size and the KV length (the per-shape kernel choice of the
 * TensorRT-LLM FMHA page, section 3, and the heuristic dataflow of the
 * FlashDecoding++ summary, section 5).
 *
 * attn_decode_plan: host-only.  Given the shape, the host-side upper bound
 * max_kv_len and the compute-unit count (num_cus <= 0: the current
 * device's, 256 when no device can be queried),
 * returns in *split_tokens the chunk length (a multiple of 64, at most 1024)
 * and in *max_splits the number of chunks of the longest sequence.
 * requested_split > 0 forces that chunk length (rounded up to a multiple of
 * 64).  Returns ATTN_OK or ATTN_E_SHAPE.
 */
int attn_decode_plan(int batch, int heads_kv, int max_kv_len, int num_cus,
                     int requested_split, int *split_tokens, int *max_splits);

/*
 * Bytes of workspace attn_decode_paged needs for this shape (0 if none).
 * split_tokens: 0 = the planner's choice, else as for attn_decode_plan.
 */
size_t attn_decode_workspace_bytes(int batch, int heads_q, int heads_kv, int head_dim,
                                   int max_kv_len, int split_tokens);

/*
 * attn_decode_paged -- one query token per sequence over a paged KV cache.
 *
 * Paged attention as in the xhh.club summary ("how does paged attention
 * manage the KV cache"): the cache is cut into fixed-size blocks and a block
 * table maps each sequence's logical blocks to physical ones; the kernel
 * reads K and V through the table, so logical order is contiguous while the
 * physical placement is arbitrary.
 *
 *   q, o        : [batch, heads_q, head_dim]                   `dtype` / `o_dtype`
 *   k_pages,
 *   v_pages     : [num_pages, heads_kv, page_size, head_dim]   `dtype`
 *                 (each (page, kv head) tile is contiguous)
 *   block_table : int32 [batch, max_pages_per_seq]; token t of sequence b is
 *                 slot t % page_size of page block_table[b][t / page_size]
 *   kv_lens     : int32 [batch]; sequence b's query attends exactly its
 *                 kv_lens[b] cached tokens
 *   lse         : fp32 [batch, heads_q], or NULL
 *   max_kv_len  : host-side upper bound of kv_lens (plans the splits with no
 *                 device-to-host copy)
 *   workspace   : device memory of at least attn_decode_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0)
 *
 * Device-side preconditions (not checked): 0 <= kv_lens[b] <= max_kv_len
 * (a larger value is clamped to max_kv_len, a negative one counts as 0) and
 * the first ceil(kv_lens[b] / page_size) entries of row b are valid page
 * indices.
 * A sequence with kv_lens[b] == 0 gets O = 0 and lse = -inf.
 * Page slots past kv_lens[b] are never used, whatever they hold.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_UNSUPPORTED (page_size != 16,
 * head_dim, dtype, heads_q / heads_kv above 16 -- or, for fp32 caches, not
 * in {1,2,4,8}), ATTN_E_WORKSPACE, ATTN_E_HIP.
 */
int attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                      const int32_t *block_table, const int32_t *kv_lens,
                      void *o, float *lse,
                      int batch, int heads_q, int heads_kv, int head_dim,
                      int page_size, int max_pages_per_seq, int max_kv_len,
                      int dtype, int o_dtype, float scale,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Options of attn_decode_paged_ex (zero-initialise, then set what you need).
 *   split_tokens    : 0 = planner's choice; > 0 forces the chunk length.
 *   use_unified_max : 1 = asynchronous softmax with a unified max value
 *                     (FlashDecoding++ summary, wenjunhu.com/d/2311396.html,
 *                     sections 1 and 3): within every chunk each exponential
 *                     is taken against the fixed scalar phi instead of a
 *                     running maximum, so partial sums need no rescaling and
 *                     no exchange of maxima.  A (query row, chunk) pair whose
 *                     largest scaled score s = scale * q.k leaves the window
 *                     phi - 60 <= max s <= phi + 60 (outside it exp(s - phi)
 *                     could overflow an fp32 sum or the largest term
 *                     underflow) falls back: its chunk is recomputed with the
 *                     exact online softmax.  Results equal the plain path's
 *                     within the same tolerance.  bf16 caches (and FP8
 *                     caches through attn_decode_paged_fp8, where s is
 *                     scale * q.(k_scale * e4m3)) with heads_q / heads_kv
 *                     <= 16 only (else ATTN_E_UNSUPPORTED).
 *   phi             : the unified max, in units of scaled scores (finite,
 *                     else ATTN_E_ARG); 0 suits scores of order one.
 *   fallback_count  : device int, or NULL.  The number of (query row, chunk)
 *                     pairs that fell back is added to it (atomically; the
 *                     caller zeroes it); a sequence shorter than one chunk is
 *                     one chunk.
 */
typedef struct {
    int split_tokens;
    int use_unified_max;
    float phi;
    int reserved0;
    int *fallback_count;
    int reserved[4];
} attn_decode_opts;

/* attn_decode_paged with options (opts may be NULL = defaults). */
int attn_decode_paged_ex(const void *q, const void *k_pages, const void *v_pages,
                         const int32_t *block_table, const int32_t *kv_lens,
                         void *o, float *lse,
                         int batch, int heads_q, int heads_kv, int head_dim,
                         int page_size, int max_pages_per_seq, int max_kv_len,
                         int dtype, int o_dtype, float scale,
                         void *workspace, size_t workspace_bytes, void *stream,
                         const attn_decode_opts *opts);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, types, layouts,
 * preconditions and results, minus the workspace.  The split partials go to
 * a file-scope device array of the library, ATTN_NOALLOC_SCRATCH_BYTES
 * (32 MiB) per GPU, held from the call that first needs it on a GPU until
 * the process ends; the call itself allocates nothing.  The planner's split
 * is used (as attn_decode_paged).  A shape whose partials exceed the array
 * (attn_decode_workspace_bytes(...) > ATTN_NOALLOC_SCRATCH_BYTES) returns
 * ATTN_E_SCRATCH and launches nothing.  Every call on one GPU shares that
 * GPU's array: calls that can overlap on one GPU (different streams, or
 * several host threads) race and must be serialised by the caller.  The
 * current device must be the stream's device.
 * Errors: those of attn_decode_paged, ATTN_E_SCRATCH; ATTN_E_HIP also when
 * the array's device address cannot be obtained.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_paged_noalloc(const void *q, const void *k_pages, const void *v_pages,
                              const int32_t *block_table, const int32_t *kv_lens,
                              void *o, float *lse,
                              int batch, int heads_q, int heads_kv, int head_dim,
                              int page_size, int max_pages_per_seq, int max_kv_len,
                              int dtype, int o_dtype, float scale, void *stream);

/*
 * attn_decode_paged_fp8 -- attn_decode_paged over an FP8 KV cache.
 *
 * Quantised KV caches are the inference optimisation the TensorRT-LLM FMHA
 * page (zyxy.net/?p=24414) lists in sections 3, 4 and 7; decode is bound by
 * reading the cache, so one byte per element halves the traffic.  The cache
 * holds OCP FP8 E4M3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite value 448) with one scale per tensor:
 *     key element = k_scale * e4m3(byte),  value element = v_scale * e4m3(byte),
 * and the result is attention over those values, exactly as
 * attn_decode_paged computes it (the bytes are widened in registers; every
 * E4M3 value is a bf16 value, so nothing is rounded on the way).
 *
 *   q, o        : [batch, heads_q, head_dim], q bf16, o `o_dtype`
 *                 (ATTN_BF16 or ATTN_F32)
 *   k_pages,
 *   v_pages     : uint8 [num_pages, heads_kv, page_size, head_dim], E4M3
 *   k_scale,
 *   v_scale     : the per-tensor scales (finite and > 0, else ATTN_E_ARG)
 *   opts        : as for attn_decode_paged_ex (may be NULL): split_tokens,
 *                 use_unified_max, phi and fallback_count
 *   everything else, the workspace size (attn_decode_workspace_bytes), the
 *   preconditions and the errors: as attn_decode_paged.  heads_q / heads_kv
 *   <= 16; chunks of at most 1024 tokens.
 */
int attn_decode_paged_fp8(const void *q, const void *k_pages, const void *v_pages,
                          float k_scale, float v_scale,
                          const int32_t *block_table, const int32_t *kv_lens,
                          void *o, float *lse,
                          int batch, int heads_q, int heads_kv, int head_dim,
                          int page_size, int max_pages_per_seq, int max_kv_len,
                          int o_dtype, float scale,
                          void *workspace, size_t workspace_bytes, void *stream,
                          const attn_decode_opts *opts);

/*
 * attn_merge_states -- combine two partial attention states in place.
 *
 * (o_a, lse_a) and (o_b, lse_b) are attention results of the same query
 * rows over two disjoint key sets; the result, written into (o_a, lse_a), is
 * the attention over their union:
 *     M = max(lse_a, lse_b),  w_x = exp(lse_x - M),
 *     lse = M + ln(w_a + w_b),  o = (w_a o_a + w_b o_b) / (w_a + w_b).
 * A side with lse = -inf is empty and contributes nothing (its o is ignored);
 * two empty sides give o = 0, lse = -inf.  This is the "update all partial
 * softmax results together at the end" step of FlashDecoding (FlashDecoding++
 * summary, section 1) and the combining stage of cascade inference
 * ("FlashInfer kernel library ...", section 4).
 *
 *   o_a, o_b   : [rows, head_dim], element type o_dtype (o_a is overwritten)
 *   lse_a, lse_b : fp32 [rows] (lse_a is overwritten)
 * o_b/lse_b may alias o_a/lse_a exactly (giving o, lse + ln 2).
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_UNSUPPORTED, ATTN_E_HIP.
 */
int attn_merge_states(void *o_a, float *lse_a, const void *o_b, const float *lse_b,
                      int rows, int head_dim, int o_dtype, void *stream);

/*
 * attn_decode_shared_prefix -- stage one of shared-prefix cascade decode.
 *
 * All `batch` requests attend the same prefix of prefix_len tokens, stored
 * once in the paged cache (prefix sharing of KV blocks, xhh.club summary,
 * "paged attention"; the staged cascade of "FlashInfer kernel library ...",
 * sections 2 and 4).  Each prefix page is read once per kv head for all
 * requests.  Combine the result with each request's own suffix attention
 * (attn_decode_paged over the suffix tables) using attn_merge_states.
 *
 *   q, o         : [batch, heads_q, head_dim]                 `dtype` / `o_dtype`
 *   k_pages,
 *   v_pages      : [num_pages, heads_kv, page_size, head_dim]  `dtype`
 *   prefix_pages : int32 [ceil(prefix_len / page_size)] physical pages
 *   lse          : fp32 [batch, heads_q], or NULL
 *   workspace    : at least attn_shared_prefix_workspace_bytes(...) bytes
 * prefix_len == 0 gives O = 0 and lse = -inf.  bf16 runs the MFMA prefix
 * kernel; fp32 (the exactness test mode) runs the paged decode kernel with
 * the one prefix table shared by every request.
 * attn_shared_prefix_workspace_bytes takes dtype ATTN_FP8_E4M3 for the
 * workspace of attn_decode_shared_prefix_fp8.
 */
size_t attn_shared_prefix_workspace_bytes(int batch, int heads_q, int heads_kv, int head_dim,
                                          int prefix_len, int dtype);
int attn_decode_shared_prefix(const void *q, const void *k_pages, const void *v_pages,
                              const int32_t *prefix_pages, int prefix_len,
                              void *o, float *lse,
                              int batch, int heads_q, int heads_kv, int head_dim,
                              int page_size, int dtype, int o_dtype, float scale,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_shared_prefix_fp8 -- attn_decode_shared_prefix over an FP8 KV
 * cache (OCP E4M3 bytes with per-tensor scales, as attn_decode_paged_fp8):
 * q bf16, o `o_dtype` (ATTN_BF16 or ATTN_F32), k_pages / v_pages uint8
 * [num_pages, heads_kv, page_size, head_dim], cached values k_scale * e4m3
 * and v_scale * e4m3 (finite and > 0, else ATTN_E_ARG).  The workspace is
 * attn_shared_prefix_workspace_bytes(..., ATTN_FP8_E4M3).  The suffix stage
 * is attn_decode_paged_fp8; the merge is attn_merge_states.  Errors as
 * attn_decode_shared_prefix.
 */
int attn_decode_shared_prefix_fp8(const void *q, const void *k_pages, const void *v_pages,
                                  float k_scale, float v_scale,
                                  const int32_t *prefix_pages, int prefix_len,
                                  void *o, float *lse,
                                  int batch, int heads_q, int heads_kv, int head_dim,
                                  int page_size, int o_dtype, float scale,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_cascade -- shared-prefix cascade decode in one call.  Every
 * request attends the prefix all requests share (prefix_len tokens through
 * prefix_pages, as attn_decode_shared_prefix) and then its own tokens
 * (suffix_lens[b] through row b of suffix_table, as attn_decode_paged); the
 * result is attention over the prefix and the request's own tokens together,
 * the cascade's two stages merged by their log-sum-exp ("FlashInfer kernel
 * library ...", sections 2 and 4).  Three launches: the prefix stage of
 * attn_decode_shared_prefix (each prefix page read once per kv head for all
 * requests) writes its chunk states into the first slots of every row of the
 * workspace, the paged decode of the requests' own tokens writes its chunk
 * states after them, and one combine merges each row's slots.  The result
 * equals attn_decode_shared_prefix + attn_decode_paged + attn_merge_states
 * up to the order of the sums, without the prefix chunk combine and the
 * merge as launches of their own.
 *
 *   q, o         : [batch, heads_q, head_dim]                 bf16 / `o_dtype`
 *   k_pages,
 *   v_pages      : [num_pages, heads_kv, page_size, head_dim]  bf16 (dtype
 *                  ATTN_BF16) or OCP E4M3 bytes (ATTN_FP8_E4M3: values
 *                  k_scale * e4m3 and v_scale * e4m3, finite and > 0; the
 *                  scales are ignored for bf16)
 *   prefix_pages : int32 [ceil(prefix_len / page_size)]
 *   suffix_table : int32 [batch, max_pages_per_seq]
 *   suffix_lens  : int32 [batch], clamped to [0, max_suffix_len], or NULL
 *                  (every request has max_suffix_len own tokens)
 *   lse          : fp32 [batch, heads_q], natural log, or NULL
 *   workspace    : attn_cascade_workspace_bytes(...) bytes, 16-byte aligned
 *                  (NULL when that is 0)
 * heads_q / heads_kv <= 16, head_dim 64 or 128, page_size 16.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE (negative sizes, heads_q % heads_kv,
 * max_pages_per_seq * page_size < max_suffix_len), ATTN_E_UNSUPPORTED (dtype
 * other than ATTN_BF16 / ATTN_FP8_E4M3, head_dim, page_size, more than 16
 * query heads per kv head), ATTN_E_ARG (scales, alignment), ATTN_E_WORKSPACE,
 * ATTN_E_HIP.
 */
size_t attn_cascade_workspace_bytes(int batch, int heads_q, int heads_kv, int head_dim,
                                    int prefix_len, int max_suffix_len, int dtype);
int attn_decode_cascade(const void *q, const void *k_pages, const void *v_pages,
                        const int32_t *prefix_pages, int prefix_len,
                        const int32_t *suffix_table, const int32_t *suffix_lens,
                        void *o, float *lse,
                        int batch, int heads_q, int heads_kv, int head_dim,
                        int page_size, int max_pages_per_seq, int max_suffix_len,
                        int dtype, int o_dtype, float scale, float k_scale, float v_scale,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Flat GEMM of the decode phase: C = A W^T.
 *
 * In decode the projections around attention (K/Q/V, O, the two FFN layers)
 * multiply the m tokens of one step (m = batch size, small) by a weight of n
 * rows and k columns: a "flat" GEMM whose cost is reading the weight once.
 * The FlashDecoding++ summary (wenjunhu.com/d/2311396.html, sections 1 and 4)
 * pads such an m only to the matrix unit's smallest tile instead of 64 and
 * hides memory latency with double buffering; its section 5 picks the kernel
 * from m, n and k (writing each projection's weight as n x k).  Here m is
 * padded to 16 on the bf16 matrix core and a larger m (prefill) is left to a
 * conventional GEMM library.
 *
 *   a : [m, k] bf16 (dtype ATTN_BF16), row-major
 *   w : [n, k] bf16, row-major (a linear layer's weight: C[i][j] = a_i . w_j)
 *   c : [m, n] `c_dtype` (ATTN_BF16, rounded to nearest even, or ATTN_F32)
 *   workspace : at least attn_flat_gemm_workspace_bytes(m, n, k, opts)
 *               bytes (NULL allowed when that is 0): fp32 partials of the
 *               k slices, added in slice order, so results do not depend on
 *               the timing of the launch
 *   opts : NULL = the planner's choices, or an attn_flat_gemm_opts
 * Products are accumulated in fp32.  m, n or k may be 0 (k == 0 gives C = 0).
 * Alignment: a, w and the workspace 16 bytes, c 4 bytes.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE (negative sizes or options),
 * ATTN_E_UNSUPPORTED (m > 64, k not a multiple of 8 or above 2^22, dtype
 * other than bf16, c_dtype other than bf16 / fp32, rows_per_workgroup other
 * than 0, 16, 32, 64, 128, 256, waves_per_workgroup other than 0, 4, 8,
 * kernel above 2, and options that fit neither kernel: the LDS-tiled one
 * forced with k > 2^20, rows below 64 or 8 wavefronts, the
 * register-streaming one forced with rows above 64),
 * ATTN_E_WORKSPACE,
 * ATTN_E_ARG (alignment), ATTN_E_HIP.
 *
 * Two kernels.  Register-streaming: operands go from HBM straight into
 * registers, 16, 32 or 64 rows of w per workgroup.  LDS-tiled (k <= 2^20):
 * a workgroup owns 64, 128 or 256 rows of w and stages 64-wide k chunks of
 * w and A in LDS, so one A tile serves all its rows.  The planner takes the
 * LDS-tiled kernel for m > 16, and for m >= 8 on weights of more than 2^24
 * elements.
 *
 * attn_flat_gemm_plan: host-only.  The planner's choice for this shape on
 * num_cus compute units (<= 0: the current device's, else 256): the kernel
 * (*kernel = 1 register-streaming, 2 LDS-tiled; kernel may be NULL), rows
 * of w per workgroup and k slices across workgroups.  Register-streaming:
 * 16 rows for m <= 8, and for m <= 16 on weights of at most 2^24 elements;
 * 32 for m <= 32 on weights with at least 1.25 blocks of 64 rows per CU;
 * else 64, so that one A fragment serves four row blocks; at most 4 slices,
 * and only when the row blocks alone leave compute units idle or unevenly
 * loaded.  LDS-tiled: 64 rows (128 when n >= 16384), slices doubled until
 * the grid holds two workgroups per CU, each slice at least 4 chunks.
 * Workgroups are 4 wavefronts.  Fields of opts that are > 0 override the
 * choice; splits is clamped to the number of 32-wide k steps
 * (register-streaming) or 64-wide chunks (LDS-tiled).
 * attn_flat_gemm_workspace_bytes returns 0 for an unsupported shape.
 */
typedef struct {
    int splits;               /* 0 = planner; > 0 forces that many k slices       */
    int rows_per_workgroup;   /* 0 = planner; 16, 32, 64 (register-streaming) or
                                 64, 128, 256 (LDS-tiled) forces it               */
    int waves_per_workgroup;  /* 0 = planner; 4 or 8 forces it (8: register-
                                 streaming kernel only)                           */
    int kernel;               /* 0 = planner; 1 register-streaming, 2 LDS-tiled   */
    int reserved[4];
} attn_flat_gemm_opts;

int attn_flat_gemm_plan(int m, int n, int k, int num_cus, const attn_flat_gemm_opts *opts,
                        int *splits, int *rows_per_workgroup, int *kernel);
size_t attn_flat_gemm_workspace_bytes(int m, int n, int k, const attn_flat_gemm_opts *opts);
int attn_flat_gemm(const void *a, const void *w, void *c, int m, int n, int k, int dtype,
                   int c_dtype, void *workspace, size_t workspace_bytes, void *stream,
                   const attn_flat_gemm_opts *opts);

/*
 * Checked build.  libattn_checked.so is built from the same sources with
 * ATTN_CHECKED=1 and exports this same interface.  Its kernels also check the
 * indices they read from device memory, which the release build takes on
 * trust (a block table maps a sequence's logical pages to scattered physical
 * ones: xhh.club summary, "how does paged attention manage the KV cache"):
 *   - a length (kv_lens[b], or a paged prefill's kv_lens[b]) outside
 *     [0, its host bound] sets ATTN_DEV_ERR_KV_LEN and is clamped as in the
 *     release build;
 *   - a page index (block-table or prefix-page entry) outside
 *     [0, num_pages) sets ATTN_DEV_ERR_PAGE and page 0 is read instead, so
 *     a bad table cannot make a kernel read outside the pool.  num_pages is
 *     the number of whole pages from k_pages (and from v_pages) to the end
 *     of the device allocation that holds it, attn_device_pool_pages below;
 *     it is INT_MAX, and only negative indices are caught, when the runtime
 *     knows no allocation at that pointer.
 * The results of a call with valid data equal the release build's bit for
 * bit.  The checks cost a little time; the release build has none of them.
 *
 * attn_checked_build: 1 in the checked library, 0 in the release one.
 * attn_device_errors: waits for the current device (hipDeviceSynchronize),
 *   stores its error word (an OR of ATTN_DEV_ERR_* bits since it was last
 *   cleared) in *flags and clears it when `clear` is nonzero.  Not
 *   capturable.  The word is shared by every call on that device.  Errors:
 *   ATTN_E_UNSUPPORTED in the release library, ATTN_E_NULL, ATTN_E_HIP.
 * attn_device_pool_pages: the page bound above, for `pages` and pages of
 *   page_bytes bytes, in *num_pages (host-only query, both builds).
 */
#define ATTN_DEV_ERR_KV_LEN 1u
#define ATTN_DEV_ERR_PAGE 2u
int attn_checked_build(void);
int attn_device_errors(unsigned int *flags, int clear);
int attn_device_pool_pages(const void *pages, size_t page_bytes, int *num_pages);

/*
 * attn_probe_hbm_read -- measurement aid, not part of the attention path: a
 * kernel that only reads, used to measure the HBM read rate that plain
 * 16-byte vector loads reach on this GPU, the practical ceiling of the
 * memory-bound paths above (decode, cascade, flat GEMM; "FlashInfer kernel
 * library", section 7: profile to find the memory bottleneck).
 *
 *   buf      : device, n_blocks * attn_probe_block_bytes() bytes (4096),
 *              16-byte aligned, read only
 *   order    : device int32 [n_blocks] or NULL; block i of the walk is the
 *              one at byte order[i] * 4096 (entries outside [0, n_blocks)
 *              are clamped into it), NULL reads the blocks in place order
 *   sink     : device, one uint32; written only when the XOR of all words
 *              read equals one fixed value, so the loads cannot be elided
 * Launches one kernel on `stream`; time it with events around the call.
 * Errors: ATTN_E_SHAPE (n_blocks < 0), ATTN_E_NULL, ATTN_E_ARG (alignment),
 * ATTN_E_HIP.
 */
int attn_probe_block_bytes(void);
int attn_probe_hbm_read(const void *buf, const int32_t *order, int n_blocks, uint32_t *sink,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
