/*
 * csa2.h - C ABI of libcsa2.so, the MI355X (gfx950) CSA2 FP4 sparse-attention
 * decode step.
 *
 * The method: DeepSeek-V4.1-Flash's Compressed Sparse Attention 2 (CSA2).
 * Each decode query runs, per layer, one of three statically assigned modes:
 *   Full    - the layer's indexer scores every compressed KV entry, Top-K
 *             picks the entries, sparse attention runs over them;
 *   Reindex - the layer reuses an earlier layer's KV cache but re-scores with
 *             its own indexer query, only inside the candidate pool (at most
 *             2048 blocks x 8 positions) an earlier Full layer chose;
 *   Reuse   - the layer reuses KV and the Top-K list; attention only.
 * The main KV cache is FP4: E2M1 values with one E4M3 scale per 16 channels,
 * no second-level global scale, quantised after RoPE.
 *
 * Page keys used in the citations below:
 *  [P1] "DeepSeek-V4.1-Flash：把 KV Cache 压缩到极限的百万上下文 MoE（技术报告全系统解读）"
 *       (ai-engineering-6yk.pages.dev, ch01/059)
 *  [P3] "552B参数干掉1.6T：DeepSeek V4.1 Flash技术深度解析" (55zb.com)
 *  [P4] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression" (agihunt.info)
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; tensors are
 *    dense row-major with the shapes given (the FP4 cache alone takes row
 *    strides); every tensor pointer must be 16-byte aligned unless stated.
 *    bf16 values are passed as raw uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on that stream and returns; nothing synchronises.
 *  - Arguments are validated on the host before anything is launched; a
 *    non-zero csa2_status is returned and nothing is enqueued.  Values that
 *    live in device memory (n_valid, indices, pool ids) cannot be checked on
 *    the host: out-of-range values there have the defined behaviour stated
 *    per function (masking / clamping), never an out-of-bounds access.
 *  - The library allocates no device memory and keeps no mutable global
 *    state; calls on different streams may run concurrently.  Where a kernel
 *    needs scratch space the caller passes a workspace whose size comes from
 *    the matching *_workspace_bytes() query.
 *  - Each kernel launch holds fewer than 2^32 work-items (workgroups x
 *    threads).  A call whose sizes would need a larger launch (e.g. an index
 *    call with B * N_cap >= 2^30, a Top-K with B * ceil(M / 16384) >= 2^22
 *    rows x chunks, an attention call with about 2^22 queries at 64 heads, or
 *    a K so large that its slices alone pass the limit) returns
 *    CSA2_ERR_RANGE before anything is enqueued.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* csa2_stream_t; /* a hipStream_t */

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,        /* a required pointer is NULL */
  CSA2_ERR_SHAPE = 2,       /* a size is negative or inconsistent */
  CSA2_ERR_ALIGN = 3,       /* a pointer or stride breaks its alignment rule */
  CSA2_ERR_RANGE = 4,       /* append past capacity, K out of [1, 2048], ... */
  CSA2_ERR_UNSUPPORTED = 5, /* dimensions without a compiled kernel */
  CSA2_ERR_HIP = 6,         /* the HIP runtime refused a launch */
  CSA2_ERR_WORKSPACE = 7    /* workspace NULL or smaller than required */
} csa2_status;

/* Static text for a status code (never NULL). */
const char* csa2_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int csa2_version(void);

/*
 * a0. FP4 quantise + append (the main-KV write).
 * Defined by [P1] section 效率组件四件, item 4 (E2M1 values, one E4M3 scale per
 * 16 channels, no global scale, quantised after RoPE) and [P4] CSA2 paragraph.
 *
 * x        bf16 [n_rows, d_c]   post-RoPE latent rows (RoPE is applied by the
 *                               caller; this call does not rotate)
 * rope_src bf16 [n_rows, d_r]   RoPE part, copied unchanged (NULL iff d_r == 0)
 * codes    u8   cache rows of d_c/2 bytes: byte j = channel 2j (low nibble) |
 *                 channel 2j+1 (high nibble); row r at codes + r * codes_stride
 * scales   u8   cache rows of d_c/16 E4M3 bytes (byte g scales channels
 *                 [16g, 16g+16)); row r at scales + r * scales_stride
 * rope_dst bf16 cache rows of d_r values; row r at rope_dst + r * rope_stride
 *                 bytes (NULL iff d_r == 0)
 * Strides are in bytes; 0 means dense rows.  The three regions may be three
 * arrays or share one buffer of fixed-size entry records (the layout the
 * attention gather reads fastest: one contiguous record per entry, e.g.
 * 512 bytes = codes at 0, scales at d_c/2, RoPE at d_c/2 + d_c/16).
 * Rows [dst_row0, dst_row0 + n_rows) are written.
 *
 * Per group of 16 channels: scale = the E4M3 value nearest to max|x| / 6
 * (ties to the even code, saturating at 448 = 0x7E); each element's code is
 * the input's sign bit plus the E2M1 magnitude nearest to |x| / scale (ties
 * to the even code, saturating at 6); a zero scale gives magnitude 0.
 * Bit-exact with the oracle for all finite inputs; codes for non-finite
 * inputs are unspecified (but written, in bounds).
 * Requires d_c % 32 == 0, 32 <= d_c <= 4096, d_r % 8 == 0, d_r <= 1024,
 * n_rows >= 0, 0 <= dst_row0, dst_row0 + n_rows <= capacity, x / codes /
 * rope pointers and codes / rope strides multiples of 16, scales pointer and
 * stride even, each stride at least its row width.
 */
int csa2_quantize_fp4(const uint16_t* x, int64_t n_rows, int32_t d_c,
                      const uint16_t* rope_src, int32_t d_r,
                      uint8_t* codes, int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                      uint16_t* rope_dst, int64_t rope_stride,
                      int64_t dst_row0, int64_t capacity, csa2_stream_t stream);

/*
 * a1. Indexer scores, Full mode: every entry of the cache is scored.
 * Defined by [P1] 架构三件套, CSA2 (Full mode runs the whole pipeline) and
 * [P4] CSA2 paragraph (Full produces its own KV and Top-K).  The pages give
 * no formula; the reading implemented is
 *   score[b, n] = sum_h w[b, h] * max(0, q_idx[b, h, :] . k_idx[b, n, :])
 * (ReLU-gated indexer heads, one key per entry shared by all heads): bf16
 * products accumulated in fp32 by the matrix cores, then the weighted head
 * terms summed in fp32 (heads 4j..4j+3 in order, then the four partial sums
 * pairwise).
 *
 * q_idx   bf16 [B, H_I, D_I]
 * w       f32  [B, H_I]  per-head weights, or NULL for all ones
 * k_idx   bf16 [B, N_cap, D_I]  indexer key cache
 * n_valid i32  [B]  valid entries per sequence, or NULL for N_cap; values are
 *                   clamped to [0, N_cap] on the device
 * scores  f32  [B, N_cap]  out; entries n >= n_valid[b] get -inf (not read)
 * Integer-valued inputs with |sums| < 2^24 give exact scores.
 * Requires 1 <= H_I <= 16, D_I in {32, 64, 128, 256}, B >= 0, N_cap >= 0.
 */
int csa2_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                    const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I,
                    int64_t N_cap, float* scores, csa2_stream_t stream);

/*
 * a2. Indexer scores, Reindex mode: only the candidate pool is scored.
 * Defined by [P1] section Hierarchical Sparse Indexer (an earlier Full layer
 * builds a block-level candidate pool of at most 2048 blocks x 8 positions;
 * later Reindex layers score only inside it, so the cost stops growing with
 * the context) and [P4] CSA2 paragraph.
 *
 * pool_blocks i32 [B, P_max]  block ids; block id p covers entries
 *                             [block*p, block*p + block)
 * n_blocks    i32 [B]         used pool slots per sequence (clamped to [0, P_max])
 * scores      f32 [B, P_max*block]  out: slot i*block + j scores entry
 *                                   block*pool_blocks[b,i] + j
 * positions   i32 [B, P_max*block]  out: that entry's global position
 * A slot is empty (score -inf, position -1, key not read) when i >=
 * n_blocks[b], the block id is negative, or the position is >= n_valid[b].
 * Other arguments as csa2_index_full.  Requires 1 <= block <= 64,
 * 1 <= P_max, P_max * block <= 2^24.
 */
int csa2_index_pool(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                    const int32_t* n_valid, const int32_t* pool_blocks,
                    const int32_t* n_blocks, int32_t B, int32_t H_I, int32_t D_I,
                    int64_t N_cap, int32_t P_max, int32_t block, float* scores,
                    int32_t* positions, csa2_stream_t stream);

/*
 * a3. Top-K selection with the lower id winning ties.
 * Top-512 per [P1] 架构三件套, CSA2; the tie rule (lower index wins) is a
 * fixed parameter of this library; ids are global entry positions.
 *
 * scores    f32 [B, M]
 * ids       i32 [B, M]  candidate ids, or NULL for the column index; id -1
 *                       marks an empty candidate (never chosen)
 * n_valid   i32 [B]     only columns c < n_valid[b] are candidates (NULL = M;
 *                       clamped to [0, M] on the device)
 * out_idx   i32 [B, K]  out: ids of the min(K, #candidates) best candidates
 *                       in order (score descending, id ascending), then -1
 * out_score f32 [B, K]  out (nullable): their scores, then -inf
 * -0.0 ranks equal to +0.0 and is reported as +0.0; NaN ranks below every
 * other score and is reported as a quiet NaN.  Ids must be >= 0 (other than
 * -1); equal (score, id) pairs are interchangeable.  Bit-exact.
 * Rows of up to 16384 columns are selected by one workgroup each.  Longer
 * rows take one of two routes with the same result:
 *   chunked reduction: each 16384-column chunk keeps its K best keys, and the
 *     winners are reduced again until one chunk remains (the workspace holds
 *     the levels' winners: B * ch_l * K * 8 bytes for each level l but the
 *     last, ch_0 = ceil(M / 16384), ch_l+1 = ceil(ch_l * K / 16384));
 *   threshold filter, for K >= 64 on rows of at most 2^20 columns whose
 *     first level would take more than 768 chunks in all (B * ch_0 > 768) or
 *     whose reduction takes more than two levels: a 16384-column sample of each
 *     row gives a score threshold, one pass keeps the candidates at or above
 *     it, and one workgroup per row selects among them (the workspace holds
 *     128 bytes and 16384 keys of 8 bytes per row).  A row whose kept
 *     candidates cannot hold its Top-K (too many, or fewer than K above a
 *     non-zero threshold) is reduced by its workgroup over the whole row.
 * Requires 1 <= K <= 2048, 1 <= M < 2^31, B >= 0, and a workspace of at
 * least csa2_topk_workspace_bytes(B, M, K) bytes (may be 0 / NULL then),
 * 16-byte aligned, caller-owned, contents not preserved.
 */
size_t csa2_topk_workspace_bytes(int32_t B, int64_t M, int32_t K);
int csa2_topk(const float* scores, const int32_t* ids, const int32_t* n_valid,
              int32_t B, int64_t M, int32_t K, int32_t* out_idx, float* out_score,
              void* workspace, size_t workspace_bytes, csa2_stream_t stream);

/*
 * a1 + a3 in one call, Full mode: the indexer scores of every entry and their
 * Top-K ([P1] 架构三件套, CSA2: a Full layer scores every entry and keeps the
 * Top-512; Hierarchical Sparse Indexer).  Bit for bit the result of
 * csa2_index_full followed by csa2_topk(scores, NULL, n_valid, B, N_cap, K,
 * ...) with the same n_valid: out_idx i32 [B, K] and out_score f32 [B, K]
 * (nullable) as csa2_topk, ids being entry positions; entries n >= n_valid[b]
 * are not candidates and their keys are not read.
 * When the rows hold at least 256 chunks of 8192 entries (B * ceil(N_cap /
 * 8192) >= 256) and D_I <= 128, one kernel scores each chunk on chip and
 * keeps its K best, so the scores never reach device memory; otherwise the
 * kernels of csa2_index_full and csa2_topk run, the scores in the workspace.
 * The workspace (at least csa2_index_topk_full_workspace_bytes(B, D_I, N_cap,
 * K) bytes, 16-byte aligned, caller-owned, contents not preserved) holds the
 * chunk winners or the scores, and the Top-K's level buffers.
 * Other arguments as csa2_index_full.  Requires 1 <= N_cap < 2^31,
 * 1 <= K <= 2048, B >= 0.
 */
size_t csa2_index_topk_full_workspace_bytes(int32_t B, int32_t D_I, int64_t N_cap, int32_t K);
int csa2_index_topk_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                         const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I,
                         int64_t N_cap, int32_t K, int32_t* out_idx, float* out_score,
                         void* workspace, size_t workspace_bytes, csa2_stream_t stream);

/*
 * a0 + a1 + a3 in one call: csa2_index_topk_full and an independent
 * csa2_quantize_fp4 (a prefill chunk's rows appended to the main cache while
 * the indexer scores the same step's queries: [P1] 效率组件四件, item 4, and
 * 架构三件套, Hierarchical Sparse Indexer).  The results are bit for bit
 * those of the two calls, in either order.  When the scoring takes the fused
 * chunk kernel, the append runs in the launch of the Top-K's last level, on
 * the CUs its B selection workgroups leave idle, so it adds no launch and
 * almost no time to the step; otherwise the append's own kernel runs first.
 * The append must not write memory the scoring reads (k_idx, q_idx, w,
 * n_valid) or the outputs and workspace (results undefined otherwise).
 * Arguments: those of csa2_index_topk_full, then those of csa2_quantize_fp4
 * (x .. capacity), each validated as in its own call (n_rows = 0: the
 * scoring alone; B = 0: the append alone).
 */
int csa2_index_topk_full_append(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I,
                                int64_t N_cap, int32_t K, int32_t* out_idx, float* out_score,
                                void* workspace, size_t workspace_bytes, const uint16_t* x,
                                int64_t n_rows, int32_t d_c, const uint16_t* rope_src, int32_t d_r,
                                uint8_t* codes, int64_t codes_stride, uint8_t* scales,
                                int64_t scales_stride, uint16_t* rope_dst, int64_t rope_stride,
                                int64_t dst_row0, int64_t capacity, csa2_stream_t stream);

/*
 * csa2_topk without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (less the workspace), same results, bit
 * for bit, as csa2_topk.  It always takes csa2_topk's chunked reduction,
 * whose level winners go to one static device array of the library (32 MiB,
 * held by each GPU the library runs on until the process ends; its device
 * address is looked up once per device).  This call allocates nothing.  Calls
 * on one GPU share that array: calls that overlap on one GPU (two streams,
 * two host threads) race, and must be ordered by the caller.  Requires the
 * chunked reduction's level buffers (see csa2_topk) to fit in 32 MiB (e.g.
 * 8192 chunks of 16384 candidates in all at K = 512); CSA2_ERR_RANGE beyond.
 * CSA2_ERR_HIP when the array's device address cannot be looked up.
 */
int csa2_topk_noalloc(const float* scores, const int32_t* ids, const int32_t* n_valid,
                      int32_t B, int64_t M, int32_t K, int32_t* out_idx, float* out_score,
                      csa2_stream_t stream);

/*
 * The decode sampler on the Top-K selection.  One Top-K implementation serves
 * the sparse attention and the sampler ([P3] DeepSelect paragraph); sampling
 * is set by a temperature and a top_p ([P1] interface paragraph).  The order
 * of the steps is this library's reading, the usual one:
 *   candidates = the row's K largest logits, in csa2_topk order (logit
 *                descending, token id ascending);
 *   w_i        = exp((l_i - l_0) / T) for the i-th candidate (0 for -inf);
 *   nucleus    = the shortest prefix of the candidates whose weight reaches
 *                top_p * sum(w) (all candidates when top_p >= 1 or when none
 *                reaches it);
 *   token      = the candidate at the first nucleus position whose running
 *                weight exceeds u * (nucleus weight) (the last position of
 *                nonzero weight if rounding leaves none);
 *   prob       = w_token / (nucleus weight), n_kept = nucleus size.
 * A row whose largest logit is -inf, or whose first slot is empty, reports
 * its first candidate with prob 1, n_kept 1.  The weights and running sums
 * are float32, so a token or nucleus end decided by a running weight within
 * float32 rounding of its threshold may differ from an exact evaluation by
 * one position; the token is always a candidate of the row.  A +inf or NaN
 * logit gives an unspecified token of the row.
 *
 * csa2_sample_draw: the draw alone, on candidates the caller already holds.
 * cand_idx   i32 [B, K] candidate token ids in csa2_topk order, -1 = empty
 *                       slot (empty slots only after the others)
 * cand_score f32 [B, K] their logits (-inf for empty slots)
 * u          f32 [B]    the uniforms, in [0, 1), drawn by the caller
 * token      i32 [B]    out: the drawn token id
 * prob       f32 [B]    out (nullable): its share of the nucleus weight
 * n_kept     i32 [B]    out (nullable): the nucleus size
 * Requires 1 <= K <= 2048, 1e-30 <= T <= 1e30, 0 < top_p (NaN rejected),
 * 16-byte aligned arrays.
 */
int csa2_sample_draw(const int32_t* cand_idx, const float* cand_score, int32_t B, int32_t K, float temperature,
                     float top_p, const float* u, int32_t* token, float* prob, int32_t* n_kept,
                     csa2_stream_t stream);

/*
 * csa2_sample: csa2_topk over the logits f32 [B, V] (row c = token id c),
 * then csa2_sample_draw, in one call.  The workspace (at least
 * csa2_sample_workspace_bytes(B, V, K) bytes, 16-byte aligned, caller-owned,
 * contents not preserved) holds the candidates and the Top-K workspace.
 * Requires 1 <= V < 2^31; the other arguments as csa2_sample_draw.
 */
size_t csa2_sample_workspace_bytes(int32_t B, int64_t V, int32_t K);
int csa2_sample(const float* logits, int32_t B, int64_t V, int32_t K, float temperature, float top_p,
                const float* u, int32_t* token, float* prob, int32_t* n_kept, void* workspace,
                size_t workspace_bytes, csa2_stream_t stream);

/*
 * The untruncated draw: the recommended sampling settings, temperature 1.0 and
 * top_p 1.0 ([P1] interface paragraph), taken literally: top_p 1.0 keeps
 * every token of the vocabulary, so no Top-K cap applies and the draw is over
 * the whole softmax of logits / T.  The order is this library's reading:
 *   w_i   = exp((l_i - l_max) / T) for every token i of the row (0 for -inf);
 *   token = the first token, in token-id order, whose running weight exceeds
 *           u * sum(w) (the last token of nonzero weight if rounding leaves
 *           none);  prob = w_token / sum(w).
 * A row whose largest logit is -inf draws token 0 with probability 1.  The
 * weights and running sums are float32 (tile totals and the running weights
 * inside a tile are summed in different orders), so a token decided by a
 * running weight within float32 rounding of u * sum(w) may differ from an
 * exact evaluation by one token; the token always has nonzero weight.  A +inf
 * or NaN logit gives an unspecified token of the row.
 *
 * logits f32 [B, V] (row b at logits + b * V), u f32 [B] in [0, 1), token
 * i32 [B] out, prob f32 [B] out (nullable).  One pass over the logits, spread
 * over several workgroups per row, then one 16384-token tile read again per
 * row.  The workspace (at least csa2_sample_full_workspace_bytes(B, V) =
 * B * ceil(V / 16384) * 128 bytes, 16-byte aligned, caller-owned, contents
 * not preserved) holds per 16384-token tile the 16 (largest scaled logit,
 * weight sum) pairs of the first pass.  Requires 1 <= V <= 2^20
 * (CSA2_ERR_RANGE beyond), 1e-30 <= T <= 1e30, 16-byte aligned arrays.
 */
size_t csa2_sample_full_workspace_bytes(int32_t B, int64_t V);
int csa2_sample_full(const float* logits, int32_t B, int64_t V, float temperature, const float* u,
                     int32_t* token, float* prob, void* workspace, size_t workspace_bytes,
                     csa2_stream_t stream);

/*
 * Sliding-window branch, write: FP8 rows of the window KV.  The window branch
 * keeps its KV in FP8 ([P4] CSA2 paragraph; [P1] 效率组件四件, item 4); the
 * pages give no scale granularity, this library uses one power-of-two scale per
 * row: sigma = 2^e, e the smallest integer with max|x| <= 448 * 2^e (1 for an
 * all-zero row, e clamped to [-126, 127]), codes = E4M3 (OCP E4M3FN) nearest
 * to |x| / sigma, ties to the even code, sign bit copied (-0 -> 0x80).
 *
 * x        bf16 [n_rows, d_c] (rows of the latent)
 * rope_src bf16 [n_rows, d_r] or NULL when d_r == 0 (copied unchanged)
 * codes    u8  rows of codes_stride bytes (0 = d_c), 8-byte aligned, stride % 8 == 0
 * sigma    f32 [capacity]  out: the row scales
 * rope_dst bf16 rows of rope_stride bytes (0 = 2 d_r), 16-byte aligned
 * Writes rows [dst_row0, dst_row0 + n_rows) of a window of `capacity` rows.
 * Bit-exact for finite inputs (an infinite or NaN element gives an
 * unspecified row, never an out-of-bounds access).  Requires d_c % 8 == 0,
 * 8 <= d_c <= 4096, d_r % 8 == 0, 0 <= d_r <= 512, 16-byte aligned x /
 * rope_src, 4-byte aligned sigma.
 */
int csa2_quantize_fp8(const uint16_t* x, int64_t n_rows, int32_t d_c, const uint16_t* rope_src,
                      int32_t d_r, uint8_t* codes, int64_t codes_stride, float* sigma,
                      uint16_t* rope_dst, int64_t rope_stride, int64_t dst_row0, int64_t capacity,
                      csa2_stream_t stream);

/*
 * The sparse attention and the sliding window in one call: one softmax over
 * the union of the selected entries and the query's window rows ([P4] CSA2
 * paragraph: the SWA branch, its KV in FP8, beside the sparse one), i.e. the
 * result csa2_sparse_attn_fp4 followed by csa2_swa_attn_fp8 merging into it
 * gives, up to rounding.  Arguments as csa2_sparse_attn_fp4 (the selected
 * entries) and csa2_swa_attn_fp8 (w_codes / w_sigma / w_rope / n_win / W_cap,
 * the window rows of query b); W_cap = 0 (window pointers may then be NULL)
 * is the sparse attention alone.  out f32 [B, H, 512], lse f32 [B, H]
 * (nullable).
 * When the batch gives at least 64 units of 32 heads (B * ceil(H / 32) >=
 * 64; each query then in at most four slices, the window in the first) one
 * kernel attends to the window rows as more tiles after the
 * selected entries': exact E4M3 values in fp16, the row scale applied to the
 * fp32 latent scores and, as sigma_j / max sigma, to the probabilities of
 * the value products (the accumulator divided by max sigma before the first
 * window tile and multiplied by it at the end).  Other batches run the
 * sparse kernels, then the window kernel merging into their result.  The
 * error is < 2e-3 of max|out| per (b, h) row.
 * Requires d_c == 512, d_r in {0, 64}, 1 <= H <= 128, K >= 1, 0 <= W_cap <=
 * 256, the alignment rules of both calls, and a workspace of at least
 * csa2_sparse_swa_attn_workspace_bytes(B, H, d_c, K) bytes (16-byte aligned,
 * caller-owned, contents not preserved).
 */
size_t csa2_sparse_swa_attn_workspace_bytes(int32_t B, int32_t H, int32_t d_c, int32_t K);
int csa2_sparse_swa_attn_fp4(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                             const uint8_t* scales, int64_t scales_stride, const uint16_t* rope,
                             int64_t rope_stride, const int32_t* idx, int32_t K, int32_t B, int32_t H,
                             int32_t d_c, int32_t d_r, int64_t N_cap, const uint8_t* w_codes,
                             int64_t w_codes_stride, const float* w_sigma, const uint16_t* w_rope,
                             int64_t w_rope_stride, const int32_t* n_win, int32_t W_cap, float sm_scale,
                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                             csa2_stream_t stream);

/*
 * Sliding-window branch, attention, and its merge with the sparse branch.  A
 * layer's sparse branch and its SWA branch ([P4] CSA2 paragraph) are read as
 * one softmax over the union of their keys: the window rows attend like the
 * selected entries (key = [dequant(latent) ; rope], value = dequant(latent),
 * dequant = E4M3 value * sigma of the row), and the two results combine as
 *   out = (e^lse_s out_s + e^lse_w out_w) / (e^lse_s + e^lse_w),
 *   lse = log(e^lse_s + e^lse_w),
 * which is why csa2_sparse_attn_fp4 exports its lse.
 *
 * q         bf16 [B, H, d_c + d_r]
 * codes     u8   window rows of csa2_quantize_fp8: row j of sequence b is row
 *                b * W_cap + j (codes_stride bytes apart, 0 = d_c), sigma f32
 *                [B, W_cap], rope bf16 rows (rope_stride bytes, 0 = 2 d_r)
 * n_win     i32  [B]  rows j < n_win[b] form the window (NULL = W_cap;
 *                clamped to [0, W_cap] on the device); their order is free
 * merge_out f32 [B, H, d_c], merge_lse f32 [B, H]: the sparse branch's result
 *                (csa2_sparse_attn_fp4), both NULL for the window branch alone;
 *                merge_out may be the same buffer as out
 * out       f32  [B, H, d_c] out;  lse f32 [B, H] out (nullable)
 * An empty window leaves the sparse result unchanged (or gives out = 0,
 * lse = -inf alone).  Scores and values use the exact E4M3 values in fp16
 * with fp32 accumulation; the row scales multiply the fp32 latent scores and
 * enter P as sigma_j / max sigma (exact for the power-of-two scales
 * csa2_quantize_fp8 writes): the error is < 2e-3 of max|out| per (b, h) row.
 * Requires d_c == 512, d_r in {0, 64}, 1 <= H <= 128, 0 <= W_cap <= 256
 * (CSA2_ERR_RANGE beyond), 16-byte aligned q, out, codes, rope and their
 * strides, 4-byte aligned sigma, window values of E4M3 codes (no 0x7F/0xFF).
 */
int csa2_swa_attn_fp8(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                      const float* sigma, const uint16_t* rope, int64_t rope_stride,
                      const int32_t* n_win, int32_t B, int32_t H, int32_t d_c, int32_t d_r,
                      int32_t W_cap, float sm_scale, const float* merge_out,
                      const float* merge_lse, float* out, float* lse, csa2_stream_t stream);

/*
 * Candidate-pool construction for Reindex mode: the block-level pool that the
 * decoder's first Full layer keeps (at most 2048 blocks x 8 positions) so that
 * later layers score only inside it ([P1] 架构三件套, Hierarchical Sparse
 * Indexer; [P4] CSA2 paragraph).  The pages give no block score; this library
 * reads it as the largest score of the block's valid positions.
 *
 * scores      f32 [B, M]  a Full layer's indexer scores (csa2_index_full)
 * n_valid     i32 [B]     positions p < n_valid[b] are valid (NULL = M;
 *                         clamped to [0, M] on the device)
 * block       positions per block (block b covers [block*b, block*b + block));
 *             a block is a candidate when its first position is valid
 * pool_blocks i32 [B, P_max]  out: the first min(P_max, #candidates) block ids
 *             by (block score descending, block id ascending), then -1; block
 *             score = max of the valid positions' scores (NaN ignored unless
 *             all are NaN).  Ready for csa2_index_pool (whose result does not
 *             depend on the order of the pool).
 * n_blocks    i32 [B]     out: min(P_max, #candidates)
 * Bit-exact (comparisons only).  Requires 1 <= block <= 64,
 * 1 <= P_max <= 2048, 1 <= M < 2^31, B >= 0, 16-byte aligned scores,
 * pool_blocks, n_blocks (and n_valid when given), and a caller workspace of at
 * least csa2_build_pool_workspace_bytes(B, M, block, P_max) bytes, 16-byte
 * aligned (block scores, candidate counts, Top-K chunk winners).
 */
size_t csa2_build_pool_workspace_bytes(int32_t B, int64_t M, int32_t block, int32_t P_max);
int csa2_build_pool(const float* scores, const int32_t* n_valid, int32_t B, int64_t M,
                    int32_t block, int32_t P_max, int32_t* pool_blocks, int32_t* n_blocks,
                    void* workspace, size_t workspace_bytes, csa2_stream_t stream);

/*
 * a4 + a5. Gather, FP4 dequantisation and softmax attention over the
 * selected entries (also the whole of Reuse mode, where idx is handed in).
 * Defined by [P1] 架构三件套, CSA2 (Reuse reuses KV and the index and runs
 * sparse attention directly), [P3] (modes paragraph) and [P4] CSA2 paragraph;
 * the entry layout is MLA-style: key_j = [dequant(latent_j) ; rope_j],
 * value_j = dequant(latent_j), shared by all H query heads.
 *
 * q      bf16 [B, H, d_c + d_r]
 * codes / scales / rope   the cache of csa2_quantize_fp4 (same row strides, 0 =
 *        dense), B sequences of N_cap rows each: entry n of sequence b is row
 *        b * N_cap + n; rope is NULL iff d_r == 0
 * idx    i32  [B, K]  selected entries; ids < 0 or >= N_cap are skipped,
 *                     repeated ids count with multiplicity
 * out    f32  [B, H, d_c]  softmax(sm_scale * q . key) . value
 * lse    f32  [B, H]  (nullable) natural-log sum-exp of the scaled scores
 * A row with no usable entry gets out = 0, lse = -inf.
 * Dequantised values are exact (E2M1 x E4M3 has at most 6 significant bits);
 * products are formed by the matrix cores with fp32 accumulation and the
 * softmax runs in fp32: the error against an exact evaluation is < 2e-3 of
 * max|out| per (b, h) row for unit-scale inputs.
 * Requires d_c in {128, 512}, d_r in {0, 64}, 1 <= H <= 128, K >= 1, B >= 0,
 * the alignment rules of csa2_quantize_fp4 for the cache, N_cap * stride <=
 * 4 GiB for each of codes, scales and rope (one sequence's rows; else
 * CSA2_ERR_RANGE), and a workspace of
 * csa2_sparse_attn_workspace_bytes(B, H, d_c, K) bytes.
 */
size_t csa2_sparse_attn_workspace_bytes(int32_t B, int32_t H, int32_t d_c, int32_t K);
int csa2_sparse_attn_fp4(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                         const uint8_t* scales, int64_t scales_stride, const uint16_t* rope,
                         int64_t rope_stride, const int32_t* idx, int32_t K, int32_t B,
                         int32_t H, int32_t d_c, int32_t d_r, int64_t N_cap, float sm_scale,
                         float* out, float* lse, void* workspace, size_t workspace_bytes,
                         csa2_stream_t stream);

/*
 * Prefill sparse attention: a chunk of T queries of each of S sequences,
 * every query with its own index list into its own sequence's cache.  The
 * Reuse layers run in prefill too ([P1] inference-kernel paragraph); each
 * prefill query attends exactly like a decode query of csa2_sparse_attn_fp4
 * (same formula, same accuracy), and causality is the lists' business: an
 * entry a query may not see must not be in its list.
 *
 * q    bf16 [S, T, H, d_c + d_r]   (query t of sequence s is row s * T + t)
 * idx  i32  [S, T, K]              entry ids into the sequence's rows, -1 = none
 * out  f32  [S, T, H, d_c], lse f32 [S, T, H] (nullable)
 * codes / scales / rope: one cache per sequence, as csa2_sparse_attn_fp4
 * (sequence s's row r at s * N_cap + r).  The workspace is
 * csa2_sparse_attn_workspace_bytes(S * T, H, d_c, K) bytes.  Requires
 * S, T >= 0 and S * T <= 2^24; the rest as csa2_sparse_attn_fp4.
 */
int csa2_prefill_sparse_attn_fp4(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                                 const uint8_t* scales, int64_t scales_stride, const uint16_t* rope,
                                 int64_t rope_stride, const int32_t* idx, int32_t K, int32_t S, int32_t T,
                                 int32_t H, int32_t d_c, int32_t d_r, int64_t N_cap, float sm_scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes, csa2_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
