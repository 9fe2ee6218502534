// Internal launch entry points of libcsa2 (host side).  Each returns the HIP
// error of its launches; arguments are validated by csa2_api.hip beforehand.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Work-items (workgroups x threads) of the largest single launch a call makes,
// computed by the same grid rules the launches use: one launch holds fewer
// than 2^32, so the entry points refuse larger calls (CSA2_ERR_RANGE) before
// anything is enqueued.
constexpr int64_t kMaxLaunchItems = ((int64_t)1 << 32) - 1;
int64_t quantize_fp4_launch_items(int64_t n_rows, int d_c, int d_r);
int64_t quantize_fp8_launch_items(int64_t n_rows);
int64_t index_launch_items(int B, int64_t M, bool pool, int block, int D_I);
int64_t topk_launch_items(int B, int64_t M, int K);
int64_t pool_launch_items(int B, int64_t M, int block, int P_max);
int64_t attn_launch_items(int B, int H, int d_c, int K);
int64_t swa_launch_items(int B, int H);
int64_t sample_draw_launch_items(int B);

// Row strides are in bytes and already resolved (non-zero).
struct CacheRef {
  uint8_t* codes;
  int64_t codes_stride;
  uint8_t* scales;
  int64_t scales_stride;
  uint16_t* rope;
  int64_t rope_stride;
};

// An FP4 append (csa2_quantize_fp4's operands, validated): rows [0, n_rows)
// of x (bf16, d_c each) and rope_src (bf16, d_r each; null when d_r == 0)
// into cache rows dst_row0 + r.
struct Fp4Append {
  const uint16_t* x;
  int64_t n_rows;
  int d_c;
  const uint16_t* rope_src;
  int d_r;
  CacheRef cache;
  int64_t dst_row0;
};

// The FP8 sliding window of each query for the attention kernels (codes null:
// no window): rows j < n_win[b] (clamped to [0, W_cap]; n_win null = W_cap)
// of query b are rows b * W_cap + j of codes / sigma / rope, as written by
// csa2_quantize_fp8.
struct WinRef {
  const uint8_t* codes;
  int64_t codes_stride;
  const float* sigma;
  const uint16_t* rope;
  int64_t rope_stride;
  const int32_t* n_win;
  int W_cap;
};

hipError_t launch_quantize_fp4(const uint16_t* x, int64_t n_rows, int d_c, const uint16_t* rope_src,
                               int d_r, CacheRef cache, int64_t dst_row0, hipStream_t stream);

hipError_t launch_index(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* n_valid,
                        int B, int H_I, int D_I, int64_t N_cap, const int32_t* pool,
                        const int32_t* n_blocks, int P_max, int block, float* scores,
                        int32_t* positions, hipStream_t stream);

// Size of the static device scratch array (scratch.hip) and the lookup of its
// device address on the current device (once per device; thread-safe).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** ptr);

// Top-K of B rows of M scores: the threshold filter for long rows (more than
// one round of chunk workgroups or more than two chunk levels), else the
// chunked reduction.  topk_chunk_* always take the chunked reduction.
size_t topk_workspace_bytes(int B, int64_t M, int K);
hipError_t launch_topk(const float* scores, const int32_t* ids, const int32_t* n_valid, int B,
                       int64_t M, int K, int32_t* out_idx, float* out_score, void* workspace,
                       hipStream_t stream);
int64_t topk_chunk_launch_items(int B, int64_t M, int K);
size_t topk_chunk_workspace_bytes(int B, int64_t M, int K);
hipError_t launch_topk_chunked(const float* scores, const int32_t* ids, const int32_t* n_valid, int B,
                               int64_t M, int K, int32_t* out_idx, float* out_score, void* workspace,
                               hipStream_t stream);
// The threshold filter's limits (rows of 16384 < M <= 2^20, K <= 2048), sizes
// and launches.
bool topk_filter_fits(int B, int64_t M, int K);
int64_t topk_filter_launch_items(int B, int64_t M);
size_t topk_filter_workspace_bytes(int B);
// The sampler's draw settings, for a Top-K whose last kernel also draws
// (csa2_sample): the draw of sample_draw_kernel over the candidate rows.
struct SampleDraw {
  float log2e_over_t;
  float top_p;
  const float* u;
  int32_t* token;
  float* prob;
  int32_t* n_kept;
};
// `draw` (nullable, scores without ids only): the last kernel draws too.
hipError_t launch_topk_filtered(const float* scores, const int32_t* ids, const int32_t* n_valid, int B, int64_t M,
                                int K, int32_t* out_idx, float* out_score, void* workspace, hipStream_t stream,
                                const SampleDraw* draw = nullptr);
// Whether csa2_topk's dispatch takes the threshold filter for these rows.
bool topk_uses_filter(int B, int64_t M, int K);
// The Top-K levels after the first, on B rows of m chunk-winner keys.
size_t topk_keys_workspace_bytes(int B, int64_t m, int K);
// `app` (nullable): an independent FP4 append run by extra workgroups of the
// final level's launch, on the CUs its B selection workgroups leave idle.
hipError_t launch_topk_from_keys(const uint64_t* keys, int B, int64_t m, int K, int32_t* out_idx,
                                 float* out_score, void* workspace, hipStream_t stream,
                                 const Fp4Append* app = nullptr);

// Full-mode indexer scores and their Top-K in one call (fused chunk kernel when
// the rows give a workgroup per CU, else the two kernels).
int64_t index_topk_launch_items(int B, int D_I, int64_t N_cap, int K);
size_t index_topk_workspace_bytes(int B, int D_I, int64_t N_cap, int K);
// `app` (nullable): an FP4 append to run in the same call, independent of the
// scoring (in the final Top-K level's launch on the fused path, else first).
hipError_t launch_index_topk(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* n_valid, int B,
                             int H_I, int D_I, int64_t N_cap, int K, int32_t* out_idx, float* out_score,
                             void* workspace, hipStream_t stream, const Fp4Append* app = nullptr);
int64_t topk_final_append_launch_items(int B, const Fp4Append& app);

size_t pool_workspace_bytes(int B, int64_t M, int block, int P_max);
hipError_t launch_build_pool(const float* scores, const int32_t* n_valid, int B, int64_t M, int block,
                             int P_max, int32_t* pool_blocks, int32_t* n_blocks, void* workspace,
                             hipStream_t stream);

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t n_rows, int d_c, const uint16_t* rope_src, int d_r,
                               uint8_t* codes, int64_t codes_stride, float* sigma, uint16_t* rope_dst,
                               int64_t rope_stride, int64_t dst_row0, hipStream_t stream);
hipError_t launch_swa_attn(const uint16_t* q, const uint8_t* codes, int64_t codes_stride, const float* sigma,
                           const uint16_t* rope, int64_t rope_stride, const int32_t* n_win, int B, int H, int d_r,
                           int W_cap, float sm_scale, const float* in_out, const float* in_lse, float* out,
                           float* lse, hipStream_t stream);

size_t sample_workspace_bytes(int B, int64_t V, int K);
hipError_t launch_sample_draw(const int32_t* cand_idx, const float* cand_score, int B, int K, float temperature,
                              float top_p, const float* u, int32_t* token, float* prob, int32_t* n_kept,
                              hipStream_t stream);
int64_t sample_full_launch_items(int B, int64_t V);
constexpr int64_t kSampleFullMaxVocab = (int64_t)1 << 20;
size_t sample_full_workspace_bytes(int B, int64_t V);
hipError_t launch_sample_full(const float* logits, int B, int64_t V, float temperature, const float* u,
                              int32_t* token, float* prob, void* workspace, hipStream_t stream);
hipError_t launch_sample(const float* logits, int B, int64_t V, int K, float temperature, float top_p,
                         const float* u, int32_t* token, float* prob, int32_t* n_kept, void* workspace,
                         hipStream_t stream);

size_t attn_workspace_bytes(int B, int H, int d_c, int K);
// Query b reads the rows of sequence b / qps (qps = 1: one query per sequence).
hipError_t launch_sparse_attn(const uint16_t* q, CacheRef cache, const int32_t* idx, int K, int B, int H,
                              int d_c, int d_r, int64_t N_cap, int qps, float sm_scale, float* out, float* lse,
                              void* workspace, hipStream_t stream);
// The sparse attention and the sliding window of each query in one softmax:
// inside the 32-head kernel when it serves the batch (window tiles first),
// else the sparse kernels, then the window kernel merging into their result
// (lse_tmp: B x H floats for that merge when lse is null).  Decode only (one
// query per sequence), d_c = 512.
bool sparse_swa_fused(int B, int H, int d_c);
size_t sparse_swa_workspace_bytes(int B, int H, int d_c, int K);
hipError_t launch_sparse_swa_attn(const uint16_t* q, CacheRef cache, const int32_t* idx, int K, int B, int H,
                                  int d_r, int64_t N_cap, WinRef win, float sm_scale, float* out, float* lse,
                                  void* workspace, hipStream_t stream);

}  // namespace csa2
