// extern "C" boundary of libcsa2: host-side validation, then the launches.
// Nothing here allocates device memory or synchronises.
#include "../../include/csa2.h"
#include "csa2_internal.h"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool opt_aligned16(const void* p) { return p == nullptr || aligned16(p); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }
inline hipStream_t as_stream(csa2_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline bool too_large(int64_t items) { return items > csa2::kMaxLaunchItems; }

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "a size is negative or inconsistent";
    case CSA2_ERR_ALIGN: return "a pointer or stride breaks its alignment rule";
    case CSA2_ERR_RANGE: return "a value is out of its allowed range";
    case CSA2_ERR_UNSUPPORTED: return "dimensions without a compiled kernel";
    case CSA2_ERR_HIP: return "the HIP runtime refused a launch";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int csa2_version(void) { return 100; }

// Resolves 0 strides to dense rows and checks the cache layout rules.
static int check_cache(int32_t d_c, int32_t d_r, const void* codes, int64_t& codes_stride,
                       const void* scales, int64_t& scales_stride, const void* rope, int64_t& rope_stride) {
  if (codes_stride == 0) codes_stride = d_c / 2;
  if (scales_stride == 0) scales_stride = d_c / 16;
  if (rope_stride == 0) rope_stride = 2 * (int64_t)d_r;
  if (codes_stride < d_c / 2 || scales_stride < d_c / 16 || (d_r > 0 && rope_stride < 2 * (int64_t)d_r))
    return CSA2_ERR_SHAPE;
  if (!aligned16(codes) || codes_stride % 16 != 0) return CSA2_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(scales) & 1u) != 0 || scales_stride % 2 != 0) return CSA2_ERR_ALIGN;
  if (d_r > 0 && (!aligned16(rope) || rope_stride % 16 != 0)) return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

// Validates csa2_quantize_fp4's operands and fills *a (n_rows == 0: CSA2_OK
// with a->n_rows = 0 and nothing else looked at).
static int check_fp4_append(const uint16_t* x, int64_t n_rows, int32_t d_c, const uint16_t* rope_src,
                            int32_t d_r, uint8_t* codes, int64_t codes_stride, uint8_t* scales,
                            int64_t scales_stride, uint16_t* rope_dst, int64_t rope_stride, int64_t dst_row0,
                            int64_t capacity, csa2::Fp4Append* a) {
  a->n_rows = 0;
  if (n_rows < 0 || capacity < 0 || d_c < 32 || d_c > 4096 || d_c % 32 != 0 || d_r < 0 ||
      d_r > 1024 || d_r % 8 != 0 || codes_stride < 0 || scales_stride < 0 || rope_stride < 0)
    return CSA2_ERR_SHAPE;
  if (dst_row0 < 0 || dst_row0 > capacity || n_rows > capacity - dst_row0) return CSA2_ERR_RANGE;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !codes || !scales || (d_r > 0 && (!rope_src || !rope_dst))) return CSA2_ERR_NULL;
  if (!aligned16(x) || !opt_aligned16(rope_src)) return CSA2_ERR_ALIGN;
  const int st = check_cache(d_c, d_r, codes, codes_stride, scales, scales_stride, rope_dst, rope_stride);
  if (st != CSA2_OK) return st;
  if (too_large(csa2::quantize_fp4_launch_items(n_rows, d_c, d_r))) return CSA2_ERR_RANGE;
  const csa2::CacheRef c{codes, codes_stride, scales, scales_stride, d_r > 0 ? rope_dst : nullptr, rope_stride};
  *a = csa2::Fp4Append{x, n_rows, d_c, d_r > 0 ? rope_src : nullptr, d_r, c, dst_row0};
  return CSA2_OK;
}

int csa2_quantize_fp4(const uint16_t* x, int64_t n_rows, int32_t d_c, const uint16_t* rope_src,
                      int32_t d_r, uint8_t* codes, int64_t codes_stride, uint8_t* scales,
                      int64_t scales_stride, uint16_t* rope_dst, int64_t rope_stride,
                      int64_t dst_row0, int64_t capacity, csa2_stream_t stream) {
  csa2::Fp4Append a;
  const int st = check_fp4_append(x, n_rows, d_c, rope_src, d_r, codes, codes_stride, scales, scales_stride,
                                  rope_dst, rope_stride, dst_row0, capacity, &a);
  if (st != CSA2_OK || a.n_rows == 0) return st;
  return hip_status(csa2::launch_quantize_fp4(a.x, a.n_rows, a.d_c, a.rope_src, a.d_r, a.cache, a.dst_row0,
                                              as_stream(stream)));
}

int csa2_quantize_fp8(const uint16_t* x, int64_t n_rows, int32_t d_c, const uint16_t* rope_src,
                      int32_t d_r, uint8_t* codes, int64_t codes_stride, float* sigma,
                      uint16_t* rope_dst, int64_t rope_stride, int64_t dst_row0, int64_t capacity,
                      csa2_stream_t stream) {
  if (n_rows < 0 || capacity < 0 || d_c < 8 || d_c > 4096 || d_c % 8 != 0 || d_r < 0 || d_r > 512 ||
      d_r % 8 != 0 || codes_stride < 0 || rope_stride < 0)
    return CSA2_ERR_SHAPE;
  if (dst_row0 < 0 || dst_row0 > capacity || n_rows > capacity - dst_row0) return CSA2_ERR_RANGE;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !codes || !sigma || (d_r > 0 && (!rope_src || !rope_dst))) return CSA2_ERR_NULL;
  if (codes_stride == 0) codes_stride = d_c;
  if (rope_stride == 0) rope_stride = 2 * (int64_t)d_r;
  if (codes_stride < d_c || (d_r > 0 && rope_stride < 2 * (int64_t)d_r)) return CSA2_ERR_SHAPE;
  if (!aligned16(x) || !opt_aligned16(rope_src) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0 ||
      codes_stride % 8 != 0 || (reinterpret_cast<uintptr_t>(sigma) & 3u) != 0 ||
      (d_r > 0 && (!aligned16(rope_dst) || rope_stride % 16 != 0)))
    return CSA2_ERR_ALIGN;
  if (too_large(csa2::quantize_fp8_launch_items(n_rows))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_quantize_fp8(x, n_rows, d_c, d_r > 0 ? rope_src : nullptr, d_r, codes,
                                              codes_stride, sigma, d_r > 0 ? rope_dst : nullptr, rope_stride,
                                              dst_row0, as_stream(stream)));
}

static int check_index_common(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                              const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I,
                              int64_t N_cap, const float* scores) {
  if (B < 0 || N_cap < 0) return CSA2_ERR_SHAPE;
  if (H_I < 1 || H_I > 16 || (D_I != 32 && D_I != 64 && D_I != 128 && D_I != 256))
    return CSA2_ERR_UNSUPPORTED;
  if (!q_idx || !k_idx || !scores) return CSA2_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(scores) || !opt_aligned16(w) ||
      !opt_aligned16(n_valid))
    return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

int csa2_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                    const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I, int64_t N_cap,
                    float* scores, csa2_stream_t stream) {
  if (B == 0 || N_cap == 0) {
    if (B < 0 || N_cap < 0) return CSA2_ERR_SHAPE;
    return CSA2_OK;
  }
  const int st = check_index_common(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, scores);
  if (st != CSA2_OK) return st;
  if (too_large(csa2::index_launch_items(B, N_cap, false, 1, D_I))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_index(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, nullptr,
                                       nullptr, 0, 1, scores, nullptr, as_stream(stream)));
}

int csa2_index_pool(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                    const int32_t* n_valid, const int32_t* pool_blocks, const int32_t* n_blocks,
                    int32_t B, int32_t H_I, int32_t D_I, int64_t N_cap, int32_t P_max, int32_t block,
                    float* scores, int32_t* positions, csa2_stream_t stream) {
  if (B < 0 || N_cap < 0 || P_max < 1) return CSA2_ERR_SHAPE;
  if (block < 1 || block > 64 || (int64_t)P_max * block > (1 << 24)) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  const int st = check_index_common(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, scores);
  if (st != CSA2_OK) return st;
  if (!pool_blocks || !n_blocks || !positions) return CSA2_ERR_NULL;
  if (!aligned16(pool_blocks) || !aligned16(n_blocks) || !aligned16(positions)) return CSA2_ERR_ALIGN;
  if (too_large(csa2::index_launch_items(B, (int64_t)P_max * block, true, block, D_I))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_index(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, pool_blocks,
                                       n_blocks, P_max, block, scores, positions,
                                       as_stream(stream)));
}

int csa2_swa_attn_fp8(const uint16_t* q, const uint8_t* codes, int64_t codes_stride, const float* sigma,
                      const uint16_t* rope, int64_t rope_stride, const int32_t* n_win, int32_t B, int32_t H,
                      int32_t d_c, int32_t d_r, int32_t W_cap, float sm_scale, const float* merge_out,
                      const float* merge_lse, float* out, float* lse, csa2_stream_t stream) {
  if (B < 0 || W_cap < 0 || codes_stride < 0 || rope_stride < 0) return CSA2_ERR_SHAPE;
  if (d_c != 512 || !(d_r == 0 || d_r == 64) || H < 1 || H > 128) return CSA2_ERR_UNSUPPORTED;
  if (W_cap > 256) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!q || !out || (W_cap > 0 && (!codes || !sigma || (d_r > 0 && !rope))) || (!merge_out != !merge_lse))
    return CSA2_ERR_NULL;
  if (codes_stride == 0) codes_stride = d_c;
  if (rope_stride == 0) rope_stride = 2 * (int64_t)d_r;
  if (codes_stride < d_c || (d_r > 0 && rope_stride < 2 * (int64_t)d_r)) return CSA2_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out) || !opt_aligned16(lse) || !opt_aligned16(merge_out) ||
      !opt_aligned16(merge_lse) || !opt_aligned16(n_win) || (W_cap > 0 && (!aligned16(codes) ||
      codes_stride % 16 != 0 || (reinterpret_cast<uintptr_t>(sigma) & 3u) != 0 ||
      (d_r > 0 && (!aligned16(rope) || rope_stride % 16 != 0)))))
    return CSA2_ERR_ALIGN;
  if (too_large(csa2::swa_launch_items(B, H))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_swa_attn(q, codes, codes_stride, sigma, d_r > 0 ? rope : nullptr, rope_stride,
                                          n_win, B, H, d_r, W_cap, sm_scale, merge_out, merge_lse, out, lse,
                                          as_stream(stream)));
}

size_t csa2_build_pool_workspace_bytes(int32_t B, int64_t M, int32_t block, int32_t P_max) {
  if (B <= 0 || M < 1 || M > INT32_MAX || block < 1 || block > 64 || P_max < 1 || P_max > 2048) return 0;
  return csa2::pool_workspace_bytes(B, M, block, P_max);
}

int csa2_build_pool(const float* scores, const int32_t* n_valid, int32_t B, int64_t M, int32_t block,
                    int32_t P_max, int32_t* pool_blocks, int32_t* n_blocks, void* workspace,
                    size_t workspace_bytes, csa2_stream_t stream) {
  if (B < 0 || M < 1 || M > INT32_MAX) return CSA2_ERR_SHAPE;
  if (block < 1 || block > 64 || P_max < 1 || P_max > 2048) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!scores || !pool_blocks || !n_blocks || !workspace) return CSA2_ERR_NULL;
  if (!aligned16(scores) || !aligned16(pool_blocks) || !aligned16(n_blocks) || !opt_aligned16(n_valid) ||
      !aligned16(workspace))
    return CSA2_ERR_ALIGN;
  if (workspace_bytes < csa2::pool_workspace_bytes(B, M, block, P_max)) return CSA2_ERR_WORKSPACE;
  if (too_large(csa2::pool_launch_items(B, M, block, P_max))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_build_pool(scores, n_valid, B, M, block, P_max, pool_blocks, n_blocks,
                                            workspace, as_stream(stream)));
}

size_t csa2_topk_workspace_bytes(int32_t B, int64_t M, int32_t K) {
  if (B <= 0 || M < 1 || K < 1 || K > 2048) return 0;
  return csa2::topk_workspace_bytes(B, M, K);
}

int csa2_topk(const float* scores, const int32_t* ids, const int32_t* n_valid, int32_t B, int64_t M,
              int32_t K, int32_t* out_idx, float* out_score, void* workspace,
              size_t workspace_bytes, csa2_stream_t stream) {
  if (B < 0 || M < 1 || M > 0x7FFFFFFFll) return CSA2_ERR_SHAPE;
  if (K < 1 || K > 2048) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!scores || !out_idx) return CSA2_ERR_NULL;
  if (!aligned16(scores) || !aligned16(out_idx) || !opt_aligned16(ids) || !opt_aligned16(n_valid) ||
      !opt_aligned16(out_score))
    return CSA2_ERR_ALIGN;
  const size_t need = csa2::topk_workspace_bytes(B, M, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return CSA2_ERR_ALIGN;
  if (too_large(csa2::topk_launch_items(B, M, K))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_topk(scores, ids, n_valid, B, M, K, out_idx, out_score, workspace,
                                      as_stream(stream)));
}

size_t csa2_index_topk_full_workspace_bytes(int32_t B, int32_t D_I, int64_t N_cap, int32_t K) {
  if (B <= 0 || N_cap < 1 || N_cap > 0x7FFFFFFFll || K < 1 || K > 2048) return 0;
  if (D_I != 32 && D_I != 64 && D_I != 128 && D_I != 256) return 0;
  return csa2::index_topk_workspace_bytes(B, D_I, N_cap, K);
}

static int check_index_topk_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                 const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I, int64_t N_cap,
                                 int32_t K, int32_t* out_idx, float* out_score, void* workspace,
                                 size_t workspace_bytes) {
  if (B < 0 || N_cap < 1 || N_cap > 0x7FFFFFFFll) return CSA2_ERR_SHAPE;
  if (K < 1 || K > 2048) return CSA2_ERR_RANGE;
  if (H_I < 1 || H_I > 16 || (D_I != 32 && D_I != 64 && D_I != 128 && D_I != 256)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!q_idx || !k_idx || !out_idx) return CSA2_ERR_NULL;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(out_idx) || !opt_aligned16(w) ||
      !opt_aligned16(n_valid) || !opt_aligned16(out_score))
    return CSA2_ERR_ALIGN;
  const size_t need = csa2::index_topk_workspace_bytes(B, D_I, N_cap, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return CSA2_ERR_ALIGN;
  if (too_large(csa2::index_topk_launch_items(B, D_I, N_cap, K))) return CSA2_ERR_RANGE;
  return CSA2_OK;
}

int csa2_index_topk_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, const int32_t* n_valid,
                         int32_t B, int32_t H_I, int32_t D_I, int64_t N_cap, int32_t K, int32_t* out_idx,
                         float* out_score, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
  const int st = check_index_topk_full(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, K, out_idx, out_score,
                                       workspace, workspace_bytes);
  if (st != CSA2_OK || B == 0) return st;
  return hip_status(csa2::launch_index_topk(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, K, out_idx, out_score,
                                            workspace, as_stream(stream)));
}

int csa2_index_topk_full_append(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                const int32_t* n_valid, int32_t B, int32_t H_I, int32_t D_I, int64_t N_cap,
                                int32_t K, int32_t* out_idx, float* out_score, void* workspace,
                                size_t workspace_bytes, const uint16_t* x, int64_t n_rows, int32_t d_c,
                                const uint16_t* rope_src, int32_t d_r, uint8_t* codes, int64_t codes_stride,
                                uint8_t* scales, int64_t scales_stride, uint16_t* rope_dst, int64_t rope_stride,
                                int64_t dst_row0, int64_t capacity, csa2_stream_t stream) {
  int st = check_index_topk_full(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, K, out_idx, out_score, workspace,
                                 workspace_bytes);
  if (st != CSA2_OK) return st;
  csa2::Fp4Append a;
  st = check_fp4_append(x, n_rows, d_c, rope_src, d_r, codes, codes_stride, scales, scales_stride, rope_dst,
                        rope_stride, dst_row0, capacity, &a);
  if (st != CSA2_OK) return st;
  if (a.n_rows > 0 && too_large(csa2::topk_final_append_launch_items(B, a))) return CSA2_ERR_RANGE;
  if (B == 0 && a.n_rows == 0) return CSA2_OK;
  return hip_status(csa2::launch_index_topk(q_idx, w, k_idx, n_valid, B, H_I, D_I, N_cap, K, out_idx, out_score,
                                            workspace, as_stream(stream), a.n_rows > 0 ? &a : nullptr));
}

int csa2_topk_noalloc(const float* scores, const int32_t* ids, const int32_t* n_valid, int32_t B, int64_t M,
                      int32_t K, int32_t* out_idx, float* out_score, csa2_stream_t stream) {
  if (B < 0 || M < 1 || M > 0x7FFFFFFFll) return CSA2_ERR_SHAPE;
  if (K < 1 || K > 2048) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!scores || !out_idx) return CSA2_ERR_NULL;
  if (!aligned16(scores) || !aligned16(out_idx) || !opt_aligned16(ids) || !opt_aligned16(n_valid) ||
      !opt_aligned16(out_score))
    return CSA2_ERR_ALIGN;
  const size_t need = csa2::topk_chunk_workspace_bytes(B, M, K);
  if (need > csa2::kStaticScratchBytes) return CSA2_ERR_RANGE;
  if (too_large(csa2::topk_chunk_launch_items(B, M, K))) return CSA2_ERR_RANGE;
  void* ws = nullptr;
  if (need > 0 && csa2::static_scratch(&ws) != hipSuccess) return CSA2_ERR_HIP;
  return hip_status(
      csa2::launch_topk_chunked(scores, ids, n_valid, B, M, K, out_idx, out_score, ws, as_stream(stream)));
}

static bool sampler_params_ok(float temperature, float top_p) {
  // 1/T must stay a finite float; top_p > 0 (NaN fails both tests)
  return temperature >= 1e-30f && temperature <= 1e30f && top_p > 0.0f && top_p <= 1e30f;
}

int csa2_sample_draw(const int32_t* cand_idx, const float* cand_score, int32_t B, int32_t K, float temperature,
                     float top_p, const float* u, int32_t* token, float* prob, int32_t* n_kept,
                     csa2_stream_t stream) {
  if (B < 0) return CSA2_ERR_SHAPE;
  if (K < 1 || K > 2048 || !sampler_params_ok(temperature, top_p)) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!cand_idx || !cand_score || !u || !token) return CSA2_ERR_NULL;
  if (!aligned16(cand_idx) || !aligned16(cand_score) || !aligned16(u) || !aligned16(token) ||
      !opt_aligned16(prob) || !opt_aligned16(n_kept))
    return CSA2_ERR_ALIGN;
  if (too_large(csa2::sample_draw_launch_items(B))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_sample_draw(cand_idx, cand_score, B, K, temperature, top_p, u, token, prob,
                                             n_kept, as_stream(stream)));
}

size_t csa2_sample_workspace_bytes(int32_t B, int64_t V, int32_t K) {
  if (B <= 0 || V < 1 || V > 0x7FFFFFFFll || K < 1 || K > 2048) return 0;
  return csa2::sample_workspace_bytes(B, V, K);
}

int csa2_sample(const float* logits, int32_t B, int64_t V, int32_t K, float temperature, float top_p,
                const float* u, int32_t* token, float* prob, int32_t* n_kept, void* workspace,
                size_t workspace_bytes, csa2_stream_t stream) {
  if (B < 0 || V < 1 || V > 0x7FFFFFFFll) return CSA2_ERR_SHAPE;
  if (K < 1 || K > 2048 || !sampler_params_ok(temperature, top_p)) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!logits || !u || !token) return CSA2_ERR_NULL;
  if (!workspace) return CSA2_ERR_WORKSPACE;
  if (!aligned16(logits) || !aligned16(u) || !aligned16(token) || !opt_aligned16(prob) ||
      !opt_aligned16(n_kept) || !aligned16(workspace))
    return CSA2_ERR_ALIGN;
  if (workspace_bytes < csa2::sample_workspace_bytes(B, V, K)) return CSA2_ERR_WORKSPACE;
  if (too_large(csa2::topk_launch_items(B, V, K)) || too_large(csa2::sample_draw_launch_items(B)))
    return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_sample(logits, B, V, K, temperature, top_p, u, token, prob, n_kept, workspace,
                                        as_stream(stream)));
}

size_t csa2_sample_full_workspace_bytes(int32_t B, int64_t V) {
  if (B <= 0 || V < 1 || V > csa2::kSampleFullMaxVocab) return 0;
  return csa2::sample_full_workspace_bytes(B, V);
}

int csa2_sample_full(const float* logits, int32_t B, int64_t V, float temperature, const float* u, int32_t* token,
                     float* prob, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
  if (B < 0 || V < 1) return CSA2_ERR_SHAPE;
  if (V > csa2::kSampleFullMaxVocab || !sampler_params_ok(temperature, 1.0f)) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!logits || !u || !token) return CSA2_ERR_NULL;
  if (!aligned16(logits) || !aligned16(u) || !aligned16(token) || !opt_aligned16(prob)) return CSA2_ERR_ALIGN;
  if (!workspace || workspace_bytes < csa2::sample_full_workspace_bytes(B, V)) return CSA2_ERR_WORKSPACE;
  if (!aligned16(workspace)) return CSA2_ERR_ALIGN;
  if (too_large(csa2::sample_full_launch_items(B, V))) return CSA2_ERR_RANGE;
  return hip_status(csa2::launch_sample_full(logits, B, V, temperature, u, token, prob, workspace,
                                             as_stream(stream)));
}

size_t csa2_sparse_attn_workspace_bytes(int32_t B, int32_t H, int32_t d_c, int32_t K) {
  if (B <= 0 || H < 1 || H > 128 || K < 1 || d_c < 1) return 0;
  return csa2::attn_workspace_bytes(B, H, d_c, K);
}

// B queries; query b reads sequence b / qps (validated by the callers: qps >= 1, B % qps == 0).
static int sparse_attn_checked(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                               const uint8_t* scales, int64_t scales_stride, const uint16_t* rope,
                               int64_t rope_stride, const int32_t* idx, int32_t K, int32_t B, int32_t qps,
                               int32_t H, int32_t d_c, int32_t d_r, int64_t N_cap, float sm_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
  if (B < 0 || K < 1 || N_cap < 0 || codes_stride < 0 || scales_stride < 0 || rope_stride < 0)
    return CSA2_ERR_SHAPE;
  if (!((d_c == 128 || d_c == 512) && (d_r == 0 || d_r == 64)) || H < 1 || H > 128)
    return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!q || !codes || !scales || !idx || !out || (d_r > 0 && !rope)) return CSA2_ERR_NULL;
  if (!aligned16(q) || !aligned16(idx) || !aligned16(out) || !opt_aligned16(lse)) return CSA2_ERR_ALIGN;
  const int st = check_cache(d_c, d_r, codes, codes_stride, scales, scales_stride, rope, rope_stride);
  if (st != CSA2_OK) return st;
  // the kernel addresses a row inside its sequence with 32-bit offsets
  const int64_t lim = (int64_t)1 << 32;
  if (N_cap > 0 && (N_cap > lim / codes_stride || N_cap > lim / scales_stride ||
                    (d_r > 0 && N_cap > lim / rope_stride)))
    return CSA2_ERR_RANGE;
  if (too_large(csa2::attn_launch_items(B, H, d_c, K))) return CSA2_ERR_RANGE;
  const size_t need = csa2::attn_workspace_bytes(B, H, d_c, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return CSA2_ERR_ALIGN;
  const csa2::CacheRef c{const_cast<uint8_t*>(codes), codes_stride, const_cast<uint8_t*>(scales),
                         scales_stride, d_r > 0 ? const_cast<uint16_t*>(rope) : nullptr, rope_stride};
  return hip_status(csa2::launch_sparse_attn(q, c, idx, K, B, H, d_c, d_r, N_cap, qps, sm_scale, out, lse,
                                             workspace, as_stream(stream)));
}

int csa2_sparse_attn_fp4(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                         const uint8_t* scales, int64_t scales_stride, const uint16_t* rope,
                         int64_t rope_stride, const int32_t* idx, int32_t K, int32_t B, int32_t H,
                         int32_t d_c, int32_t d_r, int64_t N_cap, float sm_scale, float* out,
                         float* lse, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
  return sparse_attn_checked(q, codes, codes_stride, scales, scales_stride, rope, rope_stride, idx, K, B, 1, H,
                             d_c, d_r, N_cap, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

size_t csa2_sparse_swa_attn_workspace_bytes(int32_t B, int32_t H, int32_t d_c, int32_t K) {
  if (B <= 0 || H < 1 || H > 128 || d_c != 512 || K < 1) return 0;
  return csa2::sparse_swa_workspace_bytes(B, H, d_c, K);
}

int csa2_sparse_swa_attn_fp4(const uint16_t* q, const uint8_t* codes, int64_t codes_stride, const uint8_t* scales,
                             int64_t scales_stride, const uint16_t* rope, int64_t rope_stride, const int32_t* idx,
                             int32_t K, int32_t B, int32_t H, int32_t d_c, int32_t d_r, int64_t N_cap,
                             const uint8_t* w_codes, int64_t w_codes_stride, const float* w_sigma,
                             const uint16_t* w_rope, int64_t w_rope_stride, const int32_t* n_win, int32_t W_cap,
                             float sm_scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                             csa2_stream_t stream) {
  if (B < 0 || K < 1 || N_cap < 0 || codes_stride < 0 || scales_stride < 0 || rope_stride < 0 || W_cap < 0 ||
      w_codes_stride < 0 || w_rope_stride < 0)
    return CSA2_ERR_SHAPE;
  if (d_c != 512 || !(d_r == 0 || d_r == 64) || H < 1 || H > 128) return CSA2_ERR_UNSUPPORTED;
  if (W_cap > 256) return CSA2_ERR_RANGE;
  if (B == 0) return CSA2_OK;
  if (!q || !codes || !scales || !idx || !out || (d_r > 0 && !rope) ||
      (W_cap > 0 && (!w_codes || !w_sigma || (d_r > 0 && !w_rope))))
    return CSA2_ERR_NULL;
  if (w_codes_stride == 0) w_codes_stride = d_c;
  if (w_rope_stride == 0) w_rope_stride = 2 * (int64_t)d_r;
  if (w_codes_stride < d_c || (d_r > 0 && w_rope_stride < 2 * (int64_t)d_r)) return CSA2_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(idx) || !aligned16(out) || !opt_aligned16(lse) || !opt_aligned16(n_win) ||
      (W_cap > 0 && (!aligned16(w_codes) || w_codes_stride % 16 != 0 ||
                     (reinterpret_cast<uintptr_t>(w_sigma) & 3u) != 0 ||
                     (d_r > 0 && (!aligned16(w_rope) || w_rope_stride % 16 != 0)))))
    return CSA2_ERR_ALIGN;
  const int st = check_cache(d_c, d_r, codes, codes_stride, scales, scales_stride, rope, rope_stride);
  if (st != CSA2_OK) return st;
  // the kernels address a row inside its sequence with 32-bit offsets
  const int64_t lim = (int64_t)1 << 32;
  if (N_cap > 0 && (N_cap > lim / codes_stride || N_cap > lim / scales_stride ||
                    (d_r > 0 && N_cap > lim / rope_stride)))
    return CSA2_ERR_RANGE;
  if (too_large(csa2::attn_launch_items(B, H, d_c, K)) || too_large(csa2::swa_launch_items(B, H)))
    return CSA2_ERR_RANGE;
  const size_t need = csa2::sparse_swa_workspace_bytes(B, H, d_c, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return CSA2_ERR_ALIGN;
  const csa2::CacheRef c{const_cast<uint8_t*>(codes), codes_stride, const_cast<uint8_t*>(scales), scales_stride,
                         d_r > 0 ? const_cast<uint16_t*>(rope) : nullptr, rope_stride};
  const csa2::WinRef wr{W_cap > 0 ? w_codes : nullptr, w_codes_stride, w_sigma, d_r > 0 ? w_rope : nullptr,
                        w_rope_stride, n_win, W_cap};
  return hip_status(csa2::launch_sparse_swa_attn(q, c, idx, K, B, H, d_r, N_cap, wr, sm_scale, out, lse, workspace,
                                                 as_stream(stream)));
}

int csa2_prefill_sparse_attn_fp4(const uint16_t* q, const uint8_t* codes, int64_t codes_stride,
                                 const uint8_t* scales, int64_t scales_stride, const uint16_t* rope,
                                 int64_t rope_stride, const int32_t* idx, int32_t K, int32_t S, int32_t T,
                                 int32_t H, int32_t d_c, int32_t d_r, int64_t N_cap, float sm_scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes, csa2_stream_t stream) {
  if (S < 0 || T < 0) return CSA2_ERR_SHAPE;
  if ((int64_t)S * T > (1 << 24)) return CSA2_ERR_RANGE;
  if (S == 0 || T == 0) return CSA2_OK;
  return sparse_attn_checked(q, codes, codes_stride, scales, scales_stride, rope, rope_stride, idx, K, S * T, T,
                             H, d_c, d_r, N_cap, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"
