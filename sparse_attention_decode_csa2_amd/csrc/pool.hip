// Candidate-pool construction for the hierarchical indexer: the decoder's
// first Full layer keeps a block-level pool of at most 2048 blocks x 8
// positions, and the Reindex layers after it score only inside that pool
// ([P1] 架构三件套 - Hierarchical Sparse Indexer; [P4] CSA2 paragraph).
//
// The pages give no block score.  Block beta covers positions [block * beta,
// block * beta + block); it is a candidate when its first position is valid;
// its score is the largest Full-layer score among its valid positions (NaN
// ignored unless all are NaN).  The pool is the Top-K rule applied to blocks:
// the first min(P_max, #candidates) by (score descending, block id ascending).
//
// Two launches: one thread per block reduces its positions to the block score
// (contiguous, 16-byte loads when a block is a whole number of them), then the
// Top-K kernels select the blocks, with the per-row candidate count as their
// valid length.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

template <bool VEC4>
__global__ __launch_bounds__(256) void pool_block_max_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ n_valid, int64_t M,
                                                             int block, int64_t NB, int P_max,
                                                             float* __restrict__ block_scores,
                                                             int32_t* __restrict__ n_cand,
                                                             int32_t* __restrict__ n_blocks) {
  const int64_t chunks = (NB + 255) / 256;
  const int64_t b = blockIdx.x / chunks;
  const int64_t beta = (blockIdx.x - b * chunks) * 256 + threadIdx.x;
  const int64_t nv = n_valid ? min<int64_t>(max<int64_t>(n_valid[b], 0), M) : M;
  const int64_t nc = (nv + block - 1) / block;
  if (beta == 0) {
    n_cand[b] = (int32_t)nc;
    n_blocks[b] = (int32_t)min<int64_t>(nc, P_max);
  }
  if (beta >= NB) return;
  float m = -INFINITY;
  if (beta < nc) {
    const int64_t p0 = beta * block;
    const int64_t p1 = min<int64_t>(p0 + block, nv);
    const float* row = scores + b * M;
    m = row[p0];
    if (VEC4 && p1 - p0 == block) {
      // whole block: block / 4 aligned 16-byte loads
      for (int j = 0; j < block; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + p0 + j);
        m = fmaxf(fmaxf(m, v[0]), fmaxf(fmaxf(v[1], v[2]), v[3]));
      }
    } else {
      for (int64_t p = p0 + 1; p < p1; ++p) m = fmaxf(m, row[p]);
    }
  }
  block_scores[b * NB + beta] = m;
}

static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

size_t pool_workspace_bytes(int B, int64_t M, int block, int P_max) {
  const int64_t NB = (M + block - 1) / block;
  return align16((size_t)B * NB * sizeof(float)) + align16((size_t)B * sizeof(int32_t)) +
         topk_workspace_bytes(B, NB, P_max);
}

int64_t pool_launch_items(int B, int64_t M, int block, int P_max) {
  const int64_t NB = (M + block - 1) / block;
  const int64_t reduce = (int64_t)B * ((NB + 255) / 256) * 256;
  return reduce > topk_launch_items(B, NB, P_max) ? reduce : topk_launch_items(B, NB, P_max);
}

hipError_t launch_build_pool(const float* scores, const int32_t* n_valid, int B, int64_t M, int block,
                             int P_max, int32_t* pool_blocks, int32_t* n_blocks, void* workspace,
                             hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int64_t NB = (M + block - 1) / block;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* block_scores = reinterpret_cast<float*>(ws);
  int32_t* n_cand = reinterpret_cast<int32_t*>(ws + align16((size_t)B * NB * sizeof(float)));
  void* topk_ws = ws + align16((size_t)B * NB * sizeof(float)) + align16((size_t)B * sizeof(int32_t));
  const int64_t chunks = (NB + 255) / 256;
  const dim3 grid((unsigned)(B * chunks));
  // 16-byte loads need every row and every block to start on a 16-byte boundary
  const bool vec4 = block % 4 == 0 && M % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
  if (vec4)
    hipLaunchKernelGGL(pool_block_max_kernel<true>, grid, dim3(256), 0, stream, scores, n_valid, M, block, NB,
                       P_max, block_scores, n_cand, n_blocks);
  else
    hipLaunchKernelGGL(pool_block_max_kernel<false>, grid, dim3(256), 0, stream, scores, n_valid, M, block, NB,
                       P_max, block_scores, n_cand, n_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk(block_scores, nullptr, n_cand, B, NB, P_max, pool_blocks, nullptr, topk_ws, stream);
}

}  // namespace csa2
