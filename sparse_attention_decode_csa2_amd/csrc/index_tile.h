// Indexer tile scoring, shared by the indexer kernels (index.hip) and the
// fused indexer + Top-K chunk kernel (index_topk.hip), so that both compute
// every score with the same instructions in the same order:
//   score[b, n] = sum_h w[b, h] * max(0, q_idx[b, h, :] . k_idx[b, n, :])
// ([P1] 架构三件套 - CSA2 and Hierarchical Sparse Indexer; [P4] CSA2 paragraph).
//
// One wave scores a tile of 16 keys: one v_mfma_f32_16x16x32_bf16 per 32 key
// dimensions computes a 16 (heads, padded with zero rows) x 16 (keys) tile.
// For k-step s, lane (key l % 16, group l / 16) supplies dimensions
// 32s + 8 (l / 16) .. +7 of its key; the query is laid out the same way, the
// MFMA's own k order.  The epilogue applies ReLU and the head weights (heads
// 4g .. 4g + 3 in order) and adds the four head quarters across lane groups
// (xor 16, then xor 32), leaving the key's score in every lane of its column.
#pragma once

#include "csa2_device.h"

namespace csa2 {

// A operand (query head n = lane % 16, rows >= H_I zero; dims of quarter
// g = lane / 16) and the weights of the four heads whose dot products the
// lane receives (w == nullptr: all ones).
template <int KS>
__device__ __forceinline__ void index_query(const uint16_t* __restrict__ q, const float* __restrict__ w, int64_t b,
                                            int H_I, int lane, bf16x8 (&A)[KS], float (&wv)[4]) {
  constexpr int D_I = 32 * KS;
  const int n = lane & 15, g = lane >> 4;
  const uint16_t* qrow = q + (b * H_I + n) * D_I + 8 * g;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < H_I) v = *reinterpret_cast<const u32x4*>(qrow + 32 * s);
    A[s] = __builtin_bit_cast(bf16x8, v);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    wv[i] = h < H_I ? (w ? w[b * H_I + h] : 1.0f) : 0.0f;
  }
}

// A tile loaded contiguously (load s holds 16-byte word 64 s + lane of the
// tile's 16 keys, i.e. word (64 s + lane) % KW of key (64 s + lane) / KW) into
// the MFMA layout (lane (n, g) needs word 4 s + g of key n) through the
// wave's LDS buffer kb of 16 * (KW + 1) words (rows padded by one word: the
// stores and the operand reads hit distinct banks).
template <int KS>
__device__ __forceinline__ void index_reorder(const u32x4 (&Bv)[KS], u32x4* kb, int lane, u32x4 (&Bt)[KS]) {
  constexpr int KW = 4 * KS;  // 16-byte words per key
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int w = 64 * s + lane;
    kb[(w / KW) * (KW + 1) + w % KW] = Bv[s];
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) Bt[s] = kb[n * (KW + 1) + 4 * s + g];
}

// Score of key lane % 16 of the tile whose MFMA operand words are Bt.
template <int KS>
__device__ __forceinline__ float index_tile_score(const bf16x8 (&A)[KS], const float (&wv)[4], const u32x4 (&Bt)[KS]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) acc = mfma16x16x32_bf16(A[s], __builtin_bit_cast(bf16x8, Bt[s]), acc);
  // acc[i] = dot(head 4g + i, key n of this tile)
  float part = wv[0] * fmaxf(acc[0], 0.f);
  part += wv[1] * fmaxf(acc[1], 0.f);
  part += wv[2] * fmaxf(acc[2], 0.f);
  part += wv[3] * fmaxf(acc[3], 0.f);
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  return part;
}

}  // namespace csa2
