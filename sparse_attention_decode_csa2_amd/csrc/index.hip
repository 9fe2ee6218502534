// a1 / a2: indexer scoring (Full mode over every entry, Reindex mode over the
// candidate pool).
//
// score[b, n] = sum_h w[b, h] * max(0, q_idx[b, h, :] . k_idx[b, n, :])
// ([P1] 架构三件套 - CSA2 and Hierarchical Sparse Indexer; [P4] CSA2 paragraph;
// the ReLU-gated multi-head form is the reading documented in the header).
//
// The multi-head q . K contraction of a 16-key tile runs on the matrix cores
// (index_tile.h).  A wave's tiles hold 16 whole keys (contiguous in Full
// mode, two 8-entry runs per tile in pool mode).  Full mode loads the 16 keys
// contiguously and reorders them through LDS (see below); pool mode with the
// pool's 8-position blocks runs index_pool8_kernel (eight tiles per wave,
// the block ids in one vector load, the next tile's keys in flight); other
// block sizes load contiguously when their blocks allow it, else each lane's
// operand directly.
//
// HBM-bound: 2*D_I bytes of key per scored entry against 4*H_I*D_I flops
// (8 flop/byte at H_I = 8): the matrix cores only have to keep up with HBM.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "index_tile.h"

namespace csa2 {

// BLK: positions per pool block known at compile time (the 8-position blocks of
// the candidate pool: the block lookups become shifts), 0 = the runtime `block`.
template <int KS, int TPW, bool POOL, int BLK>
__global__ __launch_bounds__(256) void index_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ n_valid, int H_I, int64_t N_cap, const int32_t* __restrict__ pool,
    const int32_t* __restrict__ n_blocks, int P_max, int block, int64_t M, int64_t wg_per_row,
    float* __restrict__ scores, int32_t* __restrict__ positions) {
  constexpr int D_I = 32 * KS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bsz = BLK > 0 ? (uint64_t)BLK : (uint64_t)block;  // columns are non-negative
  const int n = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.x / wg_per_row;
  const int64_t wg = blockIdx.x - b * wg_per_row;

  bf16x8 A[KS];
  float wv[4];
  index_query<KS>(q, w, b, H_I, lane, A, wv);
  int64_t nv = N_cap;
  if (n_valid) nv = min<int64_t>(max<int64_t>(n_valid[b], 0), N_cap);
  int nb = 0;
  if (POOL) nb = min(max(n_blocks[b], 0), P_max);

  // Key column col of the row -> cache position and validity (pool mode:
  // position 8 * pool[col / 8] + col % 8).
  auto locate = [&](int64_t col, int64_t* p_out) {
    int64_t p = col;
    bool valid;
    if (POOL) {
      const int64_t i = (int64_t)((uint64_t)col / bsz);
      const int j = (int)(col - i * (int64_t)bsz);
      const int64_t blk = (col < M && i < nb) ? (int64_t)pool[b * P_max + i] : -1;
      p = blk * (int64_t)bsz + j;
      valid = blk >= 0 && p < nv;
    } else {
      valid = col < nv;
    }
    *p_out = p;
    return valid;
  };
  // Keys are read contiguously: load s of a tile brings 16-byte word
  // 64 s + lane of the tile's 16 keys (key (64 s + lane) / KW, word
  // (64 s + lane) % KW of it), so a wave-wide load covers whole cache lines,
  // and a wave-private LDS buffer turns the tile into the MFMA layout, where
  // lane (n, g) needs word 4 s + g of key n (rows padded by one word: the
  // stores and the operand reads hit distinct banks).  Measured: 6.25 against
  // 5.46 TB/s for loads straight into the MFMA layout, whose wave-wide loads
  // touch twice the cache lines, half of each.  In pool mode a load's keys
  // must then sit in one block (block a multiple of the keys per load), so
  // that one wave-uniform block lookup serves the load; other block sizes
  // load each lane's operand directly, one lookup per key.
  constexpr int KW = D_I / 8;                 // 16-byte words per key
  static_assert(16 * KW == 64 * KS, "a tile is KS wave-wide loads");
  constexpr int KPL = 64 / KW;                // keys per wave-wide load
  // contiguous loads in pool mode when every load's keys sit in one block
  // (8-position blocks and 128-dimension keys: 4 keys per load): then a
  // load needs one block id, the same for the whole wave
  const bool contig = !POOL || bsz % KPL == 0;
  __shared__ u32x4 kbuf[4][16 * (KW + 1)];
  u32x4* kb = kbuf[wave];
  const int64_t tile0 = (int64_t)(wg * 4 + __builtin_amdgcn_readfirstlane(wave)) * TPW;
  u32x4 Bv[TPW][KS];
  int64_t pos[TPW];
  bool ok[TPW];
  uint32_t vmask[TPW];  // bit s: load s of tile t holds a key
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    vmask[t] = 0u;
    ok[t] = locate((tile0 + t) * 16 + n, &pos[t]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint16_t* kp;
      bool valid;
      const int w = 64 * s + lane;
      if (POOL && !contig) {
        valid = ok[t];
        kp = k + (b * N_cap + (valid ? pos[t] : 0)) * D_I + 8 * g + 32 * s;
      } else if (POOL) {
        // block of keys 16 t' + KPL s .. (wave-uniform), then the lane's key in it
        const int64_t c0 = (tile0 + t) * 16 + KPL * s;
        const int64_t i = (int64_t)((uint64_t)c0 / bsz);
        const int64_t blk = (c0 < M && i < nb) ? (int64_t)pool[b * P_max + i] : -1;
        const int64_t p = blk * (int64_t)bsz + (c0 - i * (int64_t)bsz) + lane / KW;
        valid = blk >= 0 && p < nv;
        kp = k + (b * N_cap + (valid ? p : 0)) * D_I + 8 * (w % KW);
      } else {
        int64_t p;
        valid = locate((tile0 + t) * 16 + w / KW, &p);
        kp = k + (b * N_cap + (valid ? p : 0)) * D_I + 8 * (w % KW);
      }
      // unconditional (an empty slot reads key 0 of the row, zeroed where
      // it is used), so that every load is in flight before the first is used
      Bv[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp));
      vmask[t] |= (uint32_t)valid << s;
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (!((vmask[t] >> s) & 1u)) Bv[t][s] = u32x4{0u, 0u, 0u, 0u};
    u32x4 Bt[KS];
    if (POOL && !contig) {
#pragma unroll
      for (int s = 0; s < KS; ++s) Bt[s] = Bv[t][s];
    } else {
      index_reorder<KS>(Bv[t], kb, lane, Bt);
    }
    const float part = index_tile_score<KS>(A, wv, Bt);
    const int64_t col = (tile0 + t) * 16 + n;
    if (g == 0 && col < M) {
      scores[b * M + col] = ok[t] ? part : -INFINITY;
      if (POOL) positions[b * M + col] = ok[t] ? (int32_t)pos[t] : -1;
    }
  }
}

// Pool mode with the candidate pool's 8-position blocks (a 16-key tile is two
// whole blocks) and keys of 64 dimensions or more: one wave scores POOL_TW
// consecutive tiles.  It loads the block ids of all its tiles with one vector
// load (block 2 t + l of its tiles in lane l) and takes each with a lane read,
// loads its query operand once, and keeps the next tile's key loads in flight
// while it scores a tile.  The loads and the LDS reorder are the contiguous
// ones of index_kernel (KPL keys of one block per wave-wide load).
// Measured on the 32 x 2048-block pool over 262144 entries: 27.0 us against
// 28.5 with 4 tiles per wave, 29.9 with 16, 28.9 for the 4-wave grid of
// index_kernel (two tiles per wave), and 31.4 with two tiles in flight.
constexpr int POOL_TW = 8;
static_assert(2 * POOL_TW <= 64, "a wave's block ids fit one vector register");

template <int KS>
__global__ __launch_bounds__(256) void index_pool8_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ n_valid, int H_I, int64_t N_cap, const int32_t* __restrict__ pool,
    const int32_t* __restrict__ n_blocks, int P_max, int64_t M, int64_t wg_per_row, float* __restrict__ scores,
    int32_t* __restrict__ positions) {
  constexpr int D_I = 32 * KS;
  constexpr int KW = D_I / 8;   // 16-byte words per key
  constexpr int KPL = 64 / KW;  // keys per wave-wide load
  static_assert(8 % KPL == 0, "a wave-wide load stays in one 8-position block");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.x / wg_per_row;
  const int64_t wg = blockIdx.x - b * wg_per_row;
  bf16x8 A[KS];
  float wv[4];
  index_query<KS>(q, w, b, H_I, lane, A, wv);
  int64_t nv = N_cap;
  if (n_valid) nv = min<int64_t>(max<int64_t>(n_valid[b], 0), N_cap);
  const int64_t nb = min(max(n_blocks[b], 0), P_max);
  const int64_t tile0 = (wg * 4 + wave) * POOL_TW;
  int blk_l = -1;  // block id of pool slot 2 tile0 + lane (-1: empty slot)
  if (lane < 2 * POOL_TW && 2 * tile0 + lane < nb) blk_l = pool[b * P_max + 2 * tile0 + lane];
  __shared__ u32x4 kbuf[4][16 * (KW + 1)];
  u32x4* kb = kbuf[wave];
  const uint16_t* krow = k + b * N_cap * D_I;
  // load s of the wave's tile t: keys KPL s .. of the tile, in block 2 t + KPL
  // s / 8.  Unconditional (an empty slot reads key 0 of the row; bit s of vm
  // clear, zeroed where it is used), so that the next tile's loads stay in
  // flight while a tile is scored.
  auto load = [&](int t, u32x4 (&Bv)[KS], uint32_t& vm) {
    vm = 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = KPL * s;
      const int64_t blk = __builtin_amdgcn_readlane(blk_l, 2 * t + c / 8);
      const int64_t p = blk * 8 + c % 8 + lane / KW;
      const bool valid = blk >= 0 && p < nv;
      Bv[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + (valid ? p : 0) * D_I + 8 * (lane % KW)));
      vm |= (uint32_t)valid << s;
    }
  };
  u32x4 cur[KS];
  uint32_t cur_m;
  load(0, cur, cur_m);
  for (int t = 0; t < POOL_TW; ++t) {
    const int64_t tile = tile0 + t;
    if (tile * 16 >= M) break;
    const bool more = t + 1 < POOL_TW && (tile + 1) * 16 < M;
    u32x4 nxt[KS];
    uint32_t nxt_m = 0u;
    if (more) load(t + 1, nxt, nxt_m);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (!((cur_m >> s) & 1u)) cur[s] = u32x4{0u, 0u, 0u, 0u};
    u32x4 Bt[KS];
    index_reorder<KS>(cur, kb, lane, Bt);
    const float part = index_tile_score<KS>(A, wv, Bt);
    const int64_t col = tile * 16 + n;
    if (g == 0 && col < M) {
      const int blk_a = __builtin_amdgcn_readlane(blk_l, 2 * t), blk_b = __builtin_amdgcn_readlane(blk_l, 2 * t + 1);
      const int64_t blk = n < 8 ? blk_a : blk_b;
      const int64_t p = blk * 8 + (n & 7);
      const bool ok = blk >= 0 && p < nv;
      scores[b * M + col] = ok ? part : -INFINITY;
      positions[b * M + col] = ok ? (int32_t)p : -1;
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < KS; ++s) cur[s] = nxt[s];
      cur_m = nxt_m;
    }
  }
}

// Grid of index_kernel: 16-key tiles, four waves per workgroup, `tpw` tiles
// per wave.  Tiles per wave, measured: Full mode is fastest with one (its
// contiguous loads keep enough in flight; prefill-full-1m 80.6 us against
// 86.7 with four); pool mode (blocks other than 8 positions, or 32-dimension
// keys), whose loads wait for block lookups, with two once the grid fills the
// GPU (the 2048 x 8 pool: 28.7 us against 30.4 with four).
static void index_grid(int B, int64_t M, bool pool, int* tpw, int64_t* wg_per_row) {
  const int64_t tiles_per_row = (M + 15) / 16;
  const int64_t total_tiles = tiles_per_row * B;
  *tpw = (pool && total_tiles >= 2 * 4 * 2048) ? 2 : 1;
  *wg_per_row = (tiles_per_row + 4 * *tpw - 1) / (4 * *tpw);
}

int64_t index_launch_items(int B, int64_t M, bool pool, int block, int D_I) {
  if (pool && block == 8 && D_I >= 64) {
    const int64_t tiles = (M + 15) / 16;
    return (tiles + 4 * POOL_TW - 1) / (4 * POOL_TW) * B * 256;
  }
  int tpw;
  int64_t wpr;
  index_grid(B, M, pool, &tpw, &wpr);
  return wpr * B * 256;
}

template <int KS, bool POOL>
static hipError_t launch_index_ks(const uint16_t* q, const float* w, const uint16_t* k,
                                  const int32_t* n_valid, int B, int H_I, int64_t N_cap,
                                  const int32_t* pool, const int32_t* n_blocks, int P_max, int block,
                                  int64_t M, float* scores, int32_t* positions, hipStream_t stream) {
  int tpw;
  int64_t wg_per_row;
  index_grid(B, M, POOL, &tpw, &wg_per_row);
  const dim3 grid((unsigned)(wg_per_row * B)), blk(256);
#define CSA2_IDX_LAUNCH(T, BL)                                                                          \
  hipLaunchKernelGGL((index_kernel<KS, T, POOL, BL>), grid, blk, 0, stream, q, w, k, n_valid, H_I, N_cap, \
                     pool, n_blocks, P_max, block, M, wg_per_row, scores, positions)
  if constexpr (POOL && KS >= 2) {
    if (block == 8) {
      const int64_t tiles = (M + 15) / 16, wpr = (tiles + 4 * POOL_TW - 1) / (4 * POOL_TW);
      hipLaunchKernelGGL((index_pool8_kernel<KS>), dim3((unsigned)(wpr * B)), blk, 0, stream, q, w, k, n_valid,
                         H_I, N_cap, pool, n_blocks, P_max, M, wpr, scores, positions);
      return hipGetLastError();
    }
  }
  if (POOL && block == 8) {
    if (tpw == 2) CSA2_IDX_LAUNCH(2, 8);
    else CSA2_IDX_LAUNCH(1, 8);
  } else {
    if (tpw == 2) CSA2_IDX_LAUNCH(2, 0);
    else CSA2_IDX_LAUNCH(1, 0);
  }
#undef CSA2_IDX_LAUNCH
  return hipGetLastError();
}

hipError_t launch_index(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* n_valid,
                        int B, int H_I, int D_I, int64_t N_cap, const int32_t* pool,
                        const int32_t* n_blocks, int P_max, int block, float* scores,
                        int32_t* positions, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const bool is_pool = pool != nullptr;
  const int64_t M = is_pool ? (int64_t)P_max * block : N_cap;
  if (M == 0) return hipSuccess;
#define CSA2_IDX_KS(KS)                                                                              \
  return is_pool ? launch_index_ks<KS, true>(q, w, k, n_valid, B, H_I, N_cap, pool, n_blocks, P_max, \
                                             block, M, scores, positions, stream)                    \
                 : launch_index_ks<KS, false>(q, w, k, n_valid, B, H_I, N_cap, pool, n_blocks, P_max, \
                                              block, M, scores, positions, stream)
  switch (D_I) {
    case 32: CSA2_IDX_KS(1);
    case 64: CSA2_IDX_KS(2);
    case 128: CSA2_IDX_KS(4);
    case 256: CSA2_IDX_KS(8);
    default: return hipErrorInvalidValue;
  }
#undef CSA2_IDX_KS
}

}  // namespace csa2
