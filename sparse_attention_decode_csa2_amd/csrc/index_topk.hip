// a1 + a3 fused, Full mode: the indexer scores of a sequence and their Top-K
// with the lower id winning ties, without the scores going through HBM
// ([P1] 架构三件套 - CSA2 (Top-512 over the indexer scores) and Hierarchical
// Sparse Indexer; [P4] CSA2 paragraph).  The result is, bit for bit, that of
// csa2_index_full followed by csa2_topk with the same n_valid.
//
// One workgroup of 1024 threads owns a chunk of 8192 consecutive entries of
// one sequence:
//  1. its 16 waves stream the chunk's index keys, wave w scoring the 16-key
//     tiles w, w + 16, ... with the indexer's own tile code (index_tile.h),
//     the loads of the next tile in flight while a tile is scored; the
//     scores go to LDS;
//  2. the block-level Top-K (topk_block.h) keeps the chunk's K best keys,
//     written unsorted to the workspace as the first level's chunk winners;
// and the Top-K's later levels (topk.hip) reduce the winners of each row.
//
// Streaming the key cache needs about one workgroup per CU: measured, a grid
// of 256 workgroups, each reading its own contiguous 2 MiB, reads 537 MB at
// 6.7-6.8 TB/s, as fast as a grid of thousands, and 128 workgroups only reach
// 5.8 TB/s.  Rows with fewer chunks than that go through the separate
// indexer (a grid of 4-wave workgroups) and Top-K kernels instead; the result
// is the same.
#include "csa2_internal.h"
#include "index_tile.h"
#include "topk_block.h"

namespace csa2 {

constexpr int IT_KEYS = TK_T * TK_E / 2;         // entries per chunk: 8192
constexpr int IT_TILES = IT_KEYS / 16;           // 16-key tiles per chunk
constexpr int IT_TPW = IT_TILES / TK_WAVES;      // tiles per wave
constexpr int IT_MIN_GROUPS = 256;               // fused only with a workgroup per CU
static_assert(IT_TILES % TK_WAVES == 0, "every wave scores the same number of tiles");

template <int KS>
__global__ __launch_bounds__(TK_T) void index_topk_kernel(const uint16_t* __restrict__ q,
                                                          const float* __restrict__ w,
                                                          const uint16_t* __restrict__ k,
                                                          const int32_t* __restrict__ n_valid, int H_I,
                                                          int64_t N_cap, int K, int chunks,
                                                          uint64_t* __restrict__ keys_out) {
  constexpr int D_I = 32 * KS;
  constexpr int KW = D_I / 8;  // 16-byte words per key
  // the tile buffers are dead once the scores are in LDS: the Top-K reuses them
  union Smem {
    TkSmem tk;
    u32x4 kbuf[TK_WAVES][16 * (KW + 1)];
  };
  __shared__ Smem sm;
  __shared__ float sc[IT_KEYS];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.x / chunks;
  const int c = (int)(blockIdx.x - b * chunks);
  const int64_t base = (int64_t)c * IT_KEYS;
  int64_t nv = N_cap;
  if (n_valid) nv = min<int64_t>(max<int64_t>(n_valid[b], 0), N_cap);
  const int64_t limit = min<int64_t>(nv, base + IT_KEYS);  // columns base .. limit-1 are candidates

  // ---- 1. scores of the chunk's valid columns into sc
  {
    bf16x8 A[KS];
    float wv[4];
    index_query<KS>(q, w, b, H_I, lane, A, wv);
    const uint16_t* krow = k + b * N_cap * D_I;
    u32x4* kb = sm.kbuf[wave];
    // load s of tile t: word 64 s + lane of its 16 keys; keys past limit not read
    auto load = [&](int t, u32x4 (&Bv)[KS]) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int wd = 64 * s + lane;
        const int64_t col = base + 16 * t + wd / KW;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (col < limit)
          v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + col * D_I + 8 * (wd % KW)));
        Bv[s] = v;
      }
    };
    u32x4 cur[KS];
    load(wave, cur);
    for (int i = 0; i < IT_TPW; ++i) {
      const int t = wave + TK_WAVES * i;
      const bool more = i + 1 < IT_TPW;
      u32x4 nxt[KS];
      if (more) load(t + TK_WAVES, nxt);
      if (base + 16 * t < limit) {  // wave-uniform: a tile wholly past limit is never a candidate
        u32x4 Bt[KS];
        index_reorder<KS>(cur, kb, lane, Bt);
        const float part = index_tile_score<KS>(A, wv, Bt);
        if (g == 0) sc[16 * t + n] = part;
      }
      if (more) {
#pragma unroll
        for (int s = 0; s < KS; ++s) cur[s] = nxt[s];
      }
    }
  }
  __syncthreads();

  // ---- 2. the chunk's K best keys: thread t holds columns base + 16 t .. + 15
  tk_init(sm.tk);
  constexpr int HALF = TK_T / 2;  // threads holding the chunk's 16-column runs
  float v[TK_E];
  uint32_t idv[TK_E];
  lanemask valid = 0;
  const int64_t col0 = base + (int64_t)TK_E * tid;
#pragma unroll
  for (int e = 0; e < TK_E; ++e) {
    const int64_t col = col0 + e;
    const bool ok = tid < HALF && col < limit;
    v[e] = ok ? sc[tid < HALF ? TK_E * tid + e : 0] : __uint_as_float(F_NAN);
    idv[e] = (uint32_t)col;
    valid |= (lanemask)ok << e;
  }
  TkDst dst;
  dst.idx = nullptr;
  dst.score = nullptr;
  dst.keys = keys_out + (b * chunks + c) * (int64_t)K;
  const uint32_t count = block_select<false>(v, idv, valid, true, K, dst, sm.tk);
  if (count == TK_WRITTEN) return;
  for (int j = tid; j < K; j += TK_T) dst.keys[j] = j < (int)count ? sm.tk.buf[j] : 0ull;
}

static int64_t it_chunks(int64_t N_cap) { return (N_cap + IT_KEYS - 1) / IT_KEYS; }

static bool it_fused(int B, int D_I, int64_t N_cap) {
  return D_I <= 128 && (int64_t)B * it_chunks(N_cap) >= IT_MIN_GROUPS;
}

int64_t index_topk_launch_items(int B, int D_I, int64_t N_cap, int K) {
  if (!it_fused(B, D_I, N_cap)) {
    const int64_t a = index_launch_items(B, N_cap, false, 1, D_I), t = topk_launch_items(B, N_cap, K);
    return a > t ? a : t;
  }
  return (int64_t)B * it_chunks(N_cap) * TK_T;
}

// Fused: the chunk winners (B x chunks x K keys, 16-byte aligned) and the
// later levels' workspace.  Separate: the scores (B x N_cap floats, rounded
// up to 16 bytes) and the Top-K workspace.
size_t index_topk_workspace_bytes(int B, int D_I, int64_t N_cap, int K) {
  if (!it_fused(B, D_I, N_cap)) {
    const size_t s = ((size_t)B * N_cap * sizeof(float) + 15) & ~(size_t)15;
    return s + topk_workspace_bytes(B, N_cap, K);
  }
  const int64_t m = it_chunks(N_cap) * K;
  return (size_t)B * m * sizeof(uint64_t) + topk_keys_workspace_bytes(B, m, K);
}

hipError_t launch_index_topk(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* n_valid, int B,
                             int H_I, int D_I, int64_t N_cap, int K, int32_t* out_idx, float* out_score,
                             void* workspace, hipStream_t stream, const Fp4Append* app) {
  if (B == 0) return app ? launch_quantize_fp4(app->x, app->n_rows, app->d_c, app->rope_src, app->d_r, app->cache,
                                               app->dst_row0, stream)
                         : hipSuccess;
  if (!it_fused(B, D_I, N_cap)) {
    // the two-kernel path has no idle final level: the append goes first
    if (app) {
      const hipError_t e = launch_quantize_fp4(app->x, app->n_rows, app->d_c, app->rope_src, app->d_r, app->cache,
                                               app->dst_row0, stream);
      if (e != hipSuccess) return e;
    }
    float* scores = static_cast<float*>(workspace);
    const size_t s = ((size_t)B * N_cap * sizeof(float) + 15) & ~(size_t)15;
    hipError_t e = launch_index(q, w, k, n_valid, B, H_I, D_I, N_cap, nullptr, nullptr, 0, 1, scores, nullptr,
                                stream);
    if (e != hipSuccess) return e;
    return launch_topk(scores, nullptr, n_valid, B, N_cap, K, out_idx, out_score,
                       static_cast<uint8_t*>(workspace) + s, stream);
  }
  const int chunks = (int)it_chunks(N_cap);
  uint64_t* keys = static_cast<uint64_t*>(workspace);
  const int64_t m = (int64_t)chunks * K;
  const dim3 grid((unsigned)((int64_t)B * chunks)), blk(TK_T);
  switch (D_I) {
    case 32: hipLaunchKernelGGL((index_topk_kernel<1>), grid, blk, 0, stream, q, w, k, n_valid, H_I, N_cap, K, chunks, keys); break;
    case 64: hipLaunchKernelGGL((index_topk_kernel<2>), grid, blk, 0, stream, q, w, k, n_valid, H_I, N_cap, K, chunks, keys); break;
    case 128: hipLaunchKernelGGL((index_topk_kernel<4>), grid, blk, 0, stream, q, w, k, n_valid, H_I, N_cap, K, chunks, keys); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_from_keys(keys, B, m, K, out_idx, out_score, keys + (size_t)B * m, stream, app);
}

}  // namespace csa2
