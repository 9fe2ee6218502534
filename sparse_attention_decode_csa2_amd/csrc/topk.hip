// a3: Top-K with the lower id winning ties (Top-512 per [P1] 架构三件套, CSA2):
// the kernels of the chunked reduction over the block-level selection of
// topk_block.h.
#include "csa2_internal.h"
#include "quantize_task.h"
#include "topk_block.h"

namespace csa2 {

// One workgroup's selection: chunk `blk` of the level (row blk / chunks).
template <bool FROM_SCORES, bool FINAL>
__device__ __forceinline__ void topk_body(TkSmem& sm, int64_t blk, const float* __restrict__ scores,
                                          const int32_t* __restrict__ ids, const int32_t* __restrict__ n_valid,
                                          const uint64_t* __restrict__ keys_in, int64_t M, int K, int chunks,
                                          uint64_t* __restrict__ keys_out, int32_t* __restrict__ out_idx,
                                          float* __restrict__ out_score) {
  const int tid = threadIdx.x;
  tk_init(sm);
  const int64_t b = blk / chunks;
  const int c = (int)(blk - b * chunks);
  const int64_t base = (int64_t)c * TK_CHUNK;
  int64_t limit = min<int64_t>(M, base + TK_CHUNK);
  const int64_t col0 = base + (int64_t)TK_E * tid;  // this thread's first score column
  // element e: score v[e] (NaN when empty), id idv[e], valid bit e
  float v[TK_E];
  uint32_t idv[TK_E];
  lanemask valid = 0;
  const float qnan = __uint_as_float(F_NAN);
  bool ids_are_columns;
  // every load is issued before any result is used: a load under a
  // per-element branch would wait for the one before it
  if (FROM_SCORES) {
    // thread t holds the TK_E consecutive columns from col0 (thread order is
    // column order)
    if (n_valid) limit = min<int64_t>(limit, max<int64_t>(n_valid[b], 0));
    ids_are_columns = ids == nullptr;
    const float* srow = scores + b * M;
    const int32_t* irow = ids ? ids + b * M : nullptr;
    float x[TK_E];
    uint32_t ii[TK_E];
    if (col0 + TK_E <= limit && (M & 3) == 0) {
      // a whole run of columns: 16-byte loads (rows stay 16-byte aligned)
      f32x4 v4[TK_E / 4];
      u32x4 i4[TK_E / 4];
#pragma unroll
      for (int q = 0; q < TK_E / 4; ++q) v4[q] = *reinterpret_cast<const f32x4*>(srow + col0 + 4 * q);
      if (irow) {
#pragma unroll
        for (int q = 0; q < TK_E / 4; ++q) i4[q] = *reinterpret_cast<const u32x4*>(irow + col0 + 4 * q);
      }
#pragma unroll
      for (int e = 0; e < TK_E; ++e) {
        x[e] = v4[e / 4][e % 4];
        ii[e] = irow ? i4[e / 4][e % 4] : (uint32_t)(col0 + e);
      }
    } else {
      // columns past the end read the last column in range (column 0 of an
      // empty row) and are then dropped
      const int64_t last = limit > 0 ? limit - 1 : 0;
#pragma unroll
      for (int e = 0; e < TK_E; ++e) {
        const int64_t cc = min<int64_t>(col0 + e, last);
        x[e] = srow[cc];
        ii[e] = irow ? (uint32_t)irow[cc] : (uint32_t)(col0 + e);
      }
#pragma unroll
      for (int e = 0; e < TK_E; ++e) ii[e] = col0 + e < limit ? ii[e] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      const bool ok = ii[e] != 0xFFFFFFFFu;
      idv[e] = ii[e];
      v[e] = ok ? x[e] : qnan;
      valid |= (lanemask)ok << e;
    }
  } else {
    // keys are held lane-contiguously: element e of thread t is key base +
    // 2 (TK_T (e / 2) + t) + e % 2, so that each 16-byte load instruction
    // reads 1 KiB of consecutive keys (8 cache lines, not 64).  Which thread
    // holds a key does not matter: keys are unique up to identical (score,
    // id) pairs, and ties between those are invisible in the output
    ids_are_columns = false;
    const uint64_t* krow = keys_in + b * M;
    auto pos = [&](int e) { return base + 2 * ((int64_t)TK_T * (e >> 1) + tid) + (e & 1); };
    uint64_t k[TK_E];
    if ((M & 1) == 0) {
      // 16-byte loads (rows stay 16-byte aligned), clamped to the row's last
      // word: the keys of a clamped word all lie past the row, hence past limit
#pragma unroll
      for (int q = 0; q < TK_E / 2; ++q) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(krow + min<int64_t>(pos(2 * q), M - 2));
        k[2 * q] = ((uint64_t)w[1] << 32) | w[0];
        k[2 * q + 1] = ((uint64_t)w[3] << 32) | w[2];
      }
    } else {
      // keys past the end read the last key in range and are then dropped
      const int64_t last = limit > 0 ? limit - 1 : 0;
#pragma unroll
      for (int e = 0; e < TK_E; ++e) k[e] = krow[min<int64_t>(pos(e), last)];
    }
#pragma unroll
    for (int e = 0; e < TK_E; ++e) k[e] = pos(e) < limit ? k[e] : 0ull;
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      const uint32_t hk = (uint32_t)(k[e] >> 32);
      idv[e] = ~(uint32_t)k[e];
      v[e] = hk != 0 ? key_score(hk) : qnan;
      valid |= (lanemask)(hk != 0) << e;
    }
  }
  TkDst dst;
  dst.idx = FINAL ? out_idx + b * K : nullptr;
  dst.score = FINAL && out_score ? out_score + b * K : nullptr;
  dst.keys = FINAL ? nullptr : keys_out + (b * chunks + c) * (int64_t)K;
  const uint32_t count = block_select<FINAL>(v, idv, valid, ids_are_columns, K, dst, sm);
  if (count == TK_WRITTEN) return;
  if (FINAL) {
    // sort the selected keys descending: (score desc, id asc)
    if (count > 1) {
      int n = 64;
      while (n < (int)count) n <<= 1;
      for (int j = (int)count + tid; j < n; j += TK_T) sm.buf[j] = 0ull;
      sort_desc_n(n, sm);
    }
    for (int j = tid; j < K; j += TK_T) {
      const bool ok = j < (int)count;
      const uint64_t k = ok ? sm.buf[j] : 0ull;
      out_idx[b * K + j] = ok ? (int32_t)(~(uint32_t)k) : -1;
      if (out_score) out_score[b * K + j] = ok ? key_score((uint32_t)(k >> 32)) : -INFINITY;
    }
  } else {
    for (int j = tid; j < K; j += TK_T)
      keys_out[(b * chunks + c) * (int64_t)K + j] = j < (int)count ? sm.buf[j] : 0ull;
  }
}

template <bool FROM_SCORES, bool FINAL>
__global__ __launch_bounds__(TK_T) void topk_kernel(const float* __restrict__ scores,
                                                    const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ n_valid,
                                                    const uint64_t* __restrict__ keys_in, int64_t M,
                                                    int K, int chunks, uint64_t* __restrict__ keys_out,
                                                    int32_t* __restrict__ out_idx,
                                                    float* __restrict__ out_score) {
  __shared__ TkSmem sm;
  topk_body<FROM_SCORES, FINAL>(sm, blockIdx.x, scores, ids, n_valid, keys_in, M, K, chunks, keys_out, out_idx,
                                out_score);
}

// The final level over B rows of keys (workgroups 0 .. B - 1, as
// topk_kernel<false, true>) and, in the workgroups after them, an
// independent FP4 append walked item by item: the selection occupies B CUs,
// the append the others, so the append costs no time of its own.
__global__ __launch_bounds__(TK_T) void topk_final_append_kernel(const uint64_t* __restrict__ keys_in, int64_t M,
                                                                 int K, int B, int32_t* __restrict__ out_idx,
                                                                 float* __restrict__ out_score, const Fp4Append app,
                                                                 int64_t n_groups, int64_t n_rope) {
  __shared__ TkSmem sm;
  if ((int)blockIdx.x < B) {
    topk_body<false, true>(sm, blockIdx.x, nullptr, nullptr, nullptr, keys_in, M, K, 1, nullptr, out_idx,
                           out_score);
    return;
  }
  const int64_t stride = (int64_t)(gridDim.x - B) * TK_T;
  for (int64_t i = (int64_t)(blockIdx.x - B) * TK_T + threadIdx.x; i < n_groups + n_rope; i += stride)
    fp4_append_item(i, app, n_groups, n_rope);
}

// Append workgroups of the fused final level: enough for about one item per
// thread, at most the CUs beyond the selection's (256 in all on MI355X).
static int64_t append_wgs(int B, int64_t items) {
  const int64_t want = (items + TK_T - 1) / TK_T;
  const int64_t room = B < 248 ? 256 - B : 8;
  return want < room ? (want > 0 ? want : 1) : room;
}

int64_t topk_final_append_launch_items(int B, const Fp4Append& app) {
  const int64_t items = app.n_rows * (app.d_c / 16) + (app.d_r > 0 ? app.n_rows * (app.d_r / 8) : 0);
  return ((int64_t)B + append_wgs(B, items)) * TK_T;
}

// Levels of the chunked reduction: level 0 reads the scores (M columns); level
// L > 0 reads the chunk winners of level L-1.
static int topk_levels(int64_t M, int K, int64_t* chunks_per_level, int max_levels) {
  int n = 0;
  int64_t m = M;
  for (;;) {
    const int64_t ch = (m + TK_CHUNK - 1) / TK_CHUNK;
    if (n < max_levels) chunks_per_level[n] = ch;
    ++n;
    if (ch <= 1) break;
    m = ch * K;
  }
  return n;
}

// The chunked reduction's first level has the most workgroups: one per
// 16384-candidate chunk.
int64_t topk_chunk_launch_items(int B, int64_t M, int K) {
  int64_t ch[16];
  topk_levels(M, K, ch, 16);
  return (int64_t)B * ch[0] * TK_T;
}

size_t topk_chunk_workspace_bytes(int B, int64_t M, int K) {
  int64_t ch[16];
  const int n = topk_levels(M, K, ch, 16);
  size_t bytes = 0;
  for (int l = 0; l + 1 < n; ++l) bytes += (size_t)B * ch[l] * K * sizeof(uint64_t);
  return bytes;
}

// The threshold filter (topk_filter.hip) serves K >= 64 on rows whose
// chunked reduction takes more than three rounds of workgroups at its first
// level (more than three chunks per CU) or more than two levels: there its
// three launches (a sample, one streaming pass, one selection per row) beat
// the levels, whose per-chunk selection costs grow with K (128 rows of
// 129280 columns: 37.7 us at K = 64, 51.3 us at K = 2048, against 30.8 and
// 36.1 us filtered).  Elsewhere, and for K below 64, where a chunk's
// selection is cheap, the levels are as fast or faster (measured on MI355X).
static bool use_filter(int B, int64_t M, int K) {
  if (!topk_filter_fits(B, M, K) || K < 64) return false;
  int64_t ch[16];
  const int n = topk_levels(M, K, ch, 16);
  return (int64_t)B * ch[0] > 768 || n > 2;
}

bool topk_uses_filter(int B, int64_t M, int K) { return use_filter(B, M, K); }

int64_t topk_launch_items(int B, int64_t M, int K) {
  return use_filter(B, M, K) ? topk_filter_launch_items(B, M) : topk_chunk_launch_items(B, M, K);
}

size_t topk_workspace_bytes(int B, int64_t M, int K) {
  return use_filter(B, M, K) ? topk_filter_workspace_bytes(B) : topk_chunk_workspace_bytes(B, M, K);
}

// The levels that reduce chunk winners: keys holds B rows of m keys (the
// winners of the level before, each row's chunks side by side).
size_t topk_keys_workspace_bytes(int B, int64_t m, int K) {
  int64_t ch[16];
  const int n = topk_levels(m, K, ch, 16);
  size_t bytes = 0;
  for (int l = 0; l + 1 < n; ++l) bytes += (size_t)B * ch[l] * K * sizeof(uint64_t);
  return bytes;
}

hipError_t launch_topk_from_keys(const uint64_t* keys, int B, int64_t m, int K, int32_t* out_idx,
                                 float* out_score, void* workspace, hipStream_t stream, const Fp4Append* app) {
  int64_t ch[16];
  const int n = topk_levels(m, K, ch, 16);
  if (n > 16) return hipErrorInvalidValue;
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  const uint64_t* prev = keys;
  for (int l = 0; l < n; ++l) {
    const dim3 grid((unsigned)(B * ch[l]));
    if (l + 1 == n) {
      if (app && app->n_rows > 0) {
        const int64_t n_groups = app->n_rows * (app->d_c / 16);
        const int64_t n_rope = app->d_r > 0 ? app->n_rows * (app->d_r / 8) : 0;
        const dim3 agrid((unsigned)(B + append_wgs(B, n_groups + n_rope)));
        hipLaunchKernelGGL(topk_final_append_kernel, agrid, dim3(TK_T), 0, stream, prev, m, K, B, out_idx,
                           out_score, *app, n_groups, n_rope);
      } else {
        hipLaunchKernelGGL((topk_kernel<false, true>), grid, dim3(TK_T), 0, stream, nullptr, nullptr,
                           nullptr, prev, m, K, 1, nullptr, out_idx, out_score);
      }
      return hipGetLastError();
    }
    hipLaunchKernelGGL((topk_kernel<false, false>), grid, dim3(TK_T), 0, stream, nullptr, nullptr,
                       nullptr, prev, m, K, (int)ch[l], ws, nullptr, nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prev = ws;
    ws += (size_t)B * ch[l] * K;
    m = ch[l] * K;
  }
  return hipSuccess;
}

// Level 0 reads the scores; the chunk winners (when the row has more than one
// chunk) go to the workspace, followed by the later levels' buffers.
hipError_t launch_topk_chunked(const float* scores, const int32_t* ids, const int32_t* n_valid, int B,
                       int64_t M, int K, int32_t* out_idx, float* out_score, void* workspace,
                       hipStream_t stream) {
  if (B == 0) return hipSuccess;
  int64_t ch[16];
  const int n = topk_levels(M, K, ch, 16);
  if (n > 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(B * ch[0]));
  if (n == 1) {
    hipLaunchKernelGGL((topk_kernel<true, true>), grid, dim3(TK_T), 0, stream, scores, ids, n_valid,
                       nullptr, M, K, 1, nullptr, out_idx, out_score);
    return hipGetLastError();
  }
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  hipLaunchKernelGGL((topk_kernel<true, false>), grid, dim3(TK_T), 0, stream, scores, ids, n_valid,
                     nullptr, M, K, (int)ch[0], ws, nullptr, nullptr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_from_keys(ws, B, ch[0] * K, K, out_idx, out_score, ws + (size_t)B * ch[0] * K, stream);
}

hipError_t launch_topk(const float* scores, const int32_t* ids, const int32_t* n_valid, int B,
                       int64_t M, int K, int32_t* out_idx, float* out_score, void* workspace,
                       hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (use_filter(B, M, K))
    return launch_topk_filtered(scores, ids, n_valid, B, M, K, out_idx, out_score, workspace, stream);
  return launch_topk_chunked(scores, ids, n_valid, B, M, K, out_idx, out_score, workspace, stream);
}

}  // namespace csa2
