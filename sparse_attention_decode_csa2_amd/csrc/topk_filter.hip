// a3 for long rows: Top-K with the lower id winning ties (Top-512 per [P1]
// 架构三件套, CSA2; the sampler's Top-K over the vocabulary, [P3] DeepSelect
// paragraph) by a threshold filter instead of chunk levels.  The result is
// bit for bit that of the chunked reduction: the same 64-bit keys, the same
// total order.
//
//  A. estimate (one 1024-thread workgroup per row): sixteen runs of 256
//     columns spread evenly over the row form a sample of 4096 scores; two
//     radix passes over their order-preserving score keys place the k'-th
//     largest sample key in a narrow range whose floor is theta, with k' the
//     sample's expected share of the row's K winners raised by a quarter,
//     four standard deviations and 8.
//     Rows of at most 16384 columns, and samples of at most k' valid
//     columns, take theta = 0 (every candidate).
//  B. filter (about two 1024-thread workgroups per CU, each a contiguous
//     range of a row's 16384-column tiles): each wave appends the keys >=
//     theta of its columns to the workgroup's list in LDS (one LDS atomic
//     per wave and tile, no barrier); one atomic on the row's counter then
//     places the list among the row's candidates.  At most 16384 keys are
//     stored; the count keeps growing (and a list longer than the LDS holds
//     pushes it past 16384).  Rows of at most 16384 columns skip this step.
//  C. select (one 1024-thread workgroup per row): with n keys appended,
//     n <= 16384 and either theta = 0 or n >= K, the list holds every
//     candidate whose key is at least the row's K-th largest (at least K keys
//     lie at or above theta), so the block-level selection of topk_block.h
//     over the list is the row's Top-K.  Otherwise (a sample that put theta
//     above the row's K-th key, or more than 16384 keys at or above it) the
//     workgroup reduces the row by itself: a running Top-K in LDS merged with
//     the next 16384 - K columns by one block selection per step (rows of at
//     most 16384 columns: that one selection).
// Every load of a thread is issued before the first result is used; a load
// under a per-element branch would wait for the one before it.
#include "csa2_internal.h"
#include "sample_draw.h"
#include "topk_block.h"

namespace csa2 {

constexpr int TF_CAP = TK_CHUNK;          // candidate slots per row: one block selection
constexpr int TF_SE = 4;                  // sample elements per thread
constexpr int TF_RUN = 64 * TF_SE;        // sample run length (columns): one wave
constexpr int TF_RUNS = TK_WAVES;
constexpr int TF_FT = 1024;               // filter threads per workgroup
constexpr int TF_FCOLS = TF_FT * TK_E;    // columns of a filter tile
constexpr int TF_LCAP = 8192;             // keys a filter workgroup gathers in LDS
constexpr int64_t TF_MAX_M = (int64_t)1 << 20;  // longest row served (bounds the in-workgroup fallback)

// One cache line per row, so the filter's counter atomics of different rows
// never share a line.
struct TfRow {
  uint32_t theta;  // score-key threshold (0: every candidate)
  uint32_t count;  // keys appended by the filter
  uint32_t pad[30];
};

__device__ __forceinline__ int64_t tf_limit(const int32_t* n_valid, int64_t b, int64_t M) {
  int64_t limit = M;
  if (n_valid) limit = min<int64_t>(limit, max<int64_t>(n_valid[b], 0));
  return limit;
}

// Scores and ids of N columns (id -1: outside the row or an empty
// candidate).  The loads are unconditional, at the column clamped into the
// row (column 0 of an empty row; a row holds at least one column), and all
// are issued before any result is used: a load under a branch would wait for
// the one before it.
template <int N>
__device__ __forceinline__ void tf_load_cols(const float* srow, const int32_t* irow, const int64_t (&col)[N],
                                             int64_t limit, float (&s)[N], uint32_t (&id)[N]) {
  const int64_t last = limit > 0 ? limit - 1 : 0;
  if (irow) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int64_t cc = min<int64_t>(col[e], last);
      s[e] = srow[cc];
      id[e] = (uint32_t)irow[cc];
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      s[e] = srow[min<int64_t>(col[e], last)];
      id[e] = (uint32_t)col[e];
    }
  }
#pragma unroll
  for (int e = 0; e < N; ++e) id[e] = col[e] < limit ? id[e] : 0xFFFFFFFFu;
}

// One column (the in-workgroup reduction's mixed steps).
__device__ __forceinline__ void tf_load(const float* srow, const int32_t* irow, int64_t col, int64_t limit,
                                        float* s, uint32_t* id) {
  const int64_t c[1] = {col};
  float s1[1];
  uint32_t i1[1];
  tf_load_cols<1>(srow, irow, c, limit, s1, i1);
  *s = s1[0];
  *id = i1[0];
}

// ---------------------------------------------------------------- A
__global__ __launch_bounds__(TK_T) void topk_estimate_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ n_valid, int64_t M,
                                                             int K, TfRow* __restrict__ rows) {
  __shared__ TkSmem sm;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t limit = tf_limit(n_valid, b, M);
  if (limit <= TF_CAP) {  // uniform: the row fits one selection
    if (tid == 0) {
      rows[b].theta = 0u;
      rows[b].count = 0u;
    }
    return;
  }
  tk_init(sm);
  const float* srow = scores + b * M;
  const int32_t* irow = ids ? ids + b * M : nullptr;
  // wave r reads run r, which starts at column r (limit - 256) / 15 (the
  // runs are evenly spaced and cover both ends of the row); element e of lane
  // l is column 64 e + l of the run, so each load is one contiguous 256-byte
  // piece.  A sample of 4096 measured faster than one of 16384 (sample-129k
  // Top-K + draw 43.1 -> 39.8 us): the estimate's loads and radix passes
  // shrink, and the threshold keeps a few hundred more candidates
  static_assert(TF_RUN == WAVE * TF_SE && TF_RUNS == TK_WAVES, "one run per wave");
  const int64_t c0 = (int64_t)wave_id() * (limit - TF_RUN) / (TF_RUNS - 1) + lane_id();
  int64_t col[TF_SE];
  float s[TF_SE];
  uint32_t id[TF_SE], key[TF_SE];
#pragma unroll
  for (int e = 0; e < TF_SE; ++e) col[e] = c0 + WAVE * e;
  tf_load_cols<TF_SE>(srow, irow, col, limit, s, id);
  lanemask act = 0;
#pragma unroll
  for (int e = 0; e < TF_SE; ++e) {
    const bool ok = id[e] != 0xFFFFFFFFu;
    key[e] = ok ? score_key(s[e]) : 0u;
    act |= (lanemask)ok << e;
  }
  int par = 0;
  uint32_t n, kmax, kmin;
  active_stats<TF_SE>(key, act, sm, par, &n, &kmax, &kmin);
  // the sample's expected share of the row's K winners, raised so that theta
  // lies below the row's K-th key unless the sample misleads (the selection
  // detects that and reduces the row itself)
  const float expct = (float)K * (float)(TF_RUN * TF_RUNS) / (float)limit;
  uint32_t kp = (uint32_t)ceilf(1.25f * expct + 4.0f * sqrtf(expct) + 8.0f);
  uint32_t theta = 0u;
  // a sample with at most k' valid keys keeps every candidate (theta 0): the
  // row then holds few of them, about as many as the list has room for
  if (kp < n) {  // uniform
    // two radix passes (22 bits below the keys' common prefix) place the
    // k'-th largest sample key in a region; its floor, at or below every key
    // of the region, is the threshold (a third pass and the exact key cost a
    // further ~1.8 us for a few more kept keys)
    const TkRegion g = radix_select<TF_SE>(key, act, kp, kmax, kmin, n, 2, sm, par);
    theta = g.prefix;
  }
  if (tid == 0) {
    rows[b].theta = theta;
    rows[b].count = 0u;
  }
}

// ---------------------------------------------------------------- B
// Workgroup g of a row filters the row's 16384-column tiles [g tpw, (g + 1)
// tpw).  Each wave appends its passing keys to the workgroup's list in LDS
// (one LDS atomic per wave and tile, no barrier); at the end one atomic on
// the row's counter places the list in the row's candidates.  Rows of at
// most 16384 columns are selected from the scores directly and skip this.
template <bool IDS>
__global__ __launch_bounds__(TF_FT) __attribute__((amdgpu_waves_per_eu(8, 8))) void topk_filter_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ n_valid, int64_t M,
                                                            int wg_per_row, int tiles_per_wg,
                                                            TfRow* __restrict__ rows, uint64_t* __restrict__ cand) {
  __shared__ uint64_t lkeys[TF_LCAP];
  __shared__ uint32_t lcount, gbase, gn;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t b = blockIdx.x / wg_per_row;
  const int g = (int)(blockIdx.x - b * wg_per_row);
  const int64_t limit = tf_limit(n_valid, b, M);
  const int64_t t0 = (int64_t)g * tiles_per_wg;
  if (limit <= TF_CAP || t0 * TF_FCOLS >= limit) return;  // uniform
  const int64_t t1 = min<int64_t>(t0 + tiles_per_wg, (limit + TF_FCOLS - 1) / TF_FCOLS);
  const uint32_t theta = rows[b].theta;
  const float* srow = scores + b * M;
  const int32_t* irow = IDS ? ids + b * M : nullptr;
  if (tid == 0) lcount = 0u;
  __syncthreads();
  for (int64_t t = t0; t < t1; ++t) {
    // element (q, j) of thread i: column 16384 t + 4096 q + 4 i + j, so each
    // 16-byte load of a wave is one contiguous 1 KiB piece
    const uint32_t cb = (uint32_t)(t * TF_FCOLS) + 4u * (uint32_t)tid;  // columns fit 31 bits
    const uint32_t lim = (uint32_t)limit;
    float v[TK_E];
    uint32_t idv[IDS ? TK_E : 1];
    uint32_t inrow = 0;  // bit e: element e is a candidate (in the row, id != -1)
    if ((M & 3) == 0) {
      // 16-byte loads (rows stay 16-byte aligned); a piece past the row's
      // end reads the row's last piece instead, its columns dropped below
      f32x4 v4[4];
      u32x4 i4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t c = min(cb + (uint32_t)(TF_FCOLS / 4 * q), (uint32_t)M - 4u);
        v4[q] = *reinterpret_cast<const f32x4*>(srow + c);
        if constexpr (IDS) i4[q] = *reinterpret_cast<const u32x4*>(irow + c);
      }
#pragma unroll
      for (int e = 0; e < TK_E; ++e) {
        const uint32_t col = cb + (uint32_t)(TF_FCOLS / 4 * (e / 4) + e % 4);
        v[e] = v4[e / 4][e % 4];
        bool ok = col < lim;
        if constexpr (IDS) {
          idv[e] = i4[e / 4][e % 4];
          ok = ok && idv[e] != 0xFFFFFFFFu;
        }
        inrow |= (uint32_t)ok << e;
      }
    } else {
      // rows of M % 4 != 0: four loads at a time
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int64_t col[4];
        float s4[4];
        uint32_t id4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) col[j] = cb + (uint32_t)(TF_FCOLS / 4 * q + j);
        tf_load_cols<4>(srow, irow, col, limit, s4, id4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[4 * q + j] = s4[j];
          if constexpr (IDS) idv[4 * q + j] = id4[j];
          inrow |= (uint32_t)(id4[j] != 0xFFFFFFFFu) << (4 * q + j);
        }
      }
    }
    uint32_t pass = 0;  // score keys of candidates are >= 1
#pragma unroll
    for (int e = 0; e < TK_E; ++e) pass |= (uint32_t)(((inrow >> e) & 1u) && score_key(v[e]) >= theta) << e;
    const uint32_t cnt = (uint32_t)__popc(pass);
    const uint32_t incl = wave_incl_scan(cnt);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (!wtot) continue;  // uniform in the wave
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&lcount, wtot);
    uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)base) + incl - cnt;
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if ((pass >> e) & 1u) {
        const uint32_t id = IDS ? idv[IDS ? e : 0] : cb + (uint32_t)(TF_FCOLS / 4 * (e / 4) + e % 4);
        if (pos < (uint32_t)TF_LCAP) lkeys[pos] = ((uint64_t)score_key(v[e]) << 32) | (uint64_t)(~id);
        ++pos;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t n = lcount;
    uint32_t base = 0;
    // a list longer than the LDS holds: push the row's count past the
    // candidate slots, so that the selection reduces the row itself
    if (n > (uint32_t)TF_LCAP) atomicAdd(&rows[b].count, (uint32_t)TF_CAP + 1u);
    else if (n) base = atomicAdd(&rows[b].count, n);
    gbase = base;
    gn = n > (uint32_t)TF_LCAP ? 0u : n;
  }
  __syncthreads();
  const uint32_t base = gbase, n = gn;
  uint64_t* crow = cand + b * (int64_t)TF_CAP;
  for (uint32_t i = (uint32_t)tid; i < n; i += TF_FT)
    if (base + i < (uint32_t)TF_CAP) crow[base + i] = lkeys[i];
}

// ---------------------------------------------------------------- C
// The final selection over the block's elements, sorted into the output row.
__device__ __forceinline__ void tf_final(const float (&v)[TK_E], const uint32_t (&idv)[TK_E], lanemask valid, bool ids_are_columns,
                         int K, int32_t* out_idx, float* out_score, TkSmem& sm) {
  TkDst dst;
  dst.idx = out_idx;
  dst.score = out_score;
  dst.keys = nullptr;
  const uint32_t count = block_select<true>(v, idv, valid, ids_are_columns, K, dst, sm);
  if (count == TK_WRITTEN) return;
  if (count > 1) {
    int nn = 64;
    while (nn < (int)count) nn <<= 1;
    for (int j = (int)count + threadIdx.x; j < nn; j += TK_T) sm.buf[j] = 0ull;
    sort_desc_n(nn, sm);
  }
  for (int j = threadIdx.x; j < K; j += TK_T) {
    const bool ok = j < (int)count;
    const uint64_t k = ok ? sm.buf[j] : 0ull;
    out_idx[j] = ok ? (int32_t)(~(uint32_t)k) : -1;
    if (out_score) out_score[j] = ok ? key_score((uint32_t)(k >> 32)) : -INFINITY;
  }
}

__device__ __forceinline__ void tf_from_key(uint64_t k, int e, float (&v)[TK_E], uint32_t (&idv)[TK_E],
                                            lanemask& valid) {
  const uint32_t hk = (uint32_t)(k >> 32);
  idv[e] = ~(uint32_t)k;
  v[e] = hk != 0 ? key_score(hk) : __uint_as_float(F_NAN);
  valid |= (lanemask)(hk != 0) << e;
}

// Row b's final selection (run_keys: the fallback's running Top-K).
__device__ __forceinline__ void tf_select_row(int64_t b, const float* __restrict__ scores,
                                              const int32_t* __restrict__ ids, const int32_t* __restrict__ n_valid,
                                              int64_t M, int K, const TfRow* __restrict__ rows,
                                              const uint64_t* __restrict__ cand, int32_t* __restrict__ out_idx,
                                              float* __restrict__ out_score, TkSmem& sm, uint64_t* run_keys) {
  const int tid = threadIdx.x;
  const uint32_t theta = rows[b].theta, n = rows[b].count;
  const int64_t limit = tf_limit(n_valid, b, M);
  float v[TK_E];
  uint32_t idv[TK_E];
  lanemask valid = 0;
  bool cols = false;  // ids rise with the position
  if (limit > TF_CAP && n <= (uint32_t)TF_CAP && (theta == 0u || n >= (uint32_t)K)) {  // uniform
    tk_init(sm);
    // key i of the list is element i / 1024 of thread i % 1024 (the list has
    // no order to keep), so each load of a wave is one contiguous piece
    const uint64_t* crow = cand + b * (int64_t)TF_CAP;
    // unconditional loads, all issued before any result is used
    uint64_t k[TK_E];
#pragma unroll
    for (int e = 0; e < TK_E; ++e) k[e] = crow[min((uint32_t)(TK_T * e + tid), (uint32_t)TF_CAP - 1u)];
#pragma unroll
    for (int e = 0; e < TK_E; ++e) tf_from_key((uint32_t)(TK_T * e + tid) < n ? k[e] : 0ull, e, v, idv, valid);
  } else {
    // the row reduced by this workgroup (rows of at most 16384 columns come
    // here directly): each step selects the Top-K of the running keys
    // (positions [0, have)) and the next 16384 - have columns; the last
    // step's selection is the final one below
    const float* srow = scores + b * M;
    const int32_t* irow = ids ? ids + b * M : nullptr;
    uint32_t have = 0;
    int64_t base = 0;
    auto load_step = [&]() {
      __syncthreads();  // the previous step is done with the LDS
      tk_init(sm);
      valid = 0;
      const int64_t c0 = base + (int64_t)TK_E * tid;
      if (have == 0 && !irow && c0 + TK_E <= limit && (M & 3) == 0) {
        // a whole run of columns: 16-byte loads (rows stay 16-byte aligned)
#pragma unroll
        for (int q = 0; q < TK_E / 4; ++q) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(srow + c0 + 4 * q);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[4 * q + j] = v4[j];
            idv[4 * q + j] = (uint32_t)(c0 + 4 * q + j);
          }
        }
        valid = (lanemask(1) << TK_E) - 1u;
        cols = true;
        return;
      }
#pragma unroll
      for (int e = 0; e < TK_E; ++e) {
        const uint32_t p = (uint32_t)(TK_E * tid + e);
        if (p < have) {
          tf_from_key(run_keys[p], e, v, idv, valid);
        } else {
          float s;
          uint32_t id;
          tf_load(srow, irow, base + (int64_t)(p - have), limit, &s, &id);
          const bool ok = id != 0xFFFFFFFFu;
          v[e] = ok ? s : __uint_as_float(F_NAN);
          idv[e] = id;
          valid |= (lanemask)ok << e;
        }
      }
      cols = have == 0 && ids == nullptr;
    };
    while (base + (TK_CHUNK - (int64_t)have) < limit) {
      load_step();
      TkDst dst;
      dst.idx = nullptr;
      dst.score = nullptr;
      dst.keys = run_keys;
      const uint32_t c = block_select<false>(v, idv, valid, cols, K, dst, sm);
      if (c != TK_WRITTEN)
        for (int j = tid; j < K; j += TK_T) run_keys[j] = j < (int)c ? sm.buf[j] : 0ull;
      base += TK_CHUNK - (int64_t)have;
      have = (uint32_t)K;
    }
    load_step();
  }
  tf_final(v, idv, valid, cols, K, out_idx + b * K, out_score ? out_score + b * K : nullptr, sm);
}

__global__ __launch_bounds__(TK_T) void topk_select_kernel(const float* __restrict__ scores,
                                                           const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ n_valid, int64_t M, int K,
                                                           const TfRow* __restrict__ rows,
                                                           const uint64_t* __restrict__ cand,
                                                           int32_t* __restrict__ out_idx,
                                                           float* __restrict__ out_score) {
  __shared__ TkSmem sm;
  __shared__ uint64_t run_keys[TK_KMAX];
  tf_select_row(blockIdx.x, scores, ids, n_valid, M, K, rows, cand, out_idx, out_score, sm, run_keys);
}

// The selection, then the sampler's draw over the row just written (the
// candidates of csa2_sample): one launch fewer than the draw kernel after
// the Top-K, the same draw (sample_draw_row).
__global__ __launch_bounds__(TK_T) void topk_select_draw_kernel(const float* __restrict__ scores,
                                                                const int32_t* __restrict__ n_valid, int64_t M,
                                                                int K, const TfRow* __restrict__ rows,
                                                                const uint64_t* __restrict__ cand,
                                                                int32_t* __restrict__ out_idx,
                                                                float* __restrict__ out_score, const SampleDraw d) {
  __shared__ TkSmem sm;
  __shared__ uint64_t run_keys[TK_KMAX];
  __shared__ SmpSmem dsm;
  const int64_t b = blockIdx.x;
  tf_select_row(b, scores, nullptr, n_valid, M, K, rows, cand, out_idx, out_score, sm, run_keys);
  __syncthreads();  // the row's candidates are written (and visible to the workgroup)
  sample_draw_row(b, out_idx + b * K, out_score + b * K, K, d.log2e_over_t, d.top_p, d.u, d.token, d.prob,
                  d.n_kept, dsm);
}

// ---------------------------------------------------------------- host
bool topk_filter_fits(int B, int64_t M, int K) { return B > 0 && M > TK_CHUNK && M <= TF_MAX_M && K <= TK_KMAX; }

size_t topk_filter_workspace_bytes(int B) {
  return (size_t)B * sizeof(TfRow) + (size_t)B * TF_CAP * sizeof(uint64_t);
}

int64_t topk_filter_launch_items(int B, int64_t M) {
  // at most one filter workgroup per tile
  return (int64_t)B * ((M + TF_FCOLS - 1) / TF_FCOLS) * TF_FT;
}

hipError_t launch_topk_filtered(const float* scores, const int32_t* ids, const int32_t* n_valid, int B, int64_t M,
                                int K, int32_t* out_idx, float* out_score, void* workspace, hipStream_t stream,
                                const SampleDraw* draw) {
  TfRow* rows = static_cast<TfRow*>(workspace);
  uint64_t* cand = reinterpret_cast<uint64_t*>(rows + B);
  hipLaunchKernelGGL(topk_estimate_kernel, dim3((unsigned)B), dim3(TK_T), 0, stream, scores, ids, n_valid, M, K,
                     rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // about two workgroups per CU: each row's tiles split over g workgroups
  const int64_t tiles = (M + TF_FCOLS - 1) / TF_FCOLS;
  int64_t g = (512 + B - 1) / B;
  if (g > tiles) g = tiles;
  const int64_t tpw = (tiles + g - 1) / g;
  const int64_t wpr = (tiles + tpw - 1) / tpw;
  if (ids)
    hipLaunchKernelGGL(topk_filter_kernel<true>, dim3((unsigned)((int64_t)B * wpr)), dim3(TF_FT), 0, stream, scores,
                       ids, n_valid, M, (int)wpr, (int)tpw, rows, cand);
  else
    hipLaunchKernelGGL(topk_filter_kernel<false>, dim3((unsigned)((int64_t)B * wpr)), dim3(TF_FT), 0, stream, scores,
                       ids, n_valid, M, (int)wpr, (int)tpw, rows, cand);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (draw && !ids && out_score)
    hipLaunchKernelGGL(topk_select_draw_kernel, dim3((unsigned)B), dim3(TK_T), 0, stream, scores, n_valid, M, K,
                       rows, cand, out_idx, out_score, *draw);
  else
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)B), dim3(TK_T), 0, stream, scores, ids, n_valid, M, K,
                       rows, cand, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace csa2
