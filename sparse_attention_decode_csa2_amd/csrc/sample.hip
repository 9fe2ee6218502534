// The decode sampler's draw over a row's Top-K candidates.
//
// The same Top-K selection serves the sparse attention and the sampler
// ([P3] DeepSelect paragraph); the sampling settings are a temperature and a
// top_p ([P1] interface paragraph).  Given the candidates in Top-K order
// (logit descending, token id ascending) this kernel draws one token per row:
//   w_i = exp2((l_i - l_0) * log2(e) / T)        (0 for a -inf logit or an empty slot)
//   nucleus = the shortest prefix whose running weight reaches top_p * sum(w)
//             (every candidate when top_p >= 1 or when none reaches it)
//   draw    = the first nucleus position whose running weight exceeds
//             u * (nucleus weight), u in [0, 1) handed in by the caller
//             (the last position of nonzero weight if rounding leaves none)
// and reports that position's share of the nucleus weight and the nucleus
// size.  A row whose first logit is -inf or NaN, or whose first slot is
// empty, reports its first candidate with probability 1.  Whatever the
// inputs, the drawn position is a slot of the row (never out of bounds).
//
// One workgroup of 256 threads (4 waves) per row: the candidates are read
// coalesced and their weights passed through LDS so that thread t holds the
// E = ceil(K / 256) consecutive candidates [tE, tE + E) in registers (K <=
// 2048, so E <= 8); wave scans of the thread sums plus the wave totals give
// every thread its running weight; the nucleus end and the drawn position are
// minima of per-thread first hits.  Both decisions read the same running
// sums, so the drawn position always lies inside the nucleus.  The
// candidates are a few KB per row: the kernel is latency-bound (a serial
// chain of loads, scans and reductions per row), and four waves per row keep
// that chain a quarter as long as one wave would.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "csa2_internal.h"
#include "sample_draw.h"

namespace csa2 {
namespace {

__global__ __launch_bounds__(SMP_T) void sample_draw_kernel(const int32_t* __restrict__ cand_idx,
                                                            const float* __restrict__ cand_score, int K,
                                                            float log2e_over_t, float top_p,
                                                            const float* __restrict__ u,
                                                            int32_t* __restrict__ token, float* __restrict__ prob,
                                                            int32_t* __restrict__ n_kept) {
  __shared__ SmpSmem sm;
  const int64_t b = blockIdx.x;
  sample_draw_row(b, cand_idx + b * K, cand_score + b * K, K, log2e_over_t, top_p, u, token, prob, n_kept, sm);
}

// ---------------------------------------------------------------------------
// The untruncated draw over the whole vocabulary: the recommended settings,
// temperature 1.0 and top_p 1.0 ([P1] interface paragraph), taken literally
// (top_p 1.0 keeps every token, so no Top-K cap applies):
//   w_i   = exp2((l_i - l_max) * log2(e) / T)   for every token (0 for -inf)
//   token = the first token, in id order, whose running weight exceeds
//           u * sum(w) (the last token of nonzero weight if rounding leaves
//           none); prob = w_token / sum(w).
// A row whose largest logit is -inf draws token 0 with probability 1.
//
// Two launches, one streaming pass.  The row is cut into segments of 1024
// consecutive tokens.  The first kernel gives each workgroup of 1024 threads
// a run of a row's 16384-token tiles (several workgroups per row, so that
// every CU streams); wave w of a tile takes its segment w, lane l the four
// 16-byte runs at tokens 256 q + 4 l of it (each load instruction reads 1 KiB
// of consecutive tokens), and keeps the segment's largest scaled logit and
// its weights summed relative to it: one (max, sum) pair per segment, written
// to the caller's workspace.  The second kernel, one workgroup of 256
// threads per row, reads the row's pairs: the segment totals are rescaled to
// the row's maximum, a prefix over the segments finds the segment holding
// u * sum(w), and only that segment is read again (4 KiB), lane l of one wave
// taking its 16 consecutive tokens: their weights relative to the row
// maximum and a wave scan give every token its running weight, and the first
// one above the target is the draw.  The segment totals and the running
// weights inside the drawn segment are summed in different orders, so
// float32 rounding may move a draw whose running weight lies within rounding
// of the target by one token; the drawn token always has nonzero weight.
constexpr int SF_T = 1024;                      // threads per row
constexpr int SF_WAVES = SF_T / 64;
constexpr int SF_PER = 16;                      // tokens per thread and tile
constexpr int SF_TILE = SF_PER * SF_T;          // tokens per tile
constexpr int SF_MAX_TILES = 64;                // V <= 2^20
constexpr int SF_RUN = 2;                       // tiles per workgroup of the statistics pass, loaded together

constexpr int SF_SEG = 1024;                    // tokens per segment (one wave of a tile)
constexpr int SD_T = 256;                       // threads of the draw workgroup
constexpr int SD_WAVES = SD_T / 64;
constexpr int SD_SEGS = SF_MAX_TILES * SF_WAVES / SD_T;  // segments per draw thread (4)

struct SdSmem {
  float wmax[SD_WAVES], wsum[SD_WAVES];
  int hit[SD_WAVES], last[SD_WAVES];
  int seg;
  float before;
};

// (m, s) pairs: s weights summed relative to m (m = -inf: nothing yet)
__device__ __forceinline__ void sf_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = (m == -INFINITY ? 0.0f : s * exp2f(m - mn)) + (m2 == -INFINITY ? 0.0f : s2 * exp2f(m2 - mn));
  m = mn;
}

// Four consecutive logits from token i0 (-inf past the row's end).
template <bool VEC>
__device__ __forceinline__ void sf_load(const float* row, int64_t V, int64_t i0, float* x) {
  if (VEC && i0 + 4 <= V) {
    const float4 v = *reinterpret_cast<const float4*>(row + i0);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = i0 + e < V ? row[i0 + e] : -INFINITY;
  }
}

// Statistics pass: workgroup (b, r) covers tiles [SF_RUN r, SF_RUN r + SF_RUN)
// of row b and writes, per segment g = 16 j + w (wave w of tile j), the pair
// (largest scaled logit, weights summed relative to it) to
// ws[b * 16 n_tiles + g].
template <bool VEC>
__global__ __launch_bounds__(SF_T) void sample_full_stats_kernel(const float* __restrict__ logits, int64_t V,
                                                                 float log2e_over_t, int runs,
                                                                 float2* __restrict__ ws) {
  // no fused multiply-add: a scaled logit is rounded once and every later use
  // sees that value (a fused x * c - m would give the maximum itself a weight
  // of exp2 of the product's rounding error instead of exactly one)
#pragma clang fp contract(off)
  const int64_t b = blockIdx.x / runs;
  const int j0 = (int)(blockIdx.x - b * runs) * SF_RUN;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* row = logits + b * V;
  const int n_tiles = (int)((V + SF_TILE - 1) / SF_TILE);
  float x[SF_RUN][SF_PER];
#pragma unroll
  for (int h = 0; h < SF_RUN; ++h)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sf_load<VEC>(row, V, (int64_t)(j0 + h) * SF_TILE + SF_SEG * wv + 256 * q + 4 * lane, &x[h][4 * q]);
#pragma unroll
  for (int h = 0; h < SF_RUN; ++h) {
    if (j0 + h >= n_tiles) break;
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < SF_PER; ++e) {
      x[h][e] *= log2e_over_t;  // -inf stays -inf
      m = fmaxf(m, x[h][e]);
    }
    float sum = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int e = 0; e < SF_PER; ++e) sum += x[h][e] == -INFINITY ? 0.0f : exp2f(x[h][e] - m);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float m2 = __shfl_xor(m, d, 64), s2 = __shfl_xor(sum, d, 64);
      sf_merge(m, sum, m2, s2);
    }
    if (lane == 0) ws[(b * n_tiles + j0 + h) * SF_WAVES + wv] = float2{m, sum};
  }
}

// Draw pass: one workgroup per row over the statistics of its segments.
template <bool VEC>
__global__ __launch_bounds__(SD_T) void sample_full_kernel(const float* __restrict__ logits, int64_t V,
                                                           float log2e_over_t, const float2* __restrict__ ws,
                                                           const float* __restrict__ u,
                                                           int32_t* __restrict__ token, float* __restrict__ prob) {
#pragma clang fp contract(off)
  __shared__ SdSmem sm;
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* row = logits + b * V;
  const int n_seg = (int)((V + SF_TILE - 1) / SF_TILE) * SF_WAVES;   // <= 1024
  // ---- thread t: segments SD_SEGS t .. + SD_SEGS - 1 (pairs past the row: empty)
  float m[SD_SEGS], sg[SD_SEGS];
#pragma unroll
  for (int i = 0; i < SD_SEGS; ++i) {
    const int g = SD_SEGS * t + i;
    const float2 p = g < n_seg ? ws[b * n_seg + g] : float2{-INFINITY, 0.0f};
    m[i] = p.x;
    sg[i] = p.y;
  }
  float mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < SD_SEGS; ++i) mt = fmaxf(mt, m[i]);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) mt = fmaxf(mt, __shfl_xor(mt, d, 64));
  if (lane == 0) sm.wmax[wv] = mt;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < SD_WAVES; ++w) M = fmaxf(M, sm.wmax[w]);
  if (M == -INFINITY) {          // every logit -inf (or NaN)
    if (t == 0) {
      token[b] = 0;
      if (prob) prob[b] = 1.0f;
    }
    return;
  }
  // ---- segment totals relative to the row maximum, their running sums
  float tt[SD_SEGS], run[SD_SEGS], local = 0.0f;
#pragma unroll
  for (int i = 0; i < SD_SEGS; ++i) {
    tt[i] = m[i] == -INFINITY ? 0.0f : sg[i] * exp2f(m[i] - M);
    local += tt[i];
    run[i] = local;
  }
  const float incl = wave_inclusive_sum(local, lane);
  if (lane == 63) sm.wsum[wv] = incl;
  __syncthreads();
  float before = incl - local, total = 0.0f;
#pragma unroll
  for (int v = 0; v < SD_WAVES; ++v) {
    before += v < wv ? sm.wsum[v] : 0.0f;
    total += sm.wsum[v];
  }
  const float target = u[b] * total;
  // only a segment of nonzero weight can hold the draw (the scan's rounding
  // differs between threads, so an empty segment's running total may still
  // step over the target); if rounding leaves none, the last segment of
  // nonzero weight (the maximum's segment has weight >= 1)
  int hit = INT32_MAX, last = -1;
#pragma unroll
  for (int i = 0; i < SD_SEGS; ++i) {
    const int g = SD_SEGS * t + i;
    last = tt[i] > 0.0f ? g : last;
    hit = min(hit, (tt[i] > 0.0f && before + run[i] > target) ? g : INT32_MAX);
  }
  hit = wave_min_i(hit);
  last = wave_max_i(last);
  if (lane == 0) {
    sm.hit[wv] = hit;
    sm.last[wv] = last;
  }
  __syncthreads();
  hit = INT32_MAX;
  last = -1;
#pragma unroll
  for (int v = 0; v < SD_WAVES; ++v) {
    hit = min(hit, sm.hit[v]);
    last = max(last, sm.last[v]);
  }
  const int seg = hit != INT32_MAX ? hit : last;
  // the running total before the segment, from the thread that holds it
#pragma unroll
  for (int i = 0; i < SD_SEGS; ++i)
    if (SD_SEGS * t + i == seg) sm.before = before + run[i] - tt[i];
  __syncthreads();
  if (wv != 0) return;
  // ---- wave 0: the segment again, lane l its 16 consecutive tokens
  float x[SF_PER];
  const int64_t i0 = (int64_t)seg * SF_SEG + SF_PER * lane;
#pragma unroll
  for (int q = 0; q < 4; ++q) sf_load<VEC>(row, V, i0 + 4 * q, &x[4 * q]);
  float w[SF_PER], wrun[SF_PER], wl = 0.0f;
#pragma unroll
  for (int e = 0; e < SF_PER; ++e) {
    const float y = x[e] * log2e_over_t;
    w[e] = y == -INFINITY ? 0.0f : exp2f(y - M);
    wl += w[e];
    wrun[e] = wl;
  }
  const float winc = wave_inclusive_sum(wl, lane);
  const float wbefore = sm.before + winc - wl;
  int khit = INT32_MAX, klast = -1;
#pragma unroll
  for (int e = 0; e < SF_PER; ++e) {
    const int k = SF_PER * lane + e;
    klast = w[e] > 0.0f ? k : klast;
    khit = min(khit, (w[e] > 0.0f && wbefore + wrun[e] > target) ? k : INT32_MAX);
  }
  khit = wave_min_i(khit);
  klast = wave_max_i(klast);
  // the segment has a token of nonzero weight (its total is positive); were
  // every weight to underflow on the second read, its first token is written
  const int k = khit != INT32_MAX ? khit : max(klast, 0);
  if (k / SF_PER == lane) {
#pragma unroll
    for (int e = 0; e < SF_PER; ++e) {
      if (k % SF_PER == e) {
        token[b] = (int32_t)(i0 + e);
        if (prob) prob[b] = w[e] / total;
      }
    }
  }
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int sf_runs(int64_t V) { return (int)(((V + SF_TILE - 1) / SF_TILE + SF_RUN - 1) / SF_RUN); }

int64_t sample_full_launch_items(int B, int64_t V) { return (int64_t)B * sf_runs(V) * SF_T; }

size_t sample_full_workspace_bytes(int B, int64_t V) {
  return (size_t)B * ((V + SF_TILE - 1) / SF_TILE) * SF_WAVES * sizeof(float2);
}

hipError_t launch_sample_full(const float* logits, int B, int64_t V, float temperature, const float* u,
                              int32_t* token, float* prob, void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (V > (int64_t)SF_MAX_TILES * SF_TILE) return hipErrorInvalidValue;
  const float log2e_over_t = (float)(1.4426950408889634 / (double)temperature);
  float2* ws = static_cast<float2*>(workspace);
  const int runs = sf_runs(V);
  // 16-byte loads when every row starts on a 16-byte boundary
  if (V % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0) {
    hipLaunchKernelGGL(sample_full_stats_kernel<true>, dim3((unsigned)((int64_t)B * runs)), dim3(SF_T), 0, stream,
                       logits, V, log2e_over_t, runs, ws);
    hipLaunchKernelGGL(sample_full_kernel<true>, dim3(B), dim3(SD_T), 0, stream, logits, V, log2e_over_t, ws, u,
                       token, prob);
  } else {
    hipLaunchKernelGGL(sample_full_stats_kernel<false>, dim3((unsigned)((int64_t)B * runs)), dim3(SF_T), 0, stream,
                       logits, V, log2e_over_t, runs, ws);
    hipLaunchKernelGGL(sample_full_kernel<false>, dim3(B), dim3(SD_T), 0, stream, logits, V, log2e_over_t, ws, u,
                       token, prob);
  }
  return hipGetLastError();
}

size_t sample_workspace_bytes(int B, int64_t V, int K) {
  return 2 * align256((size_t)B * K * 4) + topk_workspace_bytes(B, V, K);
}

int64_t sample_draw_launch_items(int B) { return (int64_t)B * SMP_T; }

hipError_t launch_sample_draw(const int32_t* cand_idx, const float* cand_score, int B, int K, float temperature,
                              float top_p, const float* u, int32_t* token, float* prob, int32_t* n_kept,
                              hipStream_t stream) {
  const float log2e_over_t = (float)(1.4426950408889634 / (double)temperature);
  hipLaunchKernelGGL(sample_draw_kernel, dim3(B), dim3(SMP_T), 0, stream, cand_idx, cand_score, K, log2e_over_t,
                     top_p, u, token, prob, n_kept);
  return hipGetLastError();
}

hipError_t launch_sample(const float* logits, int B, int64_t V, int K, float temperature, float top_p,
                         const float* u, int32_t* token, float* prob, int32_t* n_kept, void* workspace,
                         hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(ws);
  float* cand_score = reinterpret_cast<float*>(ws + align256((size_t)B * K * 4));
  void* tk_ws = ws + 2 * align256((size_t)B * K * 4);
  if (topk_uses_filter(B, V, K)) {
    // the threshold filter's last kernel draws from the rows it writes
    const SampleDraw d{(float)(1.4426950408889634 / (double)temperature), top_p, u, token, prob, n_kept};
    return launch_topk_filtered(logits, nullptr, nullptr, B, V, K, cand_idx, cand_score, tk_ws, stream, &d);
  }
  hipError_t e = launch_topk(logits, nullptr, nullptr, B, V, K, cand_idx, cand_score,
                             topk_workspace_bytes(B, V, K) ? tk_ws : nullptr, stream);
  if (e != hipSuccess) return e;
  return launch_sample_draw(cand_idx, cand_score, B, K, temperature, top_p, u, token, prob, n_kept, stream);
}

}  // namespace csa2
