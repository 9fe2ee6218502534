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

namespace csa2 {
namespace {

constexpr int SMP_T = 256;                  // threads per row (4 waves)
constexpr int SMP_WAVES = SMP_T / 64;
constexpr int SMP_E = 2048 / SMP_T;         // candidates per thread at K = 2048

__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = min(x, __shfl_xor(x, d, 64));
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, __shfl_xor(x, d, 64));
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

struct SmpSmem {
  float w[SMP_T * SMP_E + SMP_T * SMP_E / 32];   // weights, one pad word per 32
  float wsum[SMP_WAVES];
  int wint[2][SMP_WAVES];
  float cn, wp;
};

__device__ __forceinline__ int pad_idx(int i) { return i + (i >> 5); }

__global__ __launch_bounds__(SMP_T) void sample_draw_kernel(const int32_t* __restrict__ cand_idx,
                                                            const float* __restrict__ cand_score, int K,
                                                            float log2e_over_t, float top_p,
                                                            const float* __restrict__ u,
                                                            int32_t* __restrict__ token, float* __restrict__ prob,
                                                            int32_t* __restrict__ n_kept) {
  __shared__ SmpSmem sm;
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int32_t* ci = cand_idx + b * K;
  const float* cs = cand_score + b * K;
  const int E = (K + SMP_T - 1) / SMP_T;
  const int i0 = t * E;
  const float s0 = cs[0];
  const int32_t id0 = ci[0];
  if (!(s0 > -INFINITY) || id0 < 0) {   // every logit -inf, NaN at the top, or no candidate
    if (t == 0) {
      token[b] = id0;
      if (prob) prob[b] = 1.0f;
      if (n_kept) n_kept[b] = 1;
    }
    return;
  }

  // weights from coalesced loads (element 256 j + t; every load issued before
  // the first use, the index clamped into the row), handed through LDS to the
  // thread that scans them (elements [tE, tE + E))
  int32_t idv[SMP_E];
  float scv[SMP_E];
#pragma unroll
  for (int j = 0; j < SMP_E; ++j) {
    const int i = min(j * SMP_T + t, K - 1);
    idv[j] = ci[i];
    scv[j] = cs[i];
  }
  int valid = 0;
#pragma unroll
  for (int j = 0; j < SMP_E; ++j) {
    const int i = j * SMP_T + t;
    if (i < K) {
      valid += idv[j] >= 0 ? 1 : 0;
      sm.w[pad_idx(i)] = (idv[j] >= 0 && scv[j] > -INFINITY) ? exp2f((scv[j] - s0) * log2e_over_t) : 0.0f;
    }
  }
  valid = wave_sum_i(valid);
  if (lane == 0) sm.wint[0][wv] = valid;
  __syncthreads();

  float w[SMP_E], run[SMP_E];
  float local = 0.0f;
#pragma unroll
  for (int j = 0; j < SMP_E; ++j) {
    const int i = i0 + j;
    w[j] = (j < E && i < K) ? sm.w[pad_idx(i)] : 0.0f;
    local += w[j];
    run[j] = local;
  }
  int n_cand = 0;
#pragma unroll
  for (int v = 0; v < SMP_WAVES; ++v) n_cand += sm.wint[0][v];   // candidates are a prefix of the row
  const float incl = wave_inclusive_sum(local, lane);
  if (lane == 63) sm.wsum[wv] = incl;
  __syncthreads();
  float before = incl - local, total = 0.0f;
#pragma unroll
  for (int v = 0; v < SMP_WAVES; ++v) {
    const float x = sm.wsum[v];
    before += v < wv ? x : 0.0f;
    total += x;
  }
#pragma unroll
  for (int j = 0; j < SMP_E; ++j) run[j] += before;

  // nucleus end: first position whose running weight reaches top_p * total
  int n = n_cand;
  if (top_p < 1.0f) {
    const float thr = top_p * total;
    int hit = INT32_MAX;
#pragma unroll
    for (int j = 0; j < SMP_E; ++j) {
      const int i = i0 + j;
      hit = min(hit, (j < E && i < n_cand && run[j] >= thr) ? i : INT32_MAX);
    }
    hit = wave_min_i(hit);
    if (lane == 0) sm.wint[1][wv] = hit;
    __syncthreads();
    hit = INT32_MAX;
#pragma unroll
    for (int v = 0; v < SMP_WAVES; ++v) hit = min(hit, sm.wint[1][v]);
    n = hit != INT32_MAX ? hit + 1 : n_cand;
  }

  // nucleus weight: the running weight at position n - 1, written by the one
  // thread that holds that position (j < E: slots j >= E belong to no one)
  const int jn = (n - 1) - i0;
#pragma unroll
  for (int j = 0; j < SMP_E; ++j)
    if (j < E && j == jn) sm.cn = run[j];
  __syncthreads();
  const float cn = sm.cn;
  const float target = u[b] * cn;

  // draw: first position < n of nonzero weight whose running weight exceeds the target
  int hit = INT32_MAX, last = -1;
#pragma unroll
  for (int j = 0; j < SMP_E; ++j) {
    const int i = i0 + j;
    const bool live = j < E && i < n && w[j] > 0.0f;
    last = live ? i : last;
    hit = min(hit, (live && run[j] > target) ? i : INT32_MAX);
  }
  hit = wave_min_i(hit);
  last = wave_max_i(last);
  if (lane == 0) {
    sm.wint[0][wv] = hit;      // the valid counts were read before the last barrier
    sm.wint[1][wv] = last;
  }
  __syncthreads();
  hit = INT32_MAX;
  last = -1;
#pragma unroll
  for (int v = 0; v < SMP_WAVES; ++v) {
    hit = min(hit, sm.wint[0][v]);
    last = max(last, sm.wint[1][v]);
  }
  const int pos = hit != INT32_MAX ? hit : (last >= 0 ? last : 0);
  const int jp = pos - i0;
#pragma unroll
  for (int j = 0; j < SMP_E; ++j)
    if (j < E && j == jp) sm.wp = w[j];
  __syncthreads();
  if (t == 0) {
    token[b] = ci[pos];
    if (prob) prob[b] = sm.wp / cn;
    if (n_kept) n_kept[b] = n;
  }
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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
  hipError_t e = launch_topk(logits, nullptr, nullptr, B, V, K, cand_idx, cand_score,
                             topk_workspace_bytes(B, V, K) ? tk_ws : nullptr, stream);
  if (e != hipSuccess) return e;
  return launch_sample_draw(cand_idx, cand_score, B, K, temperature, top_p, u, token, prob, n_kept, stream);
}

}  // namespace csa2
