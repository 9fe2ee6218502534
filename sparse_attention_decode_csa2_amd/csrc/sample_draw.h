// The decode sampler's draw over a row's Top-K candidates, as a block-level
// function: the draw kernel runs it with a workgroup of SMP_T threads per
// row, and the Top-K's last kernel can run it after writing a row's
// candidates (same arithmetic, so both give the same draw).  The method and
// the layout of the work are described with the draw kernel in sample.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace csa2 {

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

// The draw of row b over its candidates ci / cs (Top-K order), by threads
// 0 .. SMP_T - 1 of the workgroup; the workgroup's other threads (a larger
// workgroup that calls it after its own work) pass the same barriers and do
// nothing else.  Every thread of the workgroup must call it.
__device__ __forceinline__ void sample_draw_row(int64_t b, const int32_t* __restrict__ ci,
                                                const float* __restrict__ cs, int K, float log2e_over_t,
                                                float top_p, const float* __restrict__ u,
                                                int32_t* __restrict__ token, float* __restrict__ prob,
                                                int32_t* __restrict__ n_kept, SmpSmem& sm) {
  const bool act = threadIdx.x < SMP_T;
  const int t = act ? threadIdx.x : 0;      // an idle thread mirrors thread 0's loads
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int E = (K + SMP_T - 1) / SMP_T;
  const int i0 = act ? t * E : K;           // an idle thread holds no element
  const float s0 = cs[0];
  const int32_t id0 = ci[0];
  if (!(s0 > -INFINITY) || id0 < 0) {   // every logit -inf, NaN at the top, or no candidate
    if (threadIdx.x == 0) {
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
    if (act && i < K) {
      valid += idv[j] >= 0 ? 1 : 0;
      sm.w[pad_idx(i)] = (idv[j] >= 0 && scv[j] > -INFINITY) ? exp2f((scv[j] - s0) * log2e_over_t) : 0.0f;
    }
  }
  valid = wave_sum_i(valid);
  if (act && lane == 0) sm.wint[0][wv] = valid;
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
  if (act && lane == 63) sm.wsum[wv] = incl;
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
    if (act && lane == 0) sm.wint[1][wv] = hit;
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
  if (act && lane == 0) {
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
  if (threadIdx.x == 0) {
    token[b] = ci[pos];
    if (prob) prob[b] = sm.wp / cn;
    if (n_kept) n_kept[b] = n;
  }
}


}  // namespace csa2
