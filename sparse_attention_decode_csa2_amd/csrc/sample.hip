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
// One workgroup of 1024 threads per row, one streaming pass: the row is cut
// into tiles of 16384 tokens (thread t reads the four 16-byte runs at tokens
// 4096 q + 4 t of a tile; four tiles, 16 loads per lane, in flight), and
// every wave keeps, per tile, the largest scaled logit of its 1024 tokens and
// their weights summed relative to it, in LDS.  After one barrier the tile
// totals are rescaled to the row's maximum, a prefix over the tiles finds the
// tile holding u * sum(w), and only that tile is read again, thread t taking
// its 16 consecutive tokens: their weights relative to the row maximum, wave
// scans and the wave totals give every token its running weight, and the
// first one above the target is the draw.  The tile totals and the running
// weights inside the drawn tile are summed in different orders, so float32
// rounding may move a draw whose running weight lies within rounding of the
// target by one token; the drawn token always has nonzero weight.
constexpr int SF_T = 1024;                      // threads per row
constexpr int SF_WAVES = SF_T / 64;
constexpr int SF_PER = 16;                      // tokens per thread and tile
constexpr int SF_TILE = SF_PER * SF_T;          // tokens per tile
constexpr int SF_MAX_TILES = 64;                // V <= 2^20
constexpr int SF_INFLIGHT = 4;                  // tiles loaded per step (16 loads per lane)

struct SfSmem {
  float wm[SF_MAX_TILES][SF_WAVES];             // per tile and wave: largest scaled logit
  float ws[SF_MAX_TILES][SF_WAVES];             // per tile and wave: weights summed relative to it
  float tt[SF_MAX_TILES];                       // tile totals relative to the row maximum
  float wmax[SF_WAVES];
  float wsum[SF_WAVES];
  int hit[SF_WAVES], last[SF_WAVES];
  float target, before, total;
  int tile;
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

template <bool VEC>
__global__ __launch_bounds__(SF_T) void sample_full_kernel(const float* __restrict__ logits, int64_t V,
                                                           float log2e_over_t, const float* __restrict__ u,
                                                           int32_t* __restrict__ token, float* __restrict__ prob) {
  // no fused multiply-add: a scaled logit is rounded once and every later use
  // sees that value (a fused x * c - m would give the maximum itself a weight
  // of exp2 of the product's rounding error instead of exactly one)
#pragma clang fp contract(off)
  __shared__ SfSmem sm;
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* row = logits + b * V;
  const int n_tiles = (int)((V + SF_TILE - 1) / SF_TILE);

  // ---- pass: per tile and wave, (max, sum of weights relative to it)
  float wave_max = -INFINITY;
  for (int j0 = 0; j0 < n_tiles; j0 += SF_INFLIGHT) {
    float x[SF_INFLIGHT][SF_PER];
#pragma unroll
    for (int h = 0; h < SF_INFLIGHT; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sf_load<VEC>(row, V, (int64_t)(j0 + h) * SF_TILE + (SF_TILE / 4) * q + 4 * t, &x[h][4 * q]);
#pragma unroll
    for (int h = 0; h < SF_INFLIGHT; ++h) {
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
      if (lane == 0) {
        sm.wm[j0 + h][wv] = m;
        sm.ws[j0 + h][wv] = sum;
      }
      wave_max = fmaxf(wave_max, m);
    }
  }
  if (lane == 0) sm.wmax[wv] = wave_max;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < SF_WAVES; ++w) M = fmaxf(M, sm.wmax[w]);
  if (M == -INFINITY) {          // every logit -inf (or NaN)
    if (t == 0) {
      token[b] = 0;
      if (prob) prob[b] = 1.0f;
    }
    return;
  }
  // ---- tile totals relative to the row maximum
  for (int j = t; j < n_tiles; j += SF_T) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < SF_WAVES; ++w) {
      const float m = sm.wm[j][w];
      s += m == -INFINITY ? 0.0f : sm.ws[j][w] * exp2f(m - M);
    }
    sm.tt[j] = s;
  }
  __syncthreads();
  // ---- wave 0: prefix over the tiles, the tile holding the target
  if (wv == 0) {
    const float x = lane < n_tiles ? sm.tt[lane] : 0.0f;   // n_tiles <= 64
    const float incl = wave_inclusive_sum(x, lane);
    const float total = __shfl(incl, 63, 64);
    const float target = u[b] * total;
    // only a tile of nonzero weight can hold the draw (the scan's rounding
    // differs between lanes, so an empty tile's running total may still step
    // over the target); if rounding leaves none, the last tile of nonzero weight
    const uint64_t above = __ballot(lane < n_tiles && x > 0.0f && incl > target);
    const uint64_t live = __ballot(lane < n_tiles && x > 0.0f);
    const int tile = above ? __builtin_ctzll(above) : 63 - __builtin_clzll(live);
    const float base = __shfl(incl - x, tile, 64);          // running total before that tile
    if (lane == 0) {
      sm.tile = tile;
      sm.before = base;
      sm.target = target;
      sm.total = total;
    }
  }
  __syncthreads();
  const int tile = sm.tile;
  const float target = sm.target, total = sm.total;
  // ---- the drawn tile again, thread t its 16 consecutive tokens: running weights
  float x[SF_PER];
  const int64_t i0 = (int64_t)tile * SF_TILE + SF_PER * t;
#pragma unroll
  for (int q = 0; q < 4; ++q) sf_load<VEC>(row, V, i0 + 4 * q, &x[4 * q]);
  float w[SF_PER], run[SF_PER], local = 0.0f;
#pragma unroll
  for (int e = 0; e < SF_PER; ++e) {
    const float y = x[e] * log2e_over_t;
    w[e] = y == -INFINITY ? 0.0f : exp2f(y - M);
    local += w[e];
    run[e] = local;
  }
  const float incl = wave_inclusive_sum(local, lane);
  if (lane == 63) sm.wsum[wv] = incl;
  __syncthreads();
  float before = sm.before + incl - local;
#pragma unroll
  for (int v = 0; v < SF_WAVES; ++v) before += v < wv ? sm.wsum[v] : 0.0f;
  int hit = INT32_MAX, last = -1;
#pragma unroll
  for (int e = 0; e < SF_PER; ++e) {
    const int k = SF_PER * t + e;
    last = w[e] > 0.0f ? k : last;
    hit = min(hit, (w[e] > 0.0f && before + run[e] > target) ? k : INT32_MAX);
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
  for (int v = 0; v < SF_WAVES; ++v) {
    hit = min(hit, sm.hit[v]);
    last = max(last, sm.last[v]);
  }
  // the tile has a token of nonzero weight (its total is positive); were every
  // weight to underflow on the second read, its first token is written
  const int k = hit != INT32_MAX ? hit : max(last, 0);
  if (k / SF_PER == t) {
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

int64_t sample_full_launch_items(int B) { return (int64_t)B * SF_T; }

hipError_t launch_sample_full(const float* logits, int B, int64_t V, float temperature, const float* u,
                              int32_t* token, float* prob, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (V > (int64_t)SF_MAX_TILES * SF_TILE) return hipErrorInvalidValue;
  const float log2e_over_t = (float)(1.4426950408889634 / (double)temperature);
  // 16-byte loads when every row starts on a 16-byte boundary
  if (V % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0)
    hipLaunchKernelGGL(sample_full_kernel<true>, dim3(B), dim3(SF_T), 0, stream, logits, V, log2e_over_t, u, token,
                       prob);
  else
    hipLaunchKernelGGL(sample_full_kernel<false>, dim3(B), dim3(SF_T), 0, stream, logits, V, log2e_over_t, u,
                       token, prob);
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
  hipError_t e = launch_topk(logits, nullptr, nullptr, B, V, K, cand_idx, cand_score,
                             topk_workspace_bytes(B, V, K) ? tk_ws : nullptr, stream);
  if (e != hipSuccess) return e;
  return launch_sample_draw(cand_idx, cand_score, B, K, temperature, top_p, u, token, prob, n_kept, stream);
}

}  // namespace csa2
