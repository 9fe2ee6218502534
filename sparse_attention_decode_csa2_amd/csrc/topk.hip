// a3: Top-K with the lower id winning ties (Top-512 per [P1] 架构三件套, CSA2).
//
// Every candidate becomes one 64-bit key: high word = order-preserving image of
// its fp32 score (-0 folded onto +0, NaN lowest), low word = ~id, so that
// "larger key" is exactly "higher score, then lower id" and an empty candidate
// is key 0.  Selecting the K largest keys is then a plain radix select:
//
//  * a workgroup of 1024 threads holds up to 16384 keys in registers;
//  * the bits above the highest bit where the largest and smallest valid
//    score differ are common to all candidates and are skipped;
//  * each pass histograms the next 12 bits (4096 LDS bins) of the keys that
//    still match the resolved prefix, finds the bin holding the K-th key with
//    a block scan, and stops early once that bin is taken whole;
//  * the selected keys are compacted into LDS and, on the final level, sorted
//    descending with a bitonic network, which yields (score desc, id asc).
//
// Rows longer than 16384 are cut into 16384-key chunks; each chunk keeps its
// own top K keys (the union of chunk winners contains the row's winners, the
// key order being total), and the winners are reduced again until one chunk
// remains.  Bit-exact by construction: only integer compares and counts.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int TK_T = 1024;
constexpr int TK_E = 16;
constexpr int TK_CHUNK = TK_T * TK_E;
constexpr int TK_BITS = 12;
constexpr int TK_BINS = 1 << TK_BITS;
constexpr int TK_KMAX = 2048;
constexpr int TK_WAVES = TK_T / WAVE;

struct TkSmem {
  uint32_t hist[TK_BINS];
  uint64_t sel[TK_KMAX];
  uint32_t wtmp[TK_WAVES];
  uint32_t info[8];
};

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o));
  return v;
}

// op: 0 sum, 1 max, 2 min.  All threads get the result.
template <int OP>
__device__ __forceinline__ uint32_t block_reduce(uint32_t v, TkSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = OP == 0 ? wave_sum(v) : (OP == 1 ? wave_max(v) : wave_min(v));
  if (lane == 0) sm.wtmp[wave] = v;
  __syncthreads();
  uint32_t r = sm.wtmp[0];
#pragma unroll
  for (int i = 1; i < TK_WAVES; ++i) r = OP == 0 ? r + sm.wtmp[i] : (OP == 1 ? max(r, sm.wtmp[i]) : min(r, sm.wtmp[i]));
  __syncthreads();
  return r;
}

// Inclusive prefix sum over the block in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* total, TkSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) sm.wtmp[wave] = v;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    const uint32_t s = sm.wtmp[i];
    before += i < wave ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Selects the K largest non-zero keys held by the block (TK_E per thread) into
// sm.sel[0 .. count) in no particular order; returns count = min(K, #non-zero).
__device__ int block_select(uint64_t (&key)[TK_E], int K, TkSmem& sm) {
  const int tid = threadIdx.x;
  uint32_t cnt = 0, hmax = 0, hmin = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < TK_E; ++e) {
    if (key[e] != 0) {
      const uint32_t hi = (uint32_t)(key[e] >> 32);
      ++cnt;
      hmax = max(hmax, hi);
      hmin = min(hmin, hi);
    }
  }
  const uint32_t n_all = block_reduce<0>(cnt, sm);
  if (tid == 0) { sm.info[4] = 0; sm.info[5] = 0; }
  if (n_all <= (uint32_t)K) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if (key[e] != 0) {
        const uint32_t slot = atomicAdd(&sm.info[4], 1u);
        if (slot < (uint32_t)TK_KMAX) sm.sel[slot] = key[e];
      }
    }
    __syncthreads();
    return (int)n_all;
  }
  hmax = block_reduce<1>(hmax, sm);
  hmin = block_reduce<2>(hmin, sm);

  // bits above `top` are shared by every valid key
  int top;
  uint64_t prefix, pmask;
  const uint32_t diff = hmax ^ hmin;
  if (diff) {
    top = 32 + 31 - __clz(diff);
    pmask = ~((2ull << top) - 1ull);
  } else {
    top = 31;
    pmask = 0xFFFFFFFF00000000ull;
  }
  prefix = ((uint64_t)hmax << 32) & pmask;
  uint32_t r = (uint32_t)K;  // rank still to place among keys matching prefix
  bool take_ge = false;
  for (;;) {
    const int width = min(TK_BITS, top + 1);
    const int lo = top - width + 1;
    const int nbins = 1 << width;
    for (int i = tid; i < nbins; i += TK_T) sm.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if (key[e] != 0 && (key[e] & pmask) == prefix)
        atomicAdd(&sm.hist[(uint32_t)(key[e] >> lo) & (uint32_t)(nbins - 1)], 1u);
    }
    __syncthreads();
    // bins [tid*bpt, tid*bpt + bpt) per thread; find the bin holding rank r from the top
    const int bpt = nbins >= TK_T ? nbins / TK_T : 1;
    const int b0 = tid * bpt;
    uint32_t mine = 0;
    if (b0 < nbins)
      for (int i = 0; i < bpt; ++i) mine += sm.hist[b0 + i];
    uint32_t total;
    const uint32_t incl = block_incl_scan(mine, &total, sm);
    uint32_t above = total - incl;  // keys in bins above my range
    if (b0 < nbins) {
      for (int d = b0 + bpt - 1; d >= b0; --d) {
        const uint32_t h = sm.hist[d];
        if (above < r && above + h >= r) {
          sm.info[0] = (uint32_t)d;
          sm.info[1] = above;
          sm.info[2] = h;
        }
        above += h;
      }
    }
    __syncthreads();
    const uint32_t d = sm.info[0], n_above = sm.info[1], n_eq = sm.info[2];
    __syncthreads();
    prefix |= (uint64_t)d << lo;
    pmask |= (uint64_t)(nbins - 1) << lo;
    r -= n_above;
    if (n_eq == r) { take_ge = true; break; }  // the whole bin is selected
    if (lo == 0) break;                        // prefix is the K-th key itself
    top = lo - 1;
  }
  if (take_ge) {
    // exactly K keys are >= prefix (lower bits of prefix are zero)
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if (key[e] != 0 && key[e] >= prefix) {
        const uint32_t slot = atomicAdd(&sm.info[4], 1u);
        if (slot < (uint32_t)K) sm.sel[slot] = key[e];
      }
    }
  } else {
    // K - r keys are larger than the K-th key; r copies of it (equal keys are
    // identical (score, id) pairs, so any r of them give the same output)
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      if (key[e] > prefix) {
        const uint32_t slot = atomicAdd(&sm.info[4], 1u);
        if (slot < (uint32_t)K) sm.sel[slot] = key[e];
      } else if (key[e] == prefix) {
        const uint32_t s = atomicAdd(&sm.info[5], 1u);
        if (s < r) sm.sel[K - r + s] = key[e];
      }
    }
  }
  __syncthreads();
  return K;
}

// Bitonic sort of sm.sel[0 .. kp) into descending order (kp a power of two).
__device__ void block_sort_desc(int kp, TkSmem& sm) {
  for (int size = 2; size <= kp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (kp >> 1); i += TK_T) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = sm.sel[lo], c = sm.sel[hi];
        if (desc ? (a < c) : (a > c)) {
          sm.sel[lo] = c;
          sm.sel[hi] = a;
        }
      }
      __syncthreads();
    }
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
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x / chunks;
  const int c = (int)(blockIdx.x - b * chunks);
  const int64_t base = (int64_t)c * TK_CHUNK;
  int64_t limit = min<int64_t>(M, base + TK_CHUNK);
  uint64_t key[TK_E];
  if (FROM_SCORES) {
    if (n_valid) limit = min<int64_t>(limit, max<int64_t>(n_valid[b], 0));
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      const int64_t col = base + (int64_t)e * TK_T + tid;
      uint64_t k = 0;
      if (col < limit) {
        const float s = scores[b * M + col];
        const int32_t id = ids ? ids[b * M + col] : (int32_t)col;
        if (id != -1) k = ((uint64_t)score_key(s) << 32) | (uint64_t)(~(uint32_t)id);
      }
      key[e] = k;
    }
  } else {
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      const int64_t col = base + (int64_t)e * TK_T + tid;
      key[e] = col < limit ? keys_in[b * M + col] : 0ull;
    }
  }
  const int count = block_select(key, K, sm);
  if (FINAL) {
    int kp = 1;
    while (kp < K) kp <<= 1;
    for (int j = count + tid; j < kp; j += TK_T) sm.sel[j] = 0ull;
    __syncthreads();
    block_sort_desc(kp, sm);
    for (int j = tid; j < K; j += TK_T) {
      const uint64_t k = sm.sel[j];
      const bool ok = j < count;
      out_idx[b * K + j] = ok ? (int32_t)(~(uint32_t)k) : -1;
      if (out_score) out_score[b * K + j] = ok ? key_score((uint32_t)(k >> 32)) : -INFINITY;
    }
  } else {
    uint64_t* dst = keys_out + (b * chunks + c) * (int64_t)K;
    for (int j = tid; j < K; j += TK_T) dst[j] = j < count ? sm.sel[j] : 0ull;
  }
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

size_t topk_workspace_bytes(int B, int64_t M, int K) {
  int64_t ch[16];
  const int n = topk_levels(M, K, ch, 16);
  size_t bytes = 0;
  for (int l = 0; l + 1 < n; ++l) bytes += (size_t)B * ch[l] * K * sizeof(uint64_t);
  return bytes;
}

hipError_t launch_topk(const float* scores, const int32_t* ids, const int32_t* n_valid, int B,
                       int64_t M, int K, int32_t* out_idx, float* out_score, void* workspace,
                       hipStream_t stream) {
  if (B == 0) return hipSuccess;
  int64_t ch[16];
  const int n = topk_levels(M, K, ch, 16);
  if (n > 16) return hipErrorInvalidValue;
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  const uint64_t* prev = nullptr;
  int64_t m = M;
  for (int l = 0; l < n; ++l) {
    const bool last = l + 1 == n;
    const dim3 grid((unsigned)(B * ch[l]));
    if (l == 0 && last) {
      hipLaunchKernelGGL((topk_kernel<true, true>), grid, dim3(TK_T), 0, stream, scores, ids, n_valid,
                         nullptr, m, K, 1, nullptr, out_idx, out_score);
    } else if (l == 0) {
      hipLaunchKernelGGL((topk_kernel<true, false>), grid, dim3(TK_T), 0, stream, scores, ids, n_valid,
                         nullptr, m, K, (int)ch[l], ws, nullptr, nullptr);
    } else if (last) {
      hipLaunchKernelGGL((topk_kernel<false, true>), grid, dim3(TK_T), 0, stream, nullptr, nullptr,
                         nullptr, prev, m, K, 1, nullptr, out_idx, out_score);
    } else {
      hipLaunchKernelGGL((topk_kernel<false, false>), grid, dim3(TK_T), 0, stream, nullptr, nullptr,
                         nullptr, prev, m, K, (int)ch[l], ws, nullptr, nullptr);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!last) {
      prev = ws;
      ws += (size_t)B * ch[l] * K;
      m = ch[l] * K;
    }
  }
  return hipSuccess;
}

}  // namespace csa2
