// a3: Top-K with the lower id winning ties (Top-512 per [P1] 架构三件套, CSA2).
//
// Every candidate becomes one 64-bit key: high word = order-preserving image of
// its fp32 score (-0 folded onto +0, NaN lowest), low word = ~id, so that
// "larger key" is exactly "higher score, then lower id" and an empty candidate
// is key 0.  One workgroup of 1024 threads owns up to 16384 keys (16 per
// thread, in registers):
//
//  1. skip the bits shared by every valid key (block max / min of the high
//     words), then histogram the next 13 bits into 8192 LDS bins and find,
//     with a block scan, the bin holding the K-th largest key.  Keys above that
//     bin are certainly selected ("definite", fewer than K of them); the keys
//     in it are the "boundary" set.  Should the boundary set exceed 2048 keys
//     the next 13 bits of that bin are histogrammed, and so on.
//  2. compact both sets into LDS with one atomic per wave (ballot counts).
//  3. sort each set descending with a bitonic network held in registers
//     (exchanges through DPP / permlane swaps below stride 64, through LDS
//     above); the output is the sorted definite set followed by the largest
//     K - |definite| boundary keys, i.e. (score desc, id asc).
//
// Rows longer than 16384 are cut into 16384-key chunks; each chunk keeps its
// own top K keys (the union of chunk winners contains the row's winners, the
// key order being total) and the winners are reduced again until one chunk
// remains.  Bit-exact by construction: only integer compares and counts.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int TK_T = 1024;
constexpr int TK_E = 16;
constexpr int TK_CHUNK = TK_T * TK_E;
constexpr int TK_BITS = 13;
constexpr int TK_BINS = 1 << TK_BITS;
constexpr int TK_CAP = 2048;  // largest set sorted directly (>= K)
constexpr int TK_WAVES = TK_T / WAVE;

struct TkSmem {
  uint32_t hist[TK_BINS];    // histogram; later parks the sorted definite set
  uint64_t buf[2][TK_CAP];   // [0]: definite set, [1]: boundary set
  uint64_t xbuf[TK_CAP];     // second buffer of the sort's LDS exchanges
  uint32_t wtmp[3][TK_WAVES];
  uint32_t info[8];
};

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Value held by lane (lane ^ M) for M in {1, 2, 4, 8, 16, 32}, via DPP or the
// permlane swaps (no LDS traffic).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (M == 1) {
    return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const uint32_t up = dpp<0x12C>(v), dn = dpp<0x124>(v);  // row_ror 12: lane+4, row_ror 4: lane-4
    return (lane_id() & 4) ? dn : up;
  } else if constexpr (M == 8) {
    return dpp<0x128>(v);  // row_ror 8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane_id() & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane_id() & 32) ? r[0] : r[1];
  }
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  return ((uint64_t)xor_lane<M>((uint32_t)(v >> 32)) << 32) | xor_lane<M>((uint32_t)v);
}

// Wave-wide sum / max / min; every lane gets the result.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += xor_lane<1>(v);
  v += xor_lane<2>(v);
  v += xor_lane<4>(v);
  v += xor_lane<8>(v);
  v += xor_lane<16>(v);
  v += xor_lane<32>(v);
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, xor_lane<1>(v));
  v = max(v, xor_lane<2>(v));
  v = max(v, xor_lane<4>(v));
  v = max(v, xor_lane<8>(v));
  v = max(v, xor_lane<16>(v));
  v = max(v, xor_lane<32>(v));
  return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  v = min(v, xor_lane<1>(v));
  v = min(v, xor_lane<2>(v));
  v = min(v, xor_lane<4>(v));
  v = min(v, xor_lane<8>(v));
  v = min(v, xor_lane<16>(v));
  v = min(v, xor_lane<32>(v));
  return v;
}

// Inclusive prefix sum across the wave: row shifts, then row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr 1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr 2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr 4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr 8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast 15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast 31
  return v;
}

// ---------------------------------------------------------------- block ops

// Block-wide (sum of a, max of b, min of c); every thread gets the results.
__device__ __forceinline__ void block_sum_max_min(uint32_t& a, uint32_t& b, uint32_t& c, TkSmem& sm) {
  const int wave = threadIdx.x >> 6;
  a = wave_sum(a);
  b = wave_max(b);
  c = wave_min(c);
  if (lane_id() == 0) {
    sm.wtmp[0][wave] = a;
    sm.wtmp[1][wave] = b;
    sm.wtmp[2][wave] = c;
  }
  __syncthreads();
  a = 0;
  b = 0;
  c = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    a += sm.wtmp[0][i];
    b = max(b, sm.wtmp[1][i]);
    c = min(c, sm.wtmp[2][i]);
  }
  __syncthreads();
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, TkSmem& sm) {
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane_id() == 63) sm.wtmp[0][wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    const uint32_t s = sm.wtmp[0][i];
    before += i < wave ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Appends the keys for which pick(e) holds to an LDS list; one atomic per wave.
template <typename Pred>
__device__ __forceinline__ void wave_compact(const uint64_t (&key)[TK_E], Pred pick, uint32_t* counter,
                                             uint64_t* list, uint32_t cap) {
  uint64_t m[TK_E];
  uint32_t tot = 0;
#pragma unroll
  for (int e = 0; e < TK_E; ++e) {
    m[e] = __ballot(pick(e));
    tot += (uint32_t)__popcll(m[e]);
  }
  uint32_t base = 0;
  if (tot != 0) {
    if (lane_id() == 0) base = atomicAdd(counter, tot);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  }
#pragma unroll
  for (int e = 0; e < TK_E; ++e) {
    const uint32_t below =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], 0u));
    const uint32_t slot = base + below;
    if (((m[e] >> lane_id()) & 1ull) && slot < cap) list[slot] = key[e];
    base += (uint32_t)__popcll(m[e]);
  }
}

// ---------------------------------------------------------------- sort

// New value of element i after the (SIZE, STRIDE) compare-exchange with its
// partner value p: the lower element of a descending pair keeps the maximum.
template <int SIZE, int STRIDE>
__device__ __forceinline__ uint64_t cmpx(uint64_t v, uint64_t p, int i) {
  const bool lower = (i & STRIDE) == 0;
  const bool desc = (i & SIZE) == 0;
  const bool gt = v > p;
  return (gt == (lower == desc)) ? v : p;
}

template <int SIZE, int STRIDE, int N>
__device__ __forceinline__ void sort_stage(uint64_t (&v)[2], TkSmem& sm, int& pb) {
  constexpr int SLOTS = N > TK_T ? 2 : 1;
  const int tid = threadIdx.x;
  const bool active = tid < N;
  if constexpr (STRIDE >= WAVE && STRIDE < TK_T) {
    uint64_t* x = pb ? sm.xbuf : sm.buf[0];
    if (active) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) x[tid + TK_T * s] = v[s];
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        const int i = tid + TK_T * s;
        v[s] = cmpx<SIZE, STRIDE>(v[s], x[i ^ STRIDE], i);
      }
    }
    pb ^= 1;
  } else if constexpr (STRIDE == TK_T) {
    if (active) {
      const uint64_t a = v[0], b = v[1];
      v[0] = cmpx<SIZE, STRIDE>(a, b, tid);
      v[1] = cmpx<SIZE, STRIDE>(b, a, tid + TK_T);
    }
  } else {
    if (active) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        v[s] = cmpx<SIZE, STRIDE>(v[s], xor_lane64<STRIDE>(v[s]), tid + TK_T * s);
    }
  }
}

template <int SIZE, int STRIDE, int N>
__device__ __forceinline__ void sort_merge(uint64_t (&v)[2], TkSmem& sm, int& pb) {
  sort_stage<SIZE, STRIDE, N>(v, sm, pb);
  if constexpr (STRIDE > 1) sort_merge<SIZE, STRIDE / 2, N>(v, sm, pb);
}

template <int SIZE, int N>
__device__ __forceinline__ void sort_sizes(uint64_t (&v)[2], TkSmem& sm, int& pb) {
  sort_merge<SIZE, SIZE / 2, N>(v, sm, pb);
  if constexpr (SIZE < N) sort_sizes<SIZE * 2, N>(v, sm, pb);
}

// Sorts sm.buf[0][0 .. N) descending (N a power of two in [64, 2048]; entries
// past the live ones must be 0).  Element i lives in thread i % 1024, slot
// i / 1024; the LDS exchange stages alternate between sm.buf[0] and sm.xbuf.
template <int N>
__device__ void sort_desc(TkSmem& sm) {
  constexpr int SLOTS = N > TK_T ? 2 : 1;
  const int tid = threadIdx.x;
  uint64_t v[2] = {0ull, 0ull};
  __syncthreads();
  if (tid < N) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) v[s] = sm.buf[0][tid + TK_T * s];
  }
  __syncthreads();
  int pb = 0;
  sort_sizes<2, N>(v, sm, pb);
  __syncthreads();
  if (tid < N) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) sm.buf[0][tid + TK_T * s] = v[s];
  }
  __syncthreads();
}

__device__ void sort_desc_n(int n, TkSmem& sm) {
  switch (n) {
    case 64: sort_desc<64>(sm); break;
    case 128: sort_desc<128>(sm); break;
    case 256: sort_desc<256>(sm); break;
    case 512: sort_desc<512>(sm); break;
    case 1024: sort_desc<1024>(sm); break;
    default: sort_desc<2048>(sm); break;
  }
}

// ---------------------------------------------------------------- select

struct TkResult {
  uint32_t n_def;  // sorted definite keys at sm.buf[0][0 .. n_def)
  uint32_t n_bnd;  // sorted boundary keys at sm.buf[1][0 .. n_bnd)
  uint32_t count;  // min(K, #valid keys)
};

// Top K of the non-zero keys held by the block (TK_E per thread).
__device__ TkResult block_topk(uint64_t (&key)[TK_E], int K, TkSmem& sm) {
  const int tid = threadIdx.x;
  uint32_t n_all = 0, hmax = 0, hmin = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < TK_E; ++e) {
    if (key[e] != 0) {
      const uint32_t hi = (uint32_t)(key[e] >> 32);
      ++n_all;
      hmax = max(hmax, hi);
      hmin = min(hmin, hi);
    }
  }
  if (tid == 0) {
    sm.info[4] = 0;
    sm.info[5] = 0;
  }
  block_sum_max_min(n_all, hmax, hmin, sm);

  // definite: key > t_def; boundary: t_lo <= key <= t_def
  uint64_t t_def = ~0ull, t_lo = 1ull;
  bool dup = false;
  if (n_all > (uint32_t)K) {
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
    uint32_t r = (uint32_t)K;  // rank of the K-th key inside the current region
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
      // thread t owns bins [t*bpt, t*bpt + bpt); ranks count from the top bin
      const int bpt = nbins >= TK_T ? nbins / TK_T : 1;
      const int b0 = tid * bpt;
      uint32_t mine = 0;
      if (b0 < nbins)
        for (int i = 0; i < bpt; ++i) mine += sm.hist[b0 + i];
      uint32_t total;
      const uint32_t excl = block_excl_scan(mine, &total, sm);
      uint32_t above = total - excl - mine;
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
      t_lo = prefix;
      t_def = prefix | ((1ull << lo) - 1ull);
      if (n_eq <= (uint32_t)TK_CAP) break;
      if (lo == 0) {  // one exact key repeated more than TK_CAP times
        dup = true;
        break;
      }
      top = lo - 1;
    }
  }
  // compact: definite -> buf[0], boundary -> buf[1]
  wave_compact(key, [&](int e) { return key[e] > t_def; }, &sm.info[4], sm.buf[0], TK_CAP);
  wave_compact(key, [&](int e) { return key[e] != 0 && key[e] >= t_lo && key[e] <= t_def; }, &sm.info[5],
               sm.buf[1], TK_CAP);
  __syncthreads();
  TkResult res;
  res.n_def = sm.info[4];
  res.n_bnd = min(sm.info[5], (uint32_t)TK_CAP);
  res.count = min(n_all, (uint32_t)K);
  __syncthreads();
  // sort the definite set in place
  if (res.n_def > 0) {
    int n = 64;
    while (n < (int)res.n_def) n <<= 1;
    for (int j = (int)res.n_def + tid; j < n; j += TK_T) sm.buf[0][j] = 0ull;
    sort_desc_n(n, sm);
  }
  // sort the boundary set (identical keys when dup): park the definite keys in
  // the histogram area (<= 2047 keys fit in its 32 KiB), sort through buf[0]
  if (!dup && res.n_bnd > 1 && res.n_def < (uint32_t)K) {
    uint64_t* park = reinterpret_cast<uint64_t*>(sm.hist);
    for (int j = tid; j < (int)res.n_def; j += TK_T) park[j] = sm.buf[0][j];
    int nb = 64;
    while (nb < (int)res.n_bnd) nb <<= 1;
    __syncthreads();
    for (int j = tid; j < nb; j += TK_T) sm.buf[0][j] = j < (int)res.n_bnd ? sm.buf[1][j] : 0ull;
    sort_desc_n(nb, sm);
    for (int j = tid; j < (int)res.n_bnd; j += TK_T) sm.buf[1][j] = sm.buf[0][j];
    for (int j = tid; j < (int)res.n_def; j += TK_T) sm.buf[0][j] = park[j];
    __syncthreads();
  }
  return res;
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
  const TkResult res = block_topk(key, K, sm);
  // output position j: definite keys first, then the boundary keys
  for (int j = tid; j < K; j += TK_T) {
    uint64_t k = 0;
    if (j < (int)res.count)
      k = j < (int)res.n_def ? sm.buf[0][j] : sm.buf[1][min(j - (int)res.n_def, TK_CAP - 1)];
    if (FINAL) {
      const bool ok = j < (int)res.count;
      out_idx[b * K + j] = ok ? (int32_t)(~(uint32_t)k) : -1;
      if (out_score) out_score[b * K + j] = ok ? key_score((uint32_t)(k >> 32)) : -INFINITY;
    } else {
      keys_out[(b * chunks + c) * (int64_t)K + j] = k;
    }
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
