// a3: block-level Top-K with the lower id winning ties (Top-512 per [P1]
// 架构三件套, CSA2), shared by the Top-K kernels and the fused indexer.
//
// Every candidate becomes one 64-bit key: high word = order-preserving image of
// its fp32 score (-0 folded onto +0, NaN lowest), low word = ~id, so that
// "larger key" is exactly "higher score, then lower id" and an empty candidate
// is key 0.  One workgroup of 1024 threads owns up to 16384 candidates, thread
// t the 16 consecutive columns [16t, 16t + 16) of its chunk, held in registers
// as fp32 scores and ids (thread order is column order):
//
//  1. a block reduction gives the number of valid candidates and the highest
//     and lowest score;
//  2. linear score buckets (the first path): when both ends are finite and
//     distinct, bucket (s - lo) * 2048 / (hi - lo) is monotone in the score;
//     one LDS histogram and one suffix scan give the bucket holding the K-th
//     largest key and where every bucket's keys start in the output order;
//  3. the keys of the buckets above it (and of it, when it holds at most 2048)
//     are staged wave by wave into LDS and placed bucket by bucket; a key's
//     output slot is its bucket's start plus its rank among the keys of its
//     bucket, and one wave orders the boundary bucket (counting ranks up to
//     24 keys, a bitonic network up to 64) and keeps its first r keys;
//  4. exact fallbacks: a selected bucket longer than 32 keys -> bitonic sort
//     of the K keys; a boundary bucket of 65-2048 keys -> radix select on its
//     keys (ties by radix select on ~id); more than 2048 keys in one bucket,
//     non-finite ends or NaN-only rows -> radix selection on the 32-bit score
//     keys of the whole chunk (11-bit digits, suffix scans; a tie on one score
//     cut by id) and a bitonic network (DPP / permlane exchanges below stride
//     64, LDS above) that sorts the K keys descending.
//
// Rows longer than 16384 are cut into 16384-key chunks; each chunk keeps its
// own top K keys, unsorted (the union of chunk winners contains the row's
// winners, the key order being total) and the winners are reduced again
// until one chunk remains.  The bucket index is an fp32 computation that only
// routes keys; every order decision is an integer compare of the 64-bit keys,
// so the result is bit-exact.
#pragma once

#include "csa2_device.h"

namespace csa2 {

constexpr int TK_T = 1024;
constexpr int TK_E = 16;
constexpr int TK_CHUNK = TK_T * TK_E;
constexpr int TK_BITS = 11;
constexpr int TK_BINS = 1 << TK_BITS;
constexpr int TK_KMAX = 2048;            // largest K, largest candidate set
constexpr int TK_CE = TK_KMAX / TK_T;    // candidates per thread
constexpr int TK_WAVES = TK_T / WAVE;
static_assert(TK_WAVES <= 16, "block ops combine the wave partials in one 16-lane row");

struct TkSmem {
  uint32_t hist[TK_BINS + WAVE];  // radix histogram + one dummy bin per lane
  uint32_t lcnt[TK_BINS + WAVE];  // score-bucket histogram + one dummy bin per lane
  uint32_t lcur[TK_BINS];         // score-bucket output cursors
  uint16_t lbk[TK_KMAX];          // bucket of each key in buf
  uint64_t stage[2 * TK_KMAX];    // (score bits, id) of the entries placed by score buckets
  uint64_t buf[TK_KMAX];          // the selected keys
  uint64_t xbuf[TK_KMAX];         // candidates; second buffer of the sort's LDS exchanges
  uint32_t wtmp[2][3][TK_WAVES];  // wave partials of block ops, two alternating sets
  uint32_t info[5];
};

// LDS state every selection starts from: the histograms zero, no long
// bucket seen, the staging cursor at zero.  Ordered before its first use by
// the barrier of the selection's first block reduction.
__device__ __forceinline__ void tk_init(TkSmem& sm) {
  for (int i = threadIdx.x; i < TK_BINS; i += TK_T) {
    sm.hist[i] = 0;  // radix passes keep it zero
    sm.lcnt[i] = 0;
  }
  if (threadIdx.x == 0) {
    sm.info[3] = 0;
    sm.info[4] = 0;
  }
}

typedef uint64_t lanemask;  // one bit per element a thread holds

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

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

// Inclusive prefix over each 16-lane row (lanes shifted in from outside the
// row read `ident`): lane 15 of a row holds the row's whole reduction.
template <typename Op>
__device__ __forceinline__ uint32_t row_incl(uint32_t v, uint32_t ident, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x111, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x112, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x114, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x118, 0xF, 0xF, false));
  return v;
}

// Reduction over the wave, returned to every lane (formed in lane 63 by the
// row prefixes and two row broadcasts).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, uint32_t ident, Op op) {
  v = row_incl(v, ident, op);
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x142, 0xA, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
// fp32 max / min on the bit patterns; a NaN operand is ignored, so NaN is the identity
struct OpFMax {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }
};
struct OpFMin {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }
};
constexpr uint32_t F_NAN = 0x7FC00000u;

// ---------------------------------------------------------------- block ops
//
// The wave partials go through LDS once; every wave combines them in the
// lanes of one row with DPP and broadcasts the result with readlane.  Block
// ops alternate between two sets of partials (`par`, identical in every
// thread), so each needs a single barrier: a set is rewritten two ops later,
// after a barrier every thread has passed only once done reading it.

// Block-wide reductions of a, b and c under the operations OA, OB, OC (with
// identities ia, ib, ic); every thread gets the results.
template <typename OA, typename OB, typename OC>
__device__ __forceinline__ void block_reduce3(uint32_t& a, uint32_t& b, uint32_t& c, uint32_t ia, uint32_t ib,
                                              uint32_t ic, TkSmem& sm, int& par) {
  const int wave = wave_id();
  a = wave_reduce(a, ia, OA());
  b = wave_reduce(b, ib, OB());
  c = wave_reduce(c, ic, OC());
  uint32_t(&w)[3][TK_WAVES] = sm.wtmp[par];
  if (lane_id() == 0) {
    w[0][wave] = a;
    w[1][wave] = b;
    w[2][wave] = c;
  }
  __syncthreads();
  const int l = lane_id() & 15;
  const bool in = l < TK_WAVES;
  a = row_incl(in ? w[0][in ? l : 0] : ia, ia, OA());
  b = row_incl(in ? w[1][in ? l : 0] : ib, ib, OB());
  c = row_incl(in ? w[2][in ? l : 0] : ic, ic, OC());
  a = (uint32_t)__builtin_amdgcn_readlane((int)a, TK_WAVES - 1);
  b = (uint32_t)__builtin_amdgcn_readlane((int)b, TK_WAVES - 1);
  c = (uint32_t)__builtin_amdgcn_readlane((int)c, TK_WAVES - 1);
  par ^= 1;
}

// Block-wide (sum of a, max of b, min of c).
__device__ __forceinline__ void block_sum_max_min(uint32_t& a, uint32_t& b, uint32_t& c, TkSmem& sm,
                                                  int& par) {
  block_reduce3<OpAdd, OpMax, OpMin>(a, b, c, 0u, 0u, 0xFFFFFFFFu, sm, par);
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, TkSmem& sm, int& par) {
  const int wave = wave_id();
  const uint32_t incl = wave_incl_scan(v);
  uint32_t(&w)[3][TK_WAVES] = sm.wtmp[par];
  if (lane_id() == 63) w[0][wave] = incl;
  __syncthreads();
  const int l = lane_id() & 15;
  const uint32_t x = row_incl(l < TK_WAVES ? w[0][l < TK_WAVES ? l : 0] : 0u, 0u, OpAdd());
  const uint32_t before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)x, wave - 1) : 0u;
  *total = (uint32_t)__builtin_amdgcn_readlane((int)x, TK_WAVES - 1);
  par ^= 1;
  return before + incl - v;
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

template <int N>
constexpr int sort_slots() { return N > TK_T ? N / TK_T : 1; }

// Element i of the N being sorted lives in thread i % TK_T, slot i / TK_T.
template <int SIZE, int STRIDE, int N>
__device__ __forceinline__ void sort_stage(uint64_t (&v)[sort_slots<N>()], TkSmem& sm, int& pb) {
  constexpr int SLOTS = sort_slots<N>();
  const int tid = threadIdx.x;
  const bool active = tid < N;
  if constexpr (STRIDE >= TK_T) {
    // partner in another slot of the same thread
    constexpr int SS = STRIDE / TK_T;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      if ((s & SS) == 0) {
        const uint64_t a = v[s], b = v[s | SS];
        v[s] = cmpx<SIZE, STRIDE>(a, b, tid + TK_T * s);
        v[s | SS] = cmpx<SIZE, STRIDE>(b, a, tid + TK_T * (s | SS));
      }
    }
  } else if constexpr (STRIDE >= WAVE) {
    uint64_t* x = pb ? sm.xbuf : sm.buf;
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
  } else {
    if (active) {
#pragma unroll
      for (int s = 0; s < SLOTS; ++s)
        v[s] = cmpx<SIZE, STRIDE>(v[s], xor_lane64<STRIDE>(v[s]), tid + TK_T * s);
    }
  }
}

template <int SIZE, int STRIDE, int N>
__device__ __forceinline__ void sort_merge(uint64_t (&v)[sort_slots<N>()], TkSmem& sm, int& pb) {
  sort_stage<SIZE, STRIDE, N>(v, sm, pb);
  if constexpr (STRIDE > 1) sort_merge<SIZE, STRIDE / 2, N>(v, sm, pb);
}

template <int SIZE, int N>
__device__ __forceinline__ void sort_sizes(uint64_t (&v)[sort_slots<N>()], TkSmem& sm, int& pb) {
  sort_merge<SIZE, SIZE / 2, N>(v, sm, pb);
  if constexpr (SIZE < N) sort_sizes<SIZE * 2, N>(v, sm, pb);
}

// Sorts sm.buf[0 .. N) descending (N a power of two in [64, 2048]; entries
// past the live ones must be 0); the LDS exchange stages alternate between
// sm.buf and sm.xbuf.
template <int N>
__device__ void sort_desc(TkSmem& sm) {
  constexpr int SLOTS = sort_slots<N>();
  const int tid = threadIdx.x;
  uint64_t v[SLOTS];
  __syncthreads();
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) v[s] = tid < N ? sm.buf[tid + TK_T * s] : 0ull;
  __syncthreads();
  int pb = 0;
  sort_sizes<2, N>(v, sm, pb);
  __syncthreads();
  if (tid < N) {
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) sm.buf[tid + TK_T * s] = v[s];
  }
  __syncthreads();
}

__device__ inline void sort_desc_n(int n, TkSmem& sm) {
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
//
// The helpers below work on E values per thread (E = 16 for a whole chunk,
// E = 2 for the compacted candidates), thread t holding positions
// E*t .. E*t + E - 1, so thread order is position order.

// One radix pass over the values v[e] with act bit e set and (v & pmask) ==
// prefix: histogram of bits [lo, lo + width) and a suffix scan.  Returns, in
// *d / *n_above / *n_eq, the bin holding the r-th largest such value (r >= 1),
// the number of values in higher bins and the number in that bin.  The
// histogram is all zero on entry and is left so: each thread reads only the
// bins it owns and clears them after use.
template <int E>
__device__ __forceinline__ void radix_pass(const uint32_t (&v)[E], lanemask act, uint32_t prefix,
                                           uint32_t pmask, int lo, int width, uint32_t r, TkSmem& sm,
                                           int& par, uint32_t* d, uint32_t* n_above, uint32_t* n_eq) {
  const int tid = threadIdx.x;
  const int nbins = 1 << width;
  // inactive values count into the lane's own dummy bin: no branches and no
  // collisions between lanes on a shared dummy
  const uint32_t dummy = TK_BINS + (uint32_t)lane_id();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = ((act >> e) & 1u) && (v[e] & pmask) == prefix;
    atomicAdd(&sm.hist[in ? (v[e] >> lo) & (uint32_t)(nbins - 1) : dummy], 1u);
  }
  __syncthreads();
  // thread t owns bins [t*bpt, t*bpt + bpt); ranks count from the top bin
  const int bpt = nbins >= TK_T ? nbins / TK_T : 1;
  const int b0 = tid * bpt;
  uint32_t h[TK_BINS / TK_T > 0 ? TK_BINS / TK_T : 1];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < (TK_BINS / TK_T > 0 ? TK_BINS / TK_T : 1); ++i) {
    h[i] = (i < bpt && b0 < nbins) ? sm.hist[b0 + i] : 0u;
    mine += h[i];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan(mine, &total, sm, par);
  uint32_t above = total - excl - mine;
#pragma unroll
  for (int i = (TK_BINS / TK_T > 0 ? TK_BINS / TK_T : 1) - 1; i >= 0; --i) {
    if (i < bpt && b0 < nbins) {
      if (above < r && above + h[i] >= r) {
        sm.info[0] = (uint32_t)(b0 + i);
        sm.info[1] = above;
        sm.info[2] = h[i];
      }
      above += h[i];
      sm.hist[b0 + i] = 0;
    }
  }
  __syncthreads();
  *d = sm.info[0];
  *n_above = sm.info[1];
  *n_eq = sm.info[2];
}

// The region of values holding the r-th largest active value: (v & pmask) ==
// prefix, with r of its n_eq values wanted.  `whole`: all of them (r ==
// n_eq); `single`: the region is one exact value.  Neither: more bits remain.
struct TkRegion {
  uint32_t prefix, pmask, r, n_eq;
  bool whole, single;
  __device__ uint32_t top() const { return prefix | ~pmask; }  // largest value of the region
};

// Radix select of the r-th largest of the active values (r <= their count),
// starting below the bits they all share; at most max_passes passes.
template <int E>
__device__ TkRegion radix_select(const uint32_t (&v)[E], lanemask act, uint32_t r, uint32_t vmax,
                                 uint32_t vmin, uint32_t count, int max_passes, TkSmem& sm, int& par) {
  TkRegion g;
  const uint32_t diff = vmax ^ vmin;
  if (diff == 0) {  // every active value is the same
    g.prefix = vmax;
    g.pmask = 0xFFFFFFFFu;
    g.r = r;
    g.n_eq = count;
    g.whole = r == count;
    g.single = true;
    return g;
  }
  int top = 31 - __clz(diff);
  g.pmask = top == 31 ? 0u : ~((2u << top) - 1u);
  g.prefix = vmax & g.pmask;
  g.r = r;
  for (int pass = 0;; ++pass) {
    const int width = min(TK_BITS, top + 1);
    const int lo = top - width + 1;
    uint32_t d, n_above, n_eq;
    radix_pass<E>(v, act, g.prefix, g.pmask, lo, width, g.r, sm, par, &d, &n_above, &n_eq);
    g.prefix |= d << lo;
    g.pmask |= (uint32_t)((1u << width) - 1u) << lo;
    g.r -= n_above;
    g.n_eq = n_eq;
    g.whole = n_eq == g.r;
    g.single = lo == 0;
    if (g.whole || g.single || pass + 1 >= max_passes) return g;
    top = lo - 1;
  }
}

// Block-wide count, max and min of the active values.
template <int E>
__device__ __forceinline__ void active_stats(const uint32_t (&v)[E], lanemask act, TkSmem& sm, int& par,
                                             uint32_t* count, uint32_t* vmax, uint32_t* vmin) {
  uint32_t n = (uint32_t)__popcll(act), hi = 0, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool a = (act >> e) & 1u;
    hi = max(hi, a ? v[e] : 0u);
    lo = min(lo, a ? v[e] : 0xFFFFFFFFu);
  }
  block_sum_max_min(n, hi, lo, sm, par);
  *count = n;
  *vmax = hi;
  *vmin = lo;
}

template <int E>
__device__ __forceinline__ void region_masks(const uint32_t (&v)[E], lanemask act, const TkRegion& g,
                                             lanemask* above, lanemask* in) {
  lanemask a = 0, i = 0;
  const uint32_t top = g.top();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool on = (act >> e) & 1u;
    a |= (lanemask)(on && v[e] > top) << e;
    i |= (lanemask)(on && (v[e] & g.pmask) == g.prefix) << e;
  }
  *above = a;
  *in = i;
}

// The first r of the `take` elements in position order (one block scan).
template <int E>
__device__ __forceinline__ lanemask first_in_order(lanemask take, uint32_t r, TkSmem& sm, int& par) {
  uint32_t total;
  lanemask sel = 0;
  uint32_t k = block_excl_scan((uint32_t)__popcll(take), &total, sm, par);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((take >> e) & 1u) {
      if (k < r) sel |= (lanemask)1 << e;
      ++k;
    }
  }
  return sel;
}

// Given a region that is one exact score with r of its copies wanted (`in`):
// the r lowest ids, identical (score, id) pairs taken in position order.
// `nid_in_order`: nid = ~id falls with the position (ids are the columns).
template <int E>
__device__ lanemask cut_tie(const uint32_t (&nid)[E], lanemask in, uint32_t r, bool nid_in_order,
                            TkSmem& sm, int& par) {
  lanemask sel = 0, take = in;
  if (!nid_in_order) {
    uint32_t cnt, vmax, vmin;
    active_stats<E>(nid, in, sm, par, &cnt, &vmax, &vmin);
    const TkRegion h = radix_select<E>(nid, in, r, vmax, vmin, cnt, 99, sm, par);
    lanemask h_above, h_in;
    region_masks<E>(nid, in, h, &h_above, &h_in);
    sel = h_above;
    if (h.whole) return sel | h_in;
    take = h_in;  // repeated (score, id) pairs
    r = h.r;
  }
  return sel | first_in_order<E>(take, r, sm, par);
}

// Mask of the r active elements with the largest (hi, nid) pairs.
template <int E>
__device__ lanemask select_top(const uint32_t (&hi)[E], const uint32_t (&nid)[E], lanemask act, uint32_t r,
                               bool nid_in_order, TkSmem& sm, int& par) {
  uint32_t cnt, vmax, vmin;
  active_stats<E>(hi, act, sm, par, &cnt, &vmax, &vmin);
  const TkRegion g = radix_select<E>(hi, act, r, vmax, vmin, cnt, 99, sm, par);
  lanemask sel, in;
  region_masks<E>(hi, act, g, &sel, &in);
  if (g.whole) return sel | in;
  return sel | cut_tie<E>(nid, in, g.r, nid_in_order, sm, par);
}

// Writes the selected elements' keys to dst[base + ...] in position order;
// returns how many there are.
template <int E>
__device__ __forceinline__ uint32_t compact(const uint32_t (&hi)[E], const uint32_t (&nid)[E], lanemask sel,
                                            uint64_t* dst, uint32_t base, TkSmem& sm, int& par) {
  uint32_t total;
  uint32_t pos = base + block_excl_scan((uint32_t)__popcll(sel), &total, sm, par);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((sel >> e) & 1u) {
      if (pos < (uint32_t)TK_KMAX) dst[pos] = ((uint64_t)hi[e] << 32) | (uint64_t)nid[e];
      ++pos;
    }
  }
  return total;
}

// Where a workgroup's selected keys go: the final (idx, score) row, sorted, or
// a row of chunk-winner keys in any order.
struct TkDst {
  int32_t* idx;
  float* score;
  uint64_t* keys;
};

constexpr uint32_t TK_WRITTEN = 0xFFFFFFFFu;  // block_select wrote the output row itself
constexpr uint32_t TK_SEG_MAX = 32;           // longest score bucket ranked by a plain scan
constexpr uint32_t TK_WAVE_SORT = WAVE;       // boundary buckets this small are ordered by one wave,
constexpr uint32_t TK_RANK_SORT = 24;         // by counting ranks up to this size, else a sort

__device__ __forceinline__ void put_final(const TkDst& dst, uint32_t j, uint64_t key) {
  dst.idx[j] = (int32_t)(~(uint32_t)key);
  if (dst.score) dst.score[j] = key_score((uint32_t)(key >> 32));
}

// Selection by linear score buckets, for a chunk whose scores (of the valid
// elements: v[e] for valid bit e, NaN elsewhere) have a finite, nonzero range
// [lo, lo + span].  Bucket max((s - lo) * 2048 / span, 0), clamped, is a
// monotone function of the score (a NaN score, ranked lowest, lands in bucket
// 0), so the buckets above the one holding the K-th largest key are wholly
// selected and the rest of the selection happens in that one bucket.  Unlike
// the radix digits of a float key, the buckets spread scores evenly over
// their range, so a bucket holds a few keys and:
//  - the histogram's suffix sums place every key of a selected bucket in
//    the output order, bucket by bucket; within a bucket one short scan of
//    its keys ranks it;
//  - the boundary bucket, when it holds at most 64 keys, is ordered by one
//    wave and its first r keys complete the output.
// Returns TK_WRITTEN when the output row is written, else the number of keys
// left in sm.buf for the caller to sort (final) or write (chunk winners).
// Score bucket: monotone in s, NaN -> 0.  The one definition used for every
// evaluation, so that an entry always lands in the same bucket.
__device__ __forceinline__ uint32_t score_bucket(float s, float lo, float scale) {
  const float t = fmaxf((s - lo) * scale, 0.f);
  return min((uint32_t)t, (uint32_t)(TK_BINS - 1));
}

template <bool FINAL>
__device__ uint32_t bucket_select(const float (&v)[TK_E], const uint32_t (&idv)[TK_E], lanemask valid,
                                  float lo, float span, int K, const TkDst& dst, TkSmem& sm, int& par) {
  const int tid = threadIdx.x;
  const float scale = (float)TK_BINS / span;
  // empty elements count into the lane's own dummy bin (no collisions);
  // threads with none skip the test, threads with no valid element skip all
  uint32_t bk[TK_E];
#pragma unroll
  for (int e = 0; e < TK_E; ++e) bk[e] = score_bucket(v[e], lo, scale);
  constexpr lanemask all = (lanemask(1) << TK_E) - 1u;
  if (valid == all) {
#pragma unroll
    for (int e = 0; e < TK_E; ++e) atomicAdd(&sm.lcnt[bk[e]], 1u);
  } else if (valid) {
#pragma unroll
    for (int e = 0; e < TK_E; ++e)
      atomicAdd(&sm.lcnt[((valid >> e) & 1u) ? bk[e] : (uint32_t)(TK_BINS + lane_id())], 1u);
  }
  __syncthreads();
  // thread t owns buckets 2t and 2t + 1; keys in higher buckets come first
  static_assert(TK_BINS == 2 * TK_T, "two buckets per thread");
  const uint32_t h0 = sm.lcnt[2 * tid], h1 = sm.lcnt[2 * tid + 1];
  uint32_t total;
  const uint32_t excl = block_excl_scan(h0 + h1, &total, sm, par);
  const uint32_t above1 = total - excl - h0 - h1, above0 = above1 + h1;
  sm.lcur[2 * tid + 1] = above1;
  sm.lcur[2 * tid] = above0;
  if (above1 < (uint32_t)K && above0 >= (uint32_t)K) {
    sm.info[0] = 2 * tid + 1;
    sm.info[1] = above1;
    sm.info[2] = h1;
  } else if (above0 < (uint32_t)K && above0 + h0 >= (uint32_t)K) {
    sm.info[0] = 2 * tid;
    sm.info[1] = above0;
    sm.info[2] = h0;
  }
  __syncthreads();
  const uint32_t d = sm.info[0], n_above = sm.info[1], n_eq = sm.info[2];
  const uint32_t r = (uint32_t)K - n_above;  // wanted from bucket d, 1 <= r <= n_eq
  // a selected bucket too long for the plain in-bucket ranking
  if ((2 * tid > d && h0 > TK_SEG_MAX) || (2 * tid + 1 > d && h1 > TK_SEG_MAX)) sm.info[3] = 1;
  // ---- the entries of buckets above d, and of bucket d when it fits, are
  // compacted wave by wave into sm.stage as (score bits, id)
  const bool d_fits = n_eq <= (uint32_t)TK_KMAX;
  const uint32_t dd = d_fits ? d : 0xFFFFu;  // no bucket matches 0xFFFF
  auto stage = [&](auto check_valid) {
    // in bucket 0 (d == 0) only the valid elements count
    auto st = [&](int e) {
      if constexpr (decltype(check_valid)::value) return bk[e] > 0u || (d_fits && ((valid >> e) & 1u));
      else return bk[e] > d || bk[e] == dd;
    };
    uint32_t wn = 0;
#pragma unroll
    for (int e = 0; e < TK_E; ++e) wn += (uint32_t)__popcll(__ballot(st(e)));
    uint32_t wbase = 0;
    if (lane_id() == 0 && wn) wbase = atomicAdd(&sm.info[4], wn);
    wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase);
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      const uint64_t m = __ballot(st(e));
      if (m) {
        const uint32_t below =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (st(e)) sm.stage[wbase + below] = ((uint64_t)__float_as_uint(v[e]) << 32) | (uint64_t)idv[e];
        wbase += (uint32_t)__popcll(m);
      }
    }
  };
  if (d != 0) stage(std::false_type());
  else stage(std::true_type());
  __syncthreads();
  // ---- staged entries to sm.buf bucket by bucket (buckets above d) or to
  // sm.xbuf (bucket d), as 64-bit keys
  const uint32_t n_stage = n_above + (d_fits ? n_eq : 0u);
  for (uint32_t i = (uint32_t)tid; i < n_stage; i += TK_T) {
    const uint64_t sv = sm.stage[i];
    const float s = __uint_as_float((uint32_t)(sv >> 32));
    const uint32_t bk = score_bucket(s, lo, scale);
    const uint64_t key = ((uint64_t)score_key(s) << 32) | (uint64_t)(~(uint32_t)sv);
    const uint32_t p = atomicAdd(&sm.lcur[bk], 1u);
    if (bk != d) {
      sm.buf[p] = key;
      sm.lbk[p] = (uint16_t)bk;
      if (!FINAL) dst.keys[p] = key;
    } else {
      sm.xbuf[p - n_above] = key;
    }
  }
  __syncthreads();
  const bool long_seg = sm.info[3] != 0;
  if (n_eq <= TK_WAVE_SORT) {
    // one wave orders bucket d and completes the output with its first r keys
    if (wave_id() == 0) {
      uint64_t kv[1] = {(uint32_t)tid < n_eq ? sm.xbuf[tid] : 0ull};
      uint32_t slot = (uint32_t)tid;
      if (n_eq <= TK_RANK_SORT) {
        // rank among the n_eq keys, equal keys by lane
        uint32_t rank = 0;
        for (uint32_t j = 0; j < n_eq; ++j) {
          const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kv[0] >> 32), (int)j) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kv[0], (int)j);
          rank += (o > kv[0] || (o == kv[0] && j < (uint32_t)tid)) ? 1u : 0u;
        }
        slot = (uint32_t)tid < n_eq ? rank : 0xFFFFFFFFu;
      } else {
        int pb = 0;
        sort_sizes<2, WAVE>(kv, sm, pb);
      }
      if (slot < r) {
        if (!FINAL) dst.keys[n_above + slot] = kv[0];
        else if (long_seg) sm.buf[n_above + slot] = kv[0];
        else put_final(dst, n_above + slot, kv[0]);
      }
    }
    if (!FINAL) return TK_WRITTEN;
    if (long_seg) return (uint32_t)K;  // the caller sorts sm.buf (its barrier orders the writes)
    // every key of sm.buf: its bucket's place in the output plus its rank
    // among the keys of the bucket (equal keys by their place in sm.buf)
    for (uint32_t p = (uint32_t)tid; p < n_above; p += TK_T) {
      const uint64_t key = sm.buf[p];
      const uint32_t bk = sm.lbk[p];
      const uint32_t end = sm.lcur[bk], beg = end - sm.lcnt[bk];
      uint32_t rank = 0;
      for (uint32_t j = beg; j < end; ++j) {
        const uint64_t o = sm.buf[j];
        rank += (o > key || (o == key && j < p)) ? 1u : 0u;
      }
      put_final(dst, beg + rank, key);
    }
    return TK_WRITTEN;
  }
  return TK_KMAX + 1;  // bucket d is large: the caller selects in it
}

// Top K of the candidates held by the block, thread t owning positions
// 16t .. 16t + 15 in column order: element e has score v[e] and id idv[e]
// when valid bit e is set (v[e] is NaN otherwise).  Writes the selected keys
// to sm.buf[0 .. count), count = min(K, #valid), or the output row itself
// (returns TK_WRITTEN).
template <bool FINAL>
__device__ __forceinline__ uint32_t block_select(const float (&v)[TK_E], const uint32_t (&idv)[TK_E], lanemask valid,
                                 bool ids_are_columns, int K, const TkDst& dst, TkSmem& sm) {
  int par = 0;
  // count, highest and lowest score of the valid elements (NaN scores and
  // the NaN placeholders of empty elements are skipped by max / min)
  uint32_t n_all = (uint32_t)__popcll(valid), fhi = F_NAN, flo = F_NAN;
  {
    float h = __uint_as_float(F_NAN), l = __uint_as_float(F_NAN);
#pragma unroll
    for (int e = 0; e < TK_E; ++e) {
      h = fmaxf(h, v[e]);
      l = fminf(l, v[e]);
    }
    fhi = __float_as_uint(h);
    flo = __float_as_uint(l);
  }
  block_reduce3<OpAdd, OpFMax, OpFMin>(n_all, fhi, flo, 0u, F_NAN, F_NAN, sm, par);
  const float hi = __uint_as_float(fhi), lo = __uint_as_float(flo);
  const float span = hi - lo;  // NaN or infinite unless both ends are finite
  const bool linear = n_all > (uint32_t)K && span >= 1e-30f && span <= 3.4e38f;
  if (linear) {
    const uint32_t res = bucket_select<FINAL>(v, idv, valid, lo, span, K, dst, sm, par);
    if (res <= (uint32_t)TK_KMAX || res == TK_WRITTEN) return res;
    // bucket d holds more than 64 keys: select in it below
    const uint32_t d = sm.info[0], n_above = sm.info[1], n_eq = sm.info[2];
    const uint32_t r = (uint32_t)K - n_above;
    if (n_eq <= (uint32_t)TK_KMAX) {
      // its keys are in sm.xbuf[0 .. n_eq) in no particular order
      uint32_t chi[TK_CE], cnid[TK_CE];
      lanemask cact = 0;
#pragma unroll
      for (int e = 0; e < TK_CE; ++e) {
        const uint32_t j = (uint32_t)(TK_CE * threadIdx.x + e);
        const uint64_t key = j < n_eq ? sm.xbuf[j] : 0ull;
        chi[e] = (uint32_t)(key >> 32);
        cnid[e] = (uint32_t)key;
        cact |= (lanemask)(j < n_eq) << e;
      }
      const lanemask csel = select_top<TK_CE>(chi, cnid, cact, r, false, sm, par);
      (void)compact<TK_CE>(chi, cnid, csel, sm.buf, n_above, sm, par);
      __syncthreads();
      return (uint32_t)K;
    }
    // more than 2048 keys in one bucket: the radix path below, from the start
    (void)d;
    __syncthreads();
  }
  // ---- radix selection on the 32-bit score keys (0 = empty)
  uint32_t sk[TK_E], nid[TK_E];
#pragma unroll
  for (int e = 0; e < TK_E; ++e) {
    sk[e] = ((valid >> e) & 1u) ? score_key(v[e]) : 0u;
    nid[e] = ~idv[e];
  }
  uint32_t count;
  if (n_all <= (uint32_t)K) {
    count = compact<TK_E>(sk, nid, valid, sm.buf, 0, sm, par);
  } else {
    // one radix pass over the whole chunk
    uint32_t n_chk, smax, smin;
    active_stats<TK_E>(sk, valid, sm, par, &n_chk, &smax, &smin);
    const TkRegion g = radix_select<TK_E>(sk, valid, (uint32_t)K, smax, smin, n_all, 1, sm, par);
    lanemask above, in;
    region_masks<TK_E>(sk, valid, g, &above, &in);
    if (g.whole || g.single || g.n_eq > (uint32_t)TK_KMAX) {
      lanemask sel = above;
      if (g.whole) sel |= in;
      else if (g.single) sel |= cut_tie<TK_E>(nid, in, g.r, ids_are_columns, sm, par);
      else sel |= select_top<TK_E>(sk, nid, in, g.r, ids_are_columns, sm, par);  // a huge bin
      count = compact<TK_E>(sk, nid, sel, sm.buf, 0, sm, par);
    } else {
      // the keys above the boundary bin go straight to the output buffer, the
      // n_eq <= 2048 keys of the bin to the candidate buffer (both in column
      // order, one scan of packed counts); the rest of the selection runs on
      // the candidates, TK_CE per thread
      uint32_t total;
      const uint32_t x =
          block_excl_scan(((uint32_t)__popcll(above) << 16) | (uint32_t)__popcll(in), &total, sm, par);
      uint32_t pa = x >> 16, pi = x & 0xFFFFu;
#pragma unroll
      for (int e = 0; e < TK_E; ++e) {
        const uint64_t key = ((uint64_t)sk[e] << 32) | (uint64_t)nid[e];
        if ((above >> e) & 1u) sm.buf[pa++] = key;
        if ((in >> e) & 1u) sm.xbuf[pi++] = key;
      }
      const uint32_t n_above = (uint32_t)K - g.r;
      __syncthreads();
      uint32_t chi[TK_CE], cnid[TK_CE];
      lanemask cact = 0;
#pragma unroll
      for (int e = 0; e < TK_CE; ++e) {
        const uint32_t j = (uint32_t)(TK_CE * threadIdx.x + e);
        const uint64_t key = j < g.n_eq ? sm.xbuf[j] : 0ull;
        chi[e] = (uint32_t)(key >> 32);
        cnid[e] = (uint32_t)key;
        cact |= (lanemask)(j < g.n_eq) << e;
      }
      const lanemask csel = select_top<TK_CE>(chi, cnid, cact, g.r, ids_are_columns, sm, par);
      (void)compact<TK_CE>(chi, cnid, csel, sm.buf, n_above, sm, par);
      count = (uint32_t)K;
    }
  }
  __syncthreads();
  return min(count, (uint32_t)TK_KMAX);
}

}  // namespace csa2
