// a0: FP4 quantise + append of post-RoPE latent rows into the main KV cache.
//
// Format ([P1] section 效率组件四件, item 4; [P4] CSA2 paragraph): E2M1 codes
// with one E4M3 scale per 16 channels and no global scale.  One thread owns
// one 16-channel group: it reads 32 contiguous bytes of bf16 (a row of 32
// groups is 1 KiB read by 32 consecutive lanes), finds the block scale with
// exact threshold compares (no division), encodes the 16 elements with seven
// exact threshold compares each, and writes 8 code bytes + 1 scale byte.
// HBM-bound: 2 bytes in, 0.5625 bytes out per channel.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

__global__ __launch_bounds__(256) void quantize_fp4_kernel(
    const uint16_t* __restrict__ x, int64_t n_rows, int d_c, const uint16_t* __restrict__ rope_src,
    int d_r, CacheRef cache, int64_t dst_row0, int64_t n_groups, int64_t n_rope_chunks) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < n_groups) {
    const int gpr = d_c >> 4;                       // groups per row
    const int64_t r = gid / gpr;
    const int g = (int)(gid - r * gpr);
    const u32x4* src = reinterpret_cast<const u32x4*>(x + r * d_c + g * 16);
    const u32x4 a = __builtin_nontemporal_load(src);
    const u32x4 b = __builtin_nontemporal_load(src + 1);
    uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    // amax over magnitudes: non-negative floats order like their bit patterns
    uint32_t mbits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mbits = max(mbits, w[i] & 0x7FFFu);
      mbits = max(mbits, (w[i] >> 16) & 0x7FFFu);
    }
    const uint32_t S = e4m3_scale_code_fast(bf16_bits_to_f32(mbits));
    const float sigma = e4m3_value(S);
    uint64_t packed = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
      const float ax = bf16_bits_to_f32(h & 0x7FFFu);
      uint32_t mag = e2m1_mag_code(ax, sigma);
      mag = (S == 0) ? 0u : mag;
      const uint32_t code = ((h >> 12) & 8u) | mag;
      packed |= (uint64_t)code << (4 * i);
    }
    const int64_t row = dst_row0 + r;
    *reinterpret_cast<uint64_t*>(cache.codes + row * cache.codes_stride + g * 8) = packed;
    cache.scales[row * cache.scales_stride + g] = (uint8_t)S;
  } else if (gid < n_groups + n_rope_chunks) {
    // RoPE part: copied unchanged, 8 bf16 (16 bytes) per thread
    const int64_t c = gid - n_groups;
    const int cpr = d_r >> 3;
    const int64_t r = c / cpr;
    const int j = (int)(c - r * cpr);
    const u32x4 v = *reinterpret_cast<const u32x4*>(rope_src + r * d_r + j * 8);
    uint8_t* dst = reinterpret_cast<uint8_t*>(cache.rope) + (dst_row0 + r) * cache.rope_stride + j * 16;
    *reinterpret_cast<u32x4*>(dst) = v;
  }
}

// One thread per 16-channel group and per 8 RoPE channels, 256 per workgroup.
int64_t quantize_fp4_launch_items(int64_t n_rows, int d_c, int d_r) {
  const int64_t total = n_rows * (d_c / 16) + (d_r > 0 ? n_rows * (d_r / 8) : 0);
  return (total + 255) / 256 * 256;
}

hipError_t launch_quantize_fp4(const uint16_t* x, int64_t n_rows, int d_c, const uint16_t* rope_src,
                               int d_r, CacheRef cache, int64_t dst_row0, hipStream_t stream) {
  const int64_t n_groups = n_rows * (d_c / 16);
  const int64_t n_rope = d_r > 0 ? n_rows * (d_r / 8) : 0;
  const int64_t total = n_groups + n_rope;
  if (total == 0) return hipSuccess;
  const int64_t blocks = quantize_fp4_launch_items(n_rows, d_c, d_r) / 256;
  hipLaunchKernelGGL(quantize_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_rows,
                     d_c, rope_src, d_r, cache, dst_row0, n_groups, n_rope);
  return hipGetLastError();
}


// FP8 write of the sliding-window KV (the window branch keeps its KV in FP8:
// [P4] CSA2 paragraph; [P1] section 效率组件四件, item 4).  One power-of-two
// scale per row: 2^e with e the smallest integer such that max|x| <= 448 * 2^e
// (e = 0 for an all-zero row, clamped to [-126, 127]), so x / 2^e is exact and
// nothing saturates; each element is the E4M3 value nearest to |x| / 2^e, ties
// to the even code, with the input's sign bit.  One wave per row: each lane
// holds 8 channels per 512-channel chunk (one 16-byte load), the row maximum
// is a wave reduction, and 8 code bytes go out per lane and chunk.
namespace {

// E4M3 code (0..126) nearest to y in [0, 448], ties to the even code: the
// number of codes c with y above the midpoint (v(c) + v(c + 1)) / 2, or on it
// with c odd; the midpoints are exact in fp32 and increasing, so a 7-step
// binary search finds the count.
__device__ __forceinline__ uint32_t e4m3_rne_code(float y) {
  uint32_t lo = 0, hi = 126;
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    if (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      const float M = 0.5f * (e4m3_value(mid) + e4m3_value(mid + 1));
      const bool pass = (y > M) || (y == M && (mid & 1u));
      lo = pass ? mid + 1 : lo;
      hi = pass ? hi : mid;
    }
  }
  return lo;
}

}  // namespace

__global__ __launch_bounds__(256) void quantize_fp8_kernel(
    const uint16_t* __restrict__ x, int64_t n_rows, int d_c, const uint16_t* __restrict__ rope_src, int d_r,
    uint8_t* __restrict__ codes, int64_t codes_stride, float* __restrict__ sigma, uint16_t* __restrict__ rope_dst,
    int64_t rope_stride, int64_t dst_row0) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const uint16_t* src = x + r * d_c;
  uint32_t mbits = 0;  // largest magnitude: non-negative floats order like their bit patterns
  for (int c0 = 8 * lane; c0 < d_c; c0 += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + c0);
#pragma unroll
    for (int j = 0; j < 4; ++j) mbits = max(mbits, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, o));
  // amax = m * 2^E, m in [1, 2): 448 * 2^e = 1.75 * 2^(e + 8) covers it from
  // e = E - 8 when m <= 1.75, else from e = E - 7 (bf16 subnormals: E = -133..)
  int e = 0;
  if (mbits != 0) {
    const float amax = bf16_bits_to_f32(mbits);
    int E;
    const float m = 2.0f * frexpf(amax, &E);  // amax = m * 2^(E - 1), m in [1, 2)
    e = (E - 1) - 8 + (m > 1.75f ? 1 : 0);
    e = min(max(e, -126), 127);
  }
  const float inv = __builtin_amdgcn_ldexpf(1.0f, -e);  // exact power of two
  uint8_t* dst = codes + (dst_row0 + r) * codes_stride;
  for (int c0 = 8 * lane; c0 < d_c; c0 += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + c0);
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t h = (k & 1) ? (v[k >> 1] >> 16) : (v[k >> 1] & 0xFFFFu);
      const float y = bf16_bits_to_f32(h & 0x7FFFu) * inv;
      const uint32_t code = e4m3_rne_code(y) | ((h >> 8) & 0x80u);
      out[k >> 2] |= code << (8 * (k & 3));
    }
    *reinterpret_cast<u32x2*>(dst + c0) = u32x2{out[0], out[1]};
  }
  if (lane == 0) sigma[dst_row0 + r] = __builtin_amdgcn_ldexpf(1.0f, e);
  if (d_r > 0) {
    uint8_t* rd = reinterpret_cast<uint8_t*>(rope_dst) + (dst_row0 + r) * rope_stride;
    for (int c0 = 8 * lane; c0 < d_r; c0 += 512)
      *reinterpret_cast<u32x4*>(rd + 2 * c0) = *reinterpret_cast<const u32x4*>(rope_src + r * d_r + c0);
  }
}

// One wave per row, four rows per workgroup.
int64_t quantize_fp8_launch_items(int64_t n_rows) { return (n_rows + 3) / 4 * 256; }

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t n_rows, int d_c, const uint16_t* rope_src, int d_r,
                               uint8_t* codes, int64_t codes_stride, float* sigma, uint16_t* rope_dst,
                               int64_t rope_stride, int64_t dst_row0, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, stream, x, n_rows, d_c,
                     rope_src, d_r, codes, codes_stride, sigma, rope_dst, rope_stride, dst_row0);
  return hipGetLastError();
}

}  // namespace csa2
