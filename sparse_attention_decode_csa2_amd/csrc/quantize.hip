// a0: FP4 quantise + append of post-RoPE latent rows into the main KV cache
// (the work item is fp4_append_item, quantize_task.h).  HBM-bound: 2 bytes in,
// 0.5625 bytes out per channel.
#include "csa2_device.h"
#include "csa2_internal.h"
#include "quantize_task.h"

namespace csa2 {

__global__ __launch_bounds__(256) void quantize_fp4_kernel(const Fp4Append a, int64_t n_groups, int64_t n_rope) {
  fp4_append_item((int64_t)blockIdx.x * blockDim.x + threadIdx.x, a, n_groups, n_rope);
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
  const Fp4Append a{x, n_rows, d_c, rope_src, d_r, cache, dst_row0};
  hipLaunchKernelGGL(quantize_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n_groups, n_rope);
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
