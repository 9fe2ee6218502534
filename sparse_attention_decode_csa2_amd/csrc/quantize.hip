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
    const uint32_t S = e4m3_scale_code(bf16_bits_to_f32(mbits));
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

hipError_t launch_quantize_fp4(const uint16_t* x, int64_t n_rows, int d_c, const uint16_t* rope_src,
                               int d_r, CacheRef cache, int64_t dst_row0, hipStream_t stream) {
  const int64_t n_groups = n_rows * (d_c / 16);
  const int64_t n_rope = d_r > 0 ? n_rows * (d_r / 8) : 0;
  const int64_t total = n_groups + n_rope;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(quantize_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_rows,
                     d_c, rope_src, d_r, cache, dst_row0, n_groups, n_rope);
  return hipGetLastError();
}

}  // namespace csa2
