// a0: one work item of the FP4 append, shared by the append kernel and the
// Top-K final level that runs an append beside its selection (the same code,
// so both write the same bytes).
//
// Format ([P1] section 效率组件四件, item 4; [P4] CSA2 paragraph): E2M1 codes
// with one E4M3 scale per 16 channels and no global scale.  Work item gid <
// n_groups owns one 16-channel group: it reads 32 contiguous bytes of bf16
// (a row of 32 groups is 1 KiB read by 32 consecutive items), finds the block
// scale with exact threshold compares (no division), encodes the 16 elements
// with seven exact threshold compares each, and writes 8 code bytes + 1 scale
// byte.  Items n_groups .. n_groups + n_rope - 1 copy 8 RoPE channels each.
#pragma once

#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

__device__ __forceinline__ void fp4_append_item(int64_t gid, const Fp4Append& a, int64_t n_groups,
                                                int64_t n_rope) {
  if (gid < n_groups) {
    const int gpr = a.d_c >> 4;                     // groups per row
    const int64_t r = gid / gpr;
    const int g = (int)(gid - r * gpr);
    const u32x4* src = reinterpret_cast<const u32x4*>(a.x + r * a.d_c + g * 16);
    const u32x4 lo = __builtin_nontemporal_load(src);
    const u32x4 hi = __builtin_nontemporal_load(src + 1);
    uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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
    const int64_t row = a.dst_row0 + r;
    *reinterpret_cast<uint64_t*>(a.cache.codes + row * a.cache.codes_stride + g * 8) = packed;
    a.cache.scales[row * a.cache.scales_stride + g] = (uint8_t)S;
  } else if (gid < n_groups + n_rope) {
    // RoPE part: copied unchanged, 8 bf16 (16 bytes) per item
    const int64_t c = gid - n_groups;
    const int cpr = a.d_r >> 3;
    const int64_t r = c / cpr;
    const int j = (int)(c - r * cpr);
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.rope_src + r * a.d_r + j * 8);
    uint8_t* dst = reinterpret_cast<uint8_t*>(a.cache.rope) + (a.dst_row0 + r) * a.cache.rope_stride + j * 16;
    *reinterpret_cast<u32x4*>(dst) = v;
  }
}

}  // namespace csa2
