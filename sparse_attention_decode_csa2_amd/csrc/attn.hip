// a4 + a5: gather of the selected FP4 entries, exact dequantisation and
// softmax attention of the query heads over them (MLA-style: key = [latent ;
// RoPE part], value = latent, one entry shared by every head)
// ([P1] 架构三件套 - CSA2; [P3] modes paragraph; [P4] CSA2 paragraph).
//
// One workgroup (4 waves) owns one query, 16 heads and a slice of the index
// list, walked in tiles of 64 entries:
//  1. gather: each thread fetches a quarter of one entry (codes, scales, RoPE
//     part) with 16-byte loads and dequantises it into an LDS tile (latent as
//     fp16, RoPE as bf16).  E2M1 x E4M3 products have <= 6 significant bits
//     and lie in [2^-10, 2688], so the fp16 latent is exact.
//  2. scores: wave w forms S^T for entries [16w, 16w + 16) of the tile with
//     v_mfma_f32_16x16x32 (A = the entry rows from LDS, B = the 16 query
//     heads held in registers), fp16 for the latent part, bf16 for RoPE.
//     The query latent is multiplied by a power of two per head so that it
//     converts to fp16 without rounding; the factor is undone in the softmax
//     scale.
//  3. online softmax in fp32 (base 2), row max / sum exchanged through LDS.
//  4. P (fp16) . V with v_mfma_f32_16x16x32_f16, wave w owning a quarter of
//     the latent channels; V comes from the same LDS tile.
// With several slices per query the unnormalised partial results (O, max,
// sum) go to the workspace and a combine kernel merges them by log-sum-exp.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int AT_TILE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// E2M1 nibble -> fp32 value (sign included), exact.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t k = c & 7u;
  float v = k >= 2 ? __uint_as_float((k << 22) + 0x3F000000u) : 0.5f * (float)k;
  return __uint_as_float(__float_as_uint(v) | ((c & 8u) << 28));
}

template <int DC, int DR>
__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint16_t* __restrict__ rope,
    const int32_t* __restrict__ idx, int K, int H, int64_t N_cap, float sm_scale_log2e, int n_hg,
    int n_split, int per_split, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int KSL = DC / 32;           // latent k-steps
  constexpr int KSR = DR / 32;           // RoPE k-steps
  constexpr int LDK = DC + 8;            // fp16 pitch of the latent tile
  constexpr int LDR = DR + 8;            // bf16 pitch of the RoPE tile
  constexpr int CB = DC / 2;             // code bytes per entry
  constexpr int GPE = DC / 16;           // scale bytes per entry
  constexpr int QCH = DC / 4;            // latent channels per gather thread / per PV wave
  constexpr int NDB = QCH / 16;          // PV d-blocks per wave
  __shared__ __attribute__((aligned(16))) _Float16 sK[AT_TILE][LDK];
  __shared__ __attribute__((aligned(16))) __bf16 sR[AT_TILE][DR > 0 ? LDR : 8];
  __shared__ __attribute__((aligned(16))) _Float16 sP[16][AT_TILE + 8];
  __shared__ float sMax[4][16], sSum[4][16], sAlpha[16], sFinM[16], sFinL[16];
  __shared__ int sValid[AT_TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  int bid = blockIdx.x;
  const int split = bid % n_split;
  bid /= n_split;
  const int hg = bid % n_hg;
  const int64_t b = bid / n_hg;
  const int h0 = hg * 16;

  // ---- query heads h0 + n as MFMA B operands (k-step t, k-group g -> dims 32t + 8g .. +7)
  f16x8 Bq[KSL];
  bf16x8 Br[KSR > 0 ? KSR : 1];
  float fscale;  // multiplies the MFMA result into base-2 softmax logits for head h0 + n
  {
    const int h = h0 + n;
    const bool hv = h < H;
    const uint16_t* qrow = q + (b * H + (hv ? h : 0)) * (DC + DR);
    u32x4 raw[KSL + KSR];
    uint32_t mx = 0;
#pragma unroll
    for (int t = 0; t < KSL + KSR; ++t) {
      const int off = t < KSL ? 32 * t + 8 * g : DC + 32 * (t - KSL) + 8 * g;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hv) v = *reinterpret_cast<const u32x4*>(qrow + off);
      raw[t] = v;
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
    // 2^sh brings the largest |q| of the head into [2^14, 2^15): fp16 keeps all
    // of a bf16 value's bits there; bf16 subnormals are treated as exponent -126
    int e = (int)((mx >> 7) & 0xFF) - 127;
    if (e < -126) e = -126;
    int sh = mx == 0 ? 0 : min(120, max(-120, 14 - e));
    const float up = __builtin_amdgcn_ldexpf(1.0f, sh);
    fscale = sm_scale_log2e * __builtin_amdgcn_ldexpf(1.0f, -sh);
#pragma unroll
    for (int t = 0; t < KSL; ++t) {
      f16x8 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = (_Float16)(bf16_bits_to_f32(raw[t][j] & 0xFFFFu) * up);
        v[2 * j + 1] = (_Float16)(bf16_bits_to_f32(raw[t][j] >> 16) * up);
      }
      Bq[t] = v;
    }
#pragma unroll
    for (int t = 0; t < KSR; ++t) {
      bf16x8 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = (__bf16)(bf16_bits_to_f32(raw[KSL + t][j] & 0xFFFFu) * up);
        v[2 * j + 1] = (__bf16)(bf16_bits_to_f32(raw[KSL + t][j] >> 16) * up);
      }
      Br[t] = v;
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // per head h0 + n (redundant in every wave)
  f32x4 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int e_begin = split * per_split;
  const int e_end = min(K, e_begin + per_split);
  const int32_t* idx_row = idx + b * K;
  const int er = tid >> 2, part = tid & 3;  // gather: entry row, quarter

  for (int tb = e_begin; tb < e_end; tb += AT_TILE) {
    // ---- 1. gather + dequantise one quarter of entry `er`
    {
      const int e = tb + er;
      const int32_t id = e < e_end ? idx_row[e] : -1;
      const bool valid = id >= 0 && (int64_t)id < N_cap;
      const int64_t row = b * N_cap + (valid ? id : 0);
      u32x4 cw[CB / 4 / 16 > 0 ? CB / 4 / 16 : 1];
      constexpr int NCW = CB / 4 / 16;  // 16-byte code words per quarter
      const uint8_t* cp = codes + row * CB + part * (CB / 4);
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(cp + 16 * i);
        cw[i] = v;
      }
      uint8_t sb[GPE / 4];
#pragma unroll
      for (int i = 0; i < GPE / 4; ++i) sb[i] = valid ? scales[row * GPE + part * (GPE / 4) + i] : 0;
      // channels part*QCH + 32i + 2j + {0,1} come from byte j of word i
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {       // 16 channels = one scale group
          const float sg = e4m3_decode(sb[2 * i + half]);
          f16x8 lo, hi;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t word = cw[i][2 * half + (j >> 2)];
            const uint32_t byte = (word >> (8 * (j & 3))) & 0xFFu;
            const _Float16 v0 = (_Float16)(e2m1_value(byte & 15u) * sg);
            const _Float16 v1 = (_Float16)(e2m1_value(byte >> 4) * sg);
            if (j < 4) { lo[2 * j] = v0; lo[2 * j + 1] = v1; }
            else { hi[2 * (j - 4)] = v0; hi[2 * (j - 4) + 1] = v1; }
          }
          _Float16* dst = &sK[er][part * QCH + 32 * i + 16 * half];
          *reinterpret_cast<f16x8*>(dst) = lo;
          *reinterpret_cast<f16x8*>(dst + 8) = hi;
        }
      }
      if (DR > 0) {
        constexpr int RW = DR / 4 / 8;  // 16-byte RoPE words per quarter
        const uint16_t* rp = rope + row * DR + part * (DR / 4);
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (valid) v = *reinterpret_cast<const u32x4*>(rp + 8 * i);
          *reinterpret_cast<u32x4*>(&sR[er][part * (DR / 4) + 8 * i]) = v;
        }
      }
      if (part == 0) sValid[er] = valid;
    }
    __syncthreads();

    // ---- 2. S^T for entries 16*wave + (0..15): lane (entry n, k-group g) supplies A
    float s2[4];
    {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * wave + n;
#pragma unroll
      for (int t = 0; t < KSL; ++t) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&sK[r][32 * t + 8 * g]);
        c = mfma16x16x32_f16(a, Bq[t], c);
      }
#pragma unroll
      for (int t = 0; t < KSR; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sR[r][32 * t + 8 * g]);
        c = mfma16x16x32_bf16(a, Br[t], c);
      }
      // c[i] = S^T[entry 16*wave + 4g + i][head n]
#pragma unroll
      for (int i = 0; i < 4; ++i) s2[i] = sValid[16 * wave + 4 * g + i] ? c[i] * fscale : -INFINITY;
    }
    // ---- 3. online softmax for head n (lanes n, n+16, n+32, n+48 hold its 16 entries)
    float mt = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (g == 0) sMax[wave][n] = mt;
    __syncthreads();
    const float m_tile = fmaxf(fmaxf(sMax[0][n], sMax[1][n]), fmaxf(sMax[2][n], sMax[3][n]));
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float p[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = s2[i] == -INFINITY ? 0.f : exp2f(s2[i] - m_new);
      ps += p[i];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    if (g == 0) sSum[wave][n] = ps;
    if (wave == 0 && g == 0) sAlpha[n] = alpha;
    {
      _Float16* prow = &sP[n][16 * wave + 4 * g];
#pragma unroll
      for (int i = 0; i < 4; ++i) prow[i] = (_Float16)p[i];
    }
    __syncthreads();
    l_run = l_run * alpha + (sSum[0][n] + sSum[1][n] + sSum[2][n] + sSum[3][n]);
    m_run = m_new;

    // ---- 4. O[heads][channels of this wave] = alpha * O + P . V
    {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = sAlpha[4 * g + i];
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[d][i] *= al[i];
#pragma unroll
      for (int u = 0; u < AT_TILE / 32; ++u) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&sP[n][32 * u + 8 * g]);
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const int col = wave * QCH + 16 * d + n;
          f16x8 bv;
#pragma unroll
          for (int i = 0; i < 8; ++i) bv[i] = sK[32 * u + 8 * g + i][col];
          acc[d] = mfma16x16x32_f16(a, bv, acc[d]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane (channel n of each d-block, k-group g) holds heads h0 + 4g + i
  if (wave == 0 && g == 0) {
    sFinM[n] = m_run;
    sFinL[n] = l_run;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * g + i;
    const int h = h0 + hl;
    if (h >= H) continue;
    const float m = sFinM[hl], l = sFinL[hl];
    if (n_split == 1) {
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float* orow = out + (b * H + h) * DC + wave * QCH;
#pragma unroll
      for (int d = 0; d < NDB; ++d) orow[16 * d + n] = acc[d][i] * inv;
      if (lse && wave == 0 && n == 0) lse[b * H + h] = l > 0.f ? (m + __log2f(l)) * LN2 : -INFINITY;
    } else {
      const int64_t slot = (b * H + h) * n_split + split;
      float* orow = ws_o + slot * DC + wave * QCH;
#pragma unroll
      for (int d = 0; d < NDB; ++d) orow[16 * d + n] = acc[d][i];
      if (wave == 0 && n == 0) {
        ws_ml[2 * slot] = m;
        ws_ml[2 * slot + 1] = l;
      }
    }
  }
}

// Merge the per-slice partial results of one (b, h) row by log-sum-exp.
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_ml,
                                                           int n_split, int DC, int64_t rows,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  const float* ml = ws_ml + row * n_split * 2;
  float m = -INFINITY;
  for (int s = 0; s < n_split; ++s) m = fmaxf(m, ml[2 * s]);
  float L = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ms = ml[2 * s];
    L += ms == -INFINITY ? 0.f : ml[2 * s + 1] * exp2f(ms - m);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  for (int c = threadIdx.x; c < DC; c += blockDim.x) {
    float o = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ms = ml[2 * s];
      if (ms != -INFINITY) o += ws_o[(row * n_split + s) * DC + c] * exp2f(ms - m);
    }
    out[row * DC + c] = o * inv;
  }
  if (lse && threadIdx.x == 0) lse[row] = L > 0.f ? (m + __log2f(L)) * LN2 : -INFINITY;
}

// Slices per query: enough workgroups for 256 CUs, whole 64-entry tiles.
static void attn_plan(int B, int H, int K, int* n_split, int* per_split) {
  const int n_hg = (H + 15) / 16;
  const int tiles = (K + AT_TILE - 1) / AT_TILE;
  const int base = B * n_hg;
  int s = base >= 512 ? 1 : (512 + base - 1) / max(base, 1);
  s = max(1, min(s, tiles));
  const int tps = (tiles + s - 1) / s;
  s = (tiles + tps - 1) / tps;
  *n_split = s;
  *per_split = tps * AT_TILE;
}

size_t attn_workspace_bytes(int B, int H, int d_c, int K) {
  int s, ps;
  attn_plan(B, H, K, &s, &ps);
  if (s <= 1) return 0;
  return (size_t)B * H * s * ((size_t)d_c + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                              const uint16_t* rope, const int32_t* idx, int K, int B, int H, int d_c,
                              int d_r, int64_t N_cap, float sm_scale, float* out, float* lse,
                              void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  int s, ps;
  attn_plan(B, H, K, &s, &ps);
  const int n_hg = (H + 15) / 16;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = s > 1 ? ws_o + (size_t)B * H * s * d_c : nullptr;
  const dim3 grid((unsigned)(B * n_hg * s)), blk(256);
  const float sl = sm_scale * LOG2E;
#define CSA2_ATTN(DCV, DRV)                                                                     \
  hipLaunchKernelGGL((sparse_attn_kernel<DCV, DRV>), grid, blk, 0, stream, q, codes, scales, rope, \
                     idx, K, H, N_cap, sl, n_hg, s, ps, out, lse, ws_o, ws_ml)
  if (d_c == 512 && d_r == 64) CSA2_ATTN(512, 64);
  else if (d_c == 512 && d_r == 0) CSA2_ATTN(512, 0);
  else if (d_c == 128 && d_r == 0) CSA2_ATTN(128, 0);
  else if (d_c == 128 && d_r == 64) CSA2_ATTN(128, 64);
  else return hipErrorInvalidValue;
#undef CSA2_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  const int64_t rows = (int64_t)B * H;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)rows), dim3(256), 0, stream, ws_o, ws_ml, s,
                     d_c, rows, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
