// a4 + a5: gather of the selected FP4 entries, exact dequantisation and
// softmax attention of the query heads over them (MLA-style: key = [latent ;
// RoPE part], value = latent, one entry shared by every head)
// ([P1] 架构三件套 - CSA2; [P3] modes paragraph; [P4] CSA2 paragraph).
//
// One workgroup (4 waves) owns one query, 16 heads and a slice of the index
// list, walked in tiles of 64 entries:
//  1. gather: wave w fetches entries [16w, 16w + 16) of the tile, lane
//     (n, g) = (l % 16, l / 16) a quarter of entry 16w + n: the 64 code
//     bytes [64i + 16g, +16) for i < 4 (channels 128i + 32g .. +31, so the
//     four lanes of an entry read 64 contiguous bytes per load), their two
//     E4M3 scale bytes, and 16 channels of the RoPE part.
//  2. the lane dequantises its quarter (exact: E2M1 x E4M3 products have
//     <= 6 significant bits within [2^-10, 2688]) straight into the MFMA A
//     operand of the scores: S^T for the wave's 16 entries and the 16 query
//     heads comes from v_mfma_f32_16x16x32 (fp16 latent, bf16 RoPE) with the
//     heads as the B operand held in registers, whose k order is permuted to
//     match (k-step 4i + j, lane group g <-> channels 128i + 32g + 8j .. +7).
//     The query latent is multiplied by a power of two per head so that it
//     converts to fp16 without rounding; the factor is undone in the softmax
//     scale.  The same fp16 values go to an LDS tile, the value operand of
//     P . V; its 16-byte pieces are permuted within each 32-channel chunk so
//     that these stores and the transposing reads below are free of bank
//     conflicts.
//  3. online softmax in fp32 (base 2), row max / sum exchanged through LDS.
//  4. P (fp16) . V with v_mfma_f32_16x16x32_f16, wave w owning a quarter of
//     the latent channels; V comes from the same LDS tile.
// With several slices per query the unnormalised partial results (O, max,
// sum) go to the workspace and a second kernel merges them by log-sum-exp
// (merging inside the last workgroup to finish would need device-scope
// fences, which write back and invalidate the whole XCD L2 under the other
// workgroups' gathers).
//
// Workgroups are numbered so that all head groups of one (query, slice) land
// on the same XCD (consecutive workgroup ids go round-robin over the eight
// XCDs): they gather the same entries, and only the first of them misses in
// that XCD's L2; the slices of a query, which share nothing, go to different
// XCDs.
#include "csa2_device.h"
#include "csa2_internal.h"

namespace csa2 {

constexpr int AT_TILE = 64;
constexpr int AT_IDS = 512;  // entry ids one workgroup handles (8 tiles)
constexpr int AT_IDS_PAD = AT_IDS + 2 * AT_TILE;  // + two tiles of -1 for the look-ahead loads
// Base-2 logits a running softmax reference may lag behind the maximum (the
// 32-head kernel): exponentials stay below 2^8 in fp16, far from its range.
constexpr float RESCALE_SLACK = 8.0f;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D = A(32x16) * B(16x32) + C, fp32 accumulate.  Lane l supplies row (l % 32)
// of A and column (l % 32) of B, each with the 8 k-elements 8 (l / 32) .. + 7;
// element i of lane l is D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32x32x16_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Value of lane (lane ^ 16) / (lane ^ 32) through the permlane swaps.
__device__ __forceinline__ uint32_t xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float xor16f(float v) { return __uint_as_float(xor16(__float_as_uint(v))); }
__device__ __forceinline__ float xor32f(float v) { return __uint_as_float(xor32(__float_as_uint(v))); }

// Transposing LDS read (ds_read_b64_tr_b16): see the PV step below.
__device__ __forceinline__ f16x4 tr16_read(const _Float16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

// Position (in halves) of channel chunk c (32 channels), piece p (8 channels)
// of tile row r in the latent tile: pieces are permuted within a chunk by
// ((c >> 1) & 3) ^ ((r >> 2) & 1).  With a row pitch of 8 (mod 32) dwords this
// makes the dequant stores (8 lanes = 8 chunks of one row), the score reads
// (8 lanes = 8 rows, one piece) and the transposing reads (4 rows x 4 lanes
// inside one piece pair) each touch 32 distinct banks.
__device__ __forceinline__ int tile_col(int r, int c, int p) {
  return 32 * c + 8 * (p ^ ((c >> 1) & 3) ^ ((r >> 2) & 1));
}

// Latent chunk m of the 128 (32 with 128 channels) that PV wave w owns:
// chunks 8 (w >> 1) + (w & 1) + 2m, so that (chunk >> 1) & 3 = m does not
// depend on w and every transposing read address is a per-lane base plus an
// immediate offset.
template <int DC>
__device__ __forceinline__ int pv_chunk(int w, int m) {
  if constexpr (DC >= 512) return 8 * (w >> 1) + (w & 1) + 2 * m;
  else return w;
}

template <int DC, int DR>
struct GatherRegs {
  static constexpr int NCW = DC / 128;               // 16-byte code words per lane (a quarter entry)
  static constexpr int RW = DR > 0 ? DR / 32 : 1;    // 16-byte RoPE words per lane
  u32x4 cw[NCW];
  uint16_t sb[NCW];  // the two scale bytes of each code word
  u32x4 rw[RW];
  bool valid;        // the lane's entry is selected and inside the cache
};

template <int DC, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const CacheRef cache,
    const int32_t* __restrict__ idx, int K, int B, int H, int64_t N_cap, int qps, float sm_scale_log2e, int n_hg,
    int n_split, int per_split, int spread, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int KSL = DC / 32;           // latent k-steps
  constexpr int KSR = DR / 32;           // RoPE k-steps
  constexpr int LDK = DC + 16;           // fp16 pitch of the latent tile (8 mod 32 dwords)
  constexpr int QCH = DC / 4;            // latent channels per PV wave
  constexpr int NDB = QCH / 16;          // PV d-blocks per wave
  using GR = GatherRegs<DC, DR>;
  constexpr int NCW = GR::NCW, RW = GR::RW;
  static_assert(4 * NCW == KSL && (DR == 0 || RW == KSR), "gather layout = MFMA k-steps");
  __shared__ __attribute__((aligned(16))) _Float16 sK[AT_TILE][LDK];
  __shared__ __attribute__((aligned(16))) _Float16 sP[16][AT_TILE + 8];
  __shared__ float sMax[4][16], sSum[4][16], sAlpha[16], sFinM[16], sFinL[16];
  __shared__ int32_t sIdx[AT_IDS_PAD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // workgroup x runs on XCD x % 8, and the head groups of one (query, slice)
  // unit, which gather the same entries, always share that XCD's L2.  With
  // eight queries or more, all of a query's units go to XCD b % 8 (so the
  // combine of its slices finds their partials in that L2); a smaller batch
  // spreads its units, which share nothing, over the XCDs (`spread`).
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  int64_t b;
  int split;
  if (spread) {
    const int64_t unit = (int64_t)(slot / n_hg) * 8 + xcd;
    if (unit >= (int64_t)B * n_split) return;  // padding of the grid to whole groups of eight units
    b = unit / n_split;
    split = (int)(unit - b * n_split);
  } else {
    const int per_q = n_split * n_hg;
    b = (int64_t)(slot / per_q) * 8 + xcd;
    if (b >= B) return;  // padding of the grid to whole groups of eight queries
    split = (slot % per_q) / n_hg;
  }
  const int hg = slot % n_hg;
  const int h0 = hg * 16;
  const int e_begin = split * per_split;
  const int e_end = min(K, e_begin + per_split);
  const int32_t* idx_row = idx + b * K;
  // an empty slice or cache: no loads at all, the epilogue writes the empty result
  const int n_tiles = N_cap > 0 ? (e_end - e_begin + AT_TILE - 1) / AT_TILE : 0;

  // The vector-memory counter retires loads in order and the compiler can
  // only wait for "all but the last n", so every load below is issued
  // unconditionally, in the order its data is needed: entry ids, query heads,
  // then the look-ahead tiles.
  // ---- the slice's entry ids (at most AT_IDS, then -1 padding) go to LDS once
  static_assert(AT_IDS % 256 == 0 && AT_IDS_PAD - AT_IDS <= 256, "id staging layout");
  int32_t ids[AT_IDS / 256];
#pragma unroll
  for (int k = 0; k < AT_IDS / 256; ++k) {
    const int e = e_begin + tid + 256 * k;
    ids[k] = idx_row[min(e, max(e_end - 1, 0))];
  }
  // ---- query heads h0 + n as MFMA B operands: latent k-step t = 4i + j,
  // k-group g -> dims 128i + 32g + 8j .. +7 (the gather's order); RoPE k-step
  // t -> dims d_c + 16g + 8t .. +7
  f16x8 Bq[KSL];
  bf16x8 Br[KSR > 0 ? KSR : 1];
  float fscale;  // multiplies the MFMA result into base-2 softmax logits for head h0 + n
  const bool hv = h0 + n < H;
  u32x4 qraw[KSL + KSR];
  {
    const uint16_t* qrow = q + (b * H + (hv ? h0 + n : 0)) * (DC + DR);
#pragma unroll
    for (int t = 0; t < KSL + KSR; ++t) {
      const int off = t < KSL ? 128 * (t >> 2) + 32 * g + 8 * (t & 3) : DC + 16 * g + 8 * (t - KSL);
      qraw[t] = *reinterpret_cast<const u32x4*>(qrow + off);
    }
  }
#pragma unroll
  for (int k = 0; k < AT_IDS / 256; ++k) {
    const int j = tid + 256 * k;
    sIdx[j] = e_begin + j < e_end ? ids[k] : -1;
  }
  if (tid < AT_IDS_PAD - AT_IDS) sIdx[AT_IDS + tid] = -1;
  __syncthreads();

  // ---- gather (see the header): unconditional loads (a skipped entry reads
  // row 0 of its sequence and has its scales zeroed when it is used), so they
  // issue back to back.
  // Rows of one sequence span less than 4 GiB in each array (checked by the
  // host), so a row's offset from its sequence base is 32-bit arithmetic.
  // Plain (cached) loads: the other head blocks of the query gather the same
  // rows through the same XCD's L2, and a streaming hint would evict them.
  // query b reads the cache of sequence b / qps (qps = 1 in decode; a
  // prefill chunk has qps queries per sequence)
  const int64_t sq = b / qps;
  const uint8_t* seq_codes = cache.codes + sq * N_cap * cache.codes_stride + 16 * g;
  const uint8_t* seq_scales = cache.scales + sq * N_cap * cache.scales_stride + 2 * g;
  const uint8_t* seq_rope = reinterpret_cast<const uint8_t*>(cache.rope) + sq * N_cap * cache.rope_stride + 32 * g;
  const uint32_t cs32 = (uint32_t)cache.codes_stride, ss32 = (uint32_t)cache.scales_stride;
  const uint32_t rs32 = (uint32_t)cache.rope_stride, ncap32 = (uint32_t)min<int64_t>(N_cap, INT32_MAX);
  auto gather = [&](GR& gr, int tile) {
    // pinned in program order: a load hoisted above the previous tile's work
    // lands in registers that are still in flight and forces a full wait
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t id = (uint32_t)sIdx[tile * AT_TILE + 16 * wave + n];
    gr.valid = id < ncap32;  // also rejects negative ids
    const uint32_t r = gr.valid ? id : 0u;
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      gr.cw[i] = *reinterpret_cast<const u32x4*>(seq_codes + r * cs32 + 64 * i);
      gr.sb[i] = *reinterpret_cast<const uint16_t*>(seq_scales + r * ss32 + 8 * i);
    }
    if constexpr (DR > 0) {
#pragma unroll
      for (int t = 0; t < RW; ++t)
        gr.rw[t] = *reinterpret_cast<const u32x4*>(seq_rope + r * rs32 + 16 * t);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  float m_run = -INFINITY, l_run = 0.f;  // per head h0 + n (redundant in every wave)
  f32x4 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](GR& gr) {
    // The scale bytes are first used here and nowhere earlier: a use hoisted
    // into the previous tile's work would wait for loads still in flight.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NCW; ++i) asm volatile("" : "+v"(gr.sb[i]));
    // ---- 1 + 2. dequantise the lane's quarter entry: the two E4M3 scales of
    // a code word through the hardware fp8 converter (exact in fp16), the FP4
    // pairs through the fp4 converter with a unit scale, the block scale with
    // a packed fp16 multiply.  Each 8-channel piece is the A operand of one
    // score k-step and is also stored to the value tile.
    const int e = 16 * wave + n;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(gr.valid ? (uint32_t)gr.sb[i] : 0u, 1.0f, false);
      const f16x2 s_lo = {sc[0], sc[0]}, s_hi = {sc[1], sc[1]};  // channels 0-15 / 16-31 of the word
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t word = gr.cw[i][j];
        const f16x2 sv = j < 2 ? s_lo : s_hi;
        const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sv;
        const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sv;
        const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sv;
        const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sv;
        const f16x8 a = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        *reinterpret_cast<f16x8*>(&sK[e][tile_col(e, 4 * i + g, j)]) = a;
        c = mfma16x16x32_f16(a, Bq[4 * i + j], c);
      }
    }
#pragma unroll
    for (int t = 0; t < KSR; ++t) c = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, gr.rw[t]), Br[t], c);
    // c[i] = S^T[entry 16*wave + 4g + i][head n]; entry validity from lanes 0..15
    const uint64_t vb = __ballot(g == 0 && gr.valid);
    float s2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s2[i] = ((vb >> (4 * g + i)) & 1u) ? c[i] * fscale : -INFINITY;
    // ---- 3. online softmax for head n (lanes n, n+16, n+32, n+48 hold its 16 entries)
    float mt = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mt = fmaxf(mt, xor16f(mt));
    mt = fmaxf(mt, xor32f(mt));
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
    ps += xor16f(ps);
    ps += xor32f(ps);
    if (g == 0) sSum[wave][n] = ps;
    if (wave == 0 && g == 0) sAlpha[n] = alpha;
    {
      _Float16* prow = &sP[n][16 * wave + 4 * g];
      *reinterpret_cast<f16x4*>(prow) = f16x4{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    }
    __syncthreads();
    l_run = l_run * alpha + (sSum[0][n] + sSum[1][n] + sSum[2][n] + sSum[3][n]);
    m_run = m_new;

    // ---- 4. O[heads][channels of this wave] = alpha * O + P . V.  The V
    // operand (8 consecutive entries of one channel per lane) comes from the
    // row-major LDS tile through two transposing reads: in each 16-lane group
    // lane 4r + c points at 4 channels of entry row r, and lane i receives
    // channel i of the four rows.
    {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = sAlpha[4 * g + i];
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[d][i] *= al[i];
      const int tr_r = n >> 2, tr_c = n & 3;
#pragma unroll
      for (int u = 0; u < AT_TILE / 32; ++u) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&sP[n][32 * u + 8 * g]);
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          // 4 channels inside one 8-channel piece of d-block d (16 channels)
          const int ch = 32 * pv_chunk<DC>(wave, d >> 1) + 16 * (d & 1) + 4 * tr_c;
          const int r0 = 32 * u + 8 * g + tr_r, r1 = r0 + 4;
          const f16x4 v0 = tr16_read(&sK[r0][tile_col(r0, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
          const f16x4 v1 = tr16_read(&sK[r1][tile_col(r1, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
          const f16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[d] = mfma16x16x32_f16(a, bv, acc[d]);
        }
      }
    }
    __syncthreads();
  };

  if (n_tiles > 0) {
    GR ga, gb;
    gather(ga, 0);
    {
      uint32_t mx = 0;
#pragma unroll
      for (int t = 0; t < KSL + KSR; ++t) {
        if (!hv) qraw[t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = max(mx, max(qraw[t][j] & 0x7FFFu, (qraw[t][j] >> 16) & 0x7FFFu));
      }
      mx = max(mx, xor16(mx));
      mx = max(mx, xor32(mx));
      // 2^sh brings the largest |q| of the head into [2^14, 2^15): fp16 keeps all
      // of a bf16 value's bits there; bf16 subnormals are treated as exponent -126
      int e = (int)((mx >> 7) & 0xFF) - 127;
      if (e < -126) e = -126;
      const int sh = mx == 0 ? 0 : min(120, max(-120, 14 - e));
      const float up = __builtin_amdgcn_ldexpf(1.0f, sh);
      fscale = sm_scale_log2e * __builtin_amdgcn_ldexpf(1.0f, -sh);
#pragma unroll
      for (int t = 0; t < KSL; ++t) {
        f16x8 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = (_Float16)(bf16_bits_to_f32(qraw[t][j] & 0xFFFFu) * up);
          o[2 * j + 1] = (_Float16)(bf16_bits_to_f32(qraw[t][j] >> 16) * up);
        }
        Bq[t] = o;
      }
#pragma unroll
      for (int t = 0; t < KSR; ++t) {
        bf16x8 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = (__bf16)(bf16_bits_to_f32(qraw[KSL + t][j] & 0xFFFFu) * up);
          o[2 * j + 1] = (__bf16)(bf16_bits_to_f32(qraw[KSL + t][j] >> 16) * up);
        }
        Br[t] = o;
      }
    }
    // the second tile's loads go out once the query registers are converted
    gather(gb, 1);

    // two register sets in flight: while tile t is processed, tiles t+1 and t+2
    // load.  Past the last tile the padding ids (-1) load row 0 again, which
    // keeps every load unconditional; the loop has a single exit so that every
    // path into a process step has the same loads in flight.
    int t = 0;
    for (; t + 2 <= n_tiles; t += 2) {
      process(ga);
      gather(ga, t + 2);
      process(gb);
      gather(gb, t + 3);
    }
    if (t < n_tiles) process(ga);
    // the look-ahead loads past the last tile are never used: wait for them
    // before the wave can end
    __builtin_amdgcn_s_waitcnt(0);
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
      float* orow = out + (b * H + h) * DC;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
        __builtin_nontemporal_store(acc[d][i] * inv, &orow[32 * pv_chunk<DC>(wave, d >> 1) + 16 * (d & 1) + n]);
      if (lse && wave == 0 && n == 0) lse[b * H + h] = l > 0.f ? (m + __log2f(l)) * LN2 : -INFINITY;
    } else {
      const int64_t slot_o = (b * H + h) * n_split + split;
      float* orow = ws_o + slot_o * DC;
#pragma unroll
      for (int d = 0; d < NDB; ++d) orow[32 * pv_chunk<DC>(wave, d >> 1) + 16 * (d & 1) + n] = acc[d][i];
      if (wave == 0 && n == 0) {
        ws_ml[2 * slot_o] = m;
        ws_ml[2 * slot_o + 1] = l;
      }
    }
  }
}

// 32 heads per workgroup with the waves split by role, for batches that fill
// the GPU unsplit.  Waves 0-3 ("score waves") each gather, dequantise and
// score 16 entries of a 64-entry tile against all 32 heads (the dequantised
// words are the A operand of two 16x16x32 products, one per head group, so
// each entry is converted once for 32 heads), store the fp16 values to the
// value tile and their base-2 logits to the score rows.  Waves 4-7 ("value
// waves") each own 128 latent channels of all 32 heads and work on the
// previous tile: each lane takes half of one head's 64 logits, the pair of
// lanes of a head agrees on the new maximum, and the exponentials become the
// A operand of the 32x32x16 value products straight from registers (each
// value element is read from LDS once per workgroup).  Tile t is scored while
// tile t - 1 is multiplied, from two buffers, so one barrier per tile
// separates the roles and the two kinds of work of a SIMD (one wave of each
// role) overlap.
// WIN: the query's sliding window is attended as well, as more tiles of the
// same online softmax after the selected entries' tiles ([P4] CSA2
// paragraph: the SWA branch beside the sparse one, its KV in FP8); its own
// instantiation, so that the registers of the window tiles do not weigh on
// the selected-entry pipeline of the plain kernel.
template <int DR, bool WIN>
__global__ __launch_bounds__(512) void sparse_attn_role_kernel(
    const uint16_t* __restrict__ q, const CacheRef cache,
    const int32_t* __restrict__ idx, int K, int B, int H, int64_t N_cap, int qps, float sm_scale_log2e, int n_hp,
    int n_split, int per_split, int spread, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, const WinRef win) {
  constexpr int DC = 512;
  constexpr int KSL = DC / 32;           // latent k-steps of the scores
  constexpr int KSR = DR / 32;           // RoPE k-steps
  constexpr int KS = KSL + KSR;
  constexpr int LDK = DC + 16;           // fp16 pitch of the value tile
  constexpr int SP = AT_TILE + 4;        // fp32 pitch of the score rows
  using GR = GatherRegs<DC, DR>;
  constexpr int NCW = GR::NCW, RW = GR::RW;
  static_assert(4 * NCW == KSL && (DR == 0 || RW == KSR), "gather layout = MFMA k-steps");
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][AT_TILE][LDK];
  __shared__ __attribute__((aligned(16))) float sS[2][32][SP];     // buffer, head, entry: base-2 logits
  __shared__ __attribute__((aligned(16))) float sHd[4][2][32];     // value wave: per-head broadcast
  __shared__ float sFs[32];                                        // per head: MFMA result -> base-2 logit
  __shared__ int32_t sIdx[AT_IDS_PAD];
  __shared__ float sFw[2][AT_TILE];                                // window tile: sigma_j / max sigma
  __shared__ float sWm[8];                                         // per wave: largest window row scale

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  int64_t b;
  int split;
  if (spread) {
    const int64_t unit = (int64_t)(slot / n_hp) * 8 + xcd;
    if (unit >= (int64_t)B * n_split) return;
    b = unit / n_split;
    split = (int)(unit - b * n_split);
  } else {
    const int per_q = n_split * n_hp;
    b = (int64_t)(slot / per_q) * 8 + xcd;
    if (b >= B) return;
    split = (slot % per_q) / n_hp;
  }
  const int hq0 = (slot % n_hp) * 32;  // heads hq0 .. hq0 + 31
  const int e_begin = split * per_split;
  const int e_end = min(K, e_begin + per_split);
  const int32_t* idx_row = idx + b * K;
  const int n_tiles = N_cap > 0 ? (e_end - e_begin + AT_TILE - 1) / AT_TILE : 0;
  // the query's sliding window (slice 0 only): its rows j < nw are n_wt more
  // tiles after the selected entries', in a second loop (one tile gathered at
  // a time: the window's 128-byte rows per lane have no room for look-ahead
  // buffers beside the entry pipeline's).  Window values are exact E4M3
  // values in fp16; the row scale sigma_j multiplies the latent score in fp32
  // and enters the value products as P * sigma_j / sigma_max, the
  // accumulator being divided by sigma_max before the first window tile and
  // multiplied by it in the epilogue (powers of two: exact)
  const int nw = (WIN && win.codes && split == 0) ? (win.n_win ? min(max(win.n_win[b], 0), win.W_cap) : win.W_cap) : 0;
  const int n_wt = (nw + AT_TILE - 1) / AT_TILE;
  if constexpr (WIN) {
    float sg = 0.f;
    if (tid < nw) sg = win.sigma[b * win.W_cap + tid];  // nw <= 256 < 512 threads
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) sg = fmaxf(sg, __shfl_xor(sg, o));
    if (lane == 0) sWm[wave] = sg;
  }
  // wave-uniform sequence bases (query b reads sequence b / qps); rows are
  // addressed by 32-bit offsets from them
  const int64_t sq = b / qps;
  const uint8_t* seq_codes = cache.codes + sq * N_cap * cache.codes_stride;
  const uint8_t* seq_scales = cache.scales + sq * N_cap * cache.scales_stride;
  const uint8_t* seq_rope = reinterpret_cast<const uint8_t*>(cache.rope) + sq * N_cap * cache.rope_stride;
  const uint32_t cs32 = (uint32_t)cache.codes_stride, ss32 = (uint32_t)cache.scales_stride;
  const uint32_t rs32 = (uint32_t)cache.rope_stride, ncap32 = (uint32_t)min<int64_t>(N_cap, INT32_MAX);

  // ---- entry ids to LDS (one per thread).  The value waves, idle until the
  // first tile has been scored, fetch the 32 query rows meanwhile and convert
  // them (below) into the score waves' B operands: lane (8 heads per wave, 8
  // lanes per head) loads pieces p = sub + 8 m of head hh, piece p = (k-step
  // p / 4, k-group p % 4) in the order the gather lays out the latent.
  static_assert(AT_IDS == 512 && AT_IDS_PAD - AT_IDS <= 512, "id staging layout");
  static_assert(2 * KS * 64 * 16 <= (int)sizeof(sV[1]), "converted query fits the second buffer");
  const int32_t id_t = idx_row[min(e_begin + tid, max(e_end - 1, 0))];
  constexpr int NPC = KS * 4 / 8;
  const int hh = 8 * (wave & 3) + (lane >> 3), sub = lane & 7;
  u32x4 raw[NPC];
  if (wave >= 4) {
    const bool hok = hq0 + hh < H;
    const uint16_t* qrow = q + (b * H + (hok ? hq0 + hh : 0)) * (DC + DR);
#pragma unroll
    for (int m = 0; m < NPC; ++m) {
      const int p = sub + 8 * m, t = p >> 2, gg = p & 3;
      const int off = t < KSL ? 128 * (t >> 2) + 32 * gg + 8 * (t & 3) : DC + 16 * gg + 8 * (t - KSL);
      raw[m] = hok ? *reinterpret_cast<const u32x4*>(qrow + off) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  sIdx[tid] = e_begin + tid < e_end ? id_t : -1;
  if (tid < AT_IDS_PAD - AT_IDS) sIdx[AT_IDS + tid] = -1;
  __syncthreads();
  // iterations: in iteration i the score waves handle tile i (buffer i % 2)
  // and the value waves tile i - 1; an even count, one barrier each
  const int n_iter = n_tiles > 0 ? (n_tiles + 2) & ~1 : 0;
  const int n_iter_w = n_wt > 0 ? (n_wt + 2) & ~1 : 0;
  float sig_max = 0.f;
  if constexpr (WIN) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sig_max = fmaxf(sig_max, sWm[i]);
  }
  const float inv_sig_max = sig_max > 0.f ? 1.0f / sig_max : 0.f;
  // converted query: 16-byte piece (k, t, lane) = head group k, k-step t of
  // score-wave lane (n, g), in the second value buffer (first written by tile 1)
  const u32x4* qcv = reinterpret_cast<const u32x4*>(&sV[1][0][0]);

  if (wave < 4) {
    // ================= score waves: entries 16 * wave + n of each tile
    const int w = wave;
    auto gather = [&](GR& gr, int tile) {
      __builtin_amdgcn_sched_barrier(0);
      tile = min(tile, AT_IDS_PAD / AT_TILE - 1);  // past the last tile: the -1 padding
      const uint32_t id = (uint32_t)sIdx[tile * AT_TILE + 16 * w + n];
      gr.valid = id < ncap32;
      const uint32_t r = gr.valid ? id : 0u;
      const uint32_t oc = r * cs32 + 16 * g, os = r * ss32 + 2 * g, orp = r * rs32 + 32 * g;
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        gr.cw[i] = *reinterpret_cast<const u32x4*>(seq_codes + (oc + 64 * i));
        gr.sb[i] = *reinterpret_cast<const uint16_t*>(seq_scales + (os + 8 * i));
      }
      if constexpr (DR > 0) {
#pragma unroll
        for (int t = 0; t < RW; ++t)
          gr.rw[t] = *reinterpret_cast<const u32x4*>(seq_rope + (orp + 16 * t));
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    f16x8 Bq[2][KSL];
    bf16x8 Br[2][KSR > 0 ? KSR : 1];
    float fscale[2];
    auto process = [&](GR& gr, int buf) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NCW; ++i) asm volatile("" : "+v"(gr.sb[i]));
      _Float16 (*tk)[LDK] = sV[buf];
      const int e = 16 * w + n;
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(gr.valid ? (uint32_t)gr.sb[i] : 0u, 1.0f, false);
        const f16x2 s_lo = {sc[0], sc[0]}, s_hi = {sc[1], sc[1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t word = gr.cw[i][j];
          const f16x2 sv = j < 2 ? s_lo : s_hi;
          const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sv;
          const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sv;
          const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sv;
          const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sv;
          const f16x8 a = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          *reinterpret_cast<f16x8*>(&tk[e][tile_col(e, 4 * i + g, j)]) = a;
          c0 = mfma16x16x32_f16(a, Bq[0][4 * i + j], c0);
          c1 = mfma16x16x32_f16(a, Bq[1][4 * i + j], c1);
        }
      }
#pragma unroll
      for (int t = 0; t < KSR; ++t) {
        const bf16x8 rv = __builtin_bit_cast(bf16x8, gr.rw[t]);
        c0 = mfma16x16x32_bf16(rv, Br[0][t], c0);
        c1 = mfma16x16x32_bf16(rv, Br[1][t], c1);
      }
      // c_k[i] = S^T[entry 16 w + 4 g + i][head hq0 + 16 k + n]: base-2 logits
      // (-inf for a masked entry) to the score rows of the value waves
      const uint64_t vb = __ballot(g == 0 && gr.valid);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x4 c = k ? c1 : c0;
        f32x4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = ((vb >> (4 * g + i)) & 1u) ? c[i] * fscale[k] : -INFINITY;
        *reinterpret_cast<f32x4*>(&sS[buf][16 * k + n][16 * w + 4 * g]) = sv;
      }
    };

    // ---- window rows: row 64 tile + 16 w + n, the lane's channels 128 i +
    // 32 g .. + 31 (i < 4) as two 16-byte words of E4M3 values each, 16
    // channels of the RoPE part and the row scale
    struct WinRegs {
      u32x4 cw[8];
      u32x4 rw[RW];
      float sig;
      bool valid;
    };
    auto wgather = [&](WinRegs& wr, int tile) {
      __builtin_amdgcn_sched_barrier(0);
      const int row = tile * AT_TILE + 16 * w + n;
      wr.valid = row < nw;
      const int64_t rr = b * win.W_cap + (wr.valid ? row : 0);
      const uint8_t* crow = win.codes + rr * win.codes_stride + 32 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wr.cw[2 * i] = *reinterpret_cast<const u32x4*>(crow + 128 * i);
        wr.cw[2 * i + 1] = *reinterpret_cast<const u32x4*>(crow + 128 * i + 16);
      }
      if constexpr (DR > 0) {
        const uint8_t* rrow = reinterpret_cast<const uint8_t*>(win.rope) + rr * win.rope_stride + 32 * g;
#pragma unroll
        for (int t = 0; t < RW; ++t) wr.rw[t] = *reinterpret_cast<const u32x4*>(rrow + 16 * t);
      }
      wr.sig = win.sigma[rr];
      __builtin_amdgcn_sched_barrier(0);
    };
    // exact E4M3 -> fp16 into the value tile and the score products (latent
    // and RoPE in separate accumulators: the row scale multiplies the latent
    // part only); the value waves get sigma_j / max sigma for the entry.  Each
    // register of wr is refilled with the same piece of window tile `next`
    // (none when next < 0) right after its last use, so the next tile's rows
    // are in flight while this one is scored, with no second buffer.
    auto wprocess = [&](WinRegs& wr, int buf, int next) {
      __builtin_amdgcn_sched_barrier(0);
      _Float16 (*tk)[LDK] = sV[buf];
      const int e = 16 * w + n;
      const bool valid = wr.valid;
      const float sig = wr.sig;
      const int nrow = next * AT_TILE + 16 * w + n;
      const bool nvalid = next >= 0 && nrow < nw;
      const int64_t nrr = b * win.W_cap + (nvalid ? nrow : 0);
      const uint8_t* ncrow = win.codes + nrr * win.codes_stride + 32 * g;
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
      f32x4 r0 = {0.f, 0.f, 0.f, 0.f}, r1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 src = wr.cw[2 * i + (j >> 1)];
          const uint32_t lo = src[2 * (j & 1)], hi = src[2 * (j & 1) + 1];
          const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
          const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
          const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
          const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
          f16x8 a = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          if (!valid) a = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
          *reinterpret_cast<f16x8*>(&tk[e][tile_col(e, 4 * i + g, j)]) = a;
          c0 = mfma16x16x32_f16(a, Bq[0][4 * i + j], c0);
          c1 = mfma16x16x32_f16(a, Bq[1][4 * i + j], c1);
          if ((j & 1) && next >= 0)
            wr.cw[2 * i + (j >> 1)] = *reinterpret_cast<const u32x4*>(ncrow + 128 * i + 16 * (j >> 1));
        }
      }
#pragma unroll
      for (int t = 0; t < KSR; ++t) {
        const bf16x8 rv = __builtin_bit_cast(bf16x8, wr.rw[t]);
        r0 = mfma16x16x32_bf16(rv, Br[0][t], r0);
        r1 = mfma16x16x32_bf16(rv, Br[1][t], r1);
        if (next >= 0)
          wr.rw[t] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(win.rope) +
                                                     nrr * win.rope_stride + 32 * g + 16 * t);
      }
      // c_k[i], r_k[i]: entry 16 w + 4 g + i, head hq0 + 16 k + n; its row
      // scale is held by lane 4 g + i
      float sg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sg[i] = __shfl(sig, 4 * g + i);
      const uint64_t vb = __ballot(g == 0 && valid);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x4 c = k ? c1 : c0, rp = k ? r1 : r0;
        f32x4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sv[i] = ((vb >> (4 * g + i)) & 1u) ? (c[i] * sg[i] + rp[i]) * fscale[k] : -INFINITY;
        *reinterpret_cast<f32x4*>(&sS[buf][16 * k + n][16 * w + 4 * g]) = sv;
      }
      if (g == 0) sFw[buf][e] = sig * inv_sig_max;
      if (next >= 0) {
        wr.sig = win.sigma[nrr];
        wr.valid = nvalid;
      }
    };

    GR ga, gb;
    if (n_iter > 0) {
      gather(ga, 0);
      gather(gb, 1);
    }
    __syncthreads();  // the value waves have written the converted query
    if (n_iter + n_iter_w > 0) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
#pragma unroll
        for (int t = 0; t < KSL; ++t) Bq[k][t] = __builtin_bit_cast(f16x8, qcv[(k * KS + t) * 64 + lane]);
#pragma unroll
        for (int t = 0; t < KSR; ++t) Br[k][t] = __builtin_bit_cast(bf16x8, qcv[(k * KS + KSL + t) * 64 + lane]);
        fscale[k] = sFs[16 * k + n];
      }
    }
    if (n_iter > 0) {
      // every gather is unconditional (past the last tile they load row 0
      // again), so each process step waits for exactly the loads it needs
      for (int i = 0; i < n_iter; i += 2) {
        if (i < n_tiles) process(ga, 0);
        gather(ga, i + 2);
        __syncthreads();
        if (i + 1 < n_tiles) process(gb, 1);
        gather(gb, i + 3);
        __syncthreads();
      }
      // the two look-ahead gathers past the last tile are never used: the wave
      // waits for them, so that no load returns into its registers after it
      // has ended and they have been handed to another wave
      __builtin_amdgcn_s_waitcnt(0);
    }
    // window tiles: the first gathered here, each later one while the tile
    // before it is scored
    if (n_wt > 0) {
      WinRegs wr;
      wgather(wr, 0);
      for (int i = 0; i < n_iter_w; i += 2) {
        if (i < n_wt) wprocess(wr, 0, i + 1 < n_wt ? i + 1 : -1);
        __syncthreads();
        if (i + 1 < n_wt) wprocess(wr, 1, i + 2 < n_wt ? i + 2 : -1);
        __syncthreads();
      }
    }
    return;
  }

  // ================= value waves: channels 128 r .. + 127 of all 32 heads
  const int r = wave - 4;
  // ---- query conversion (the rows were fetched before the first barrier)
  {
    uint32_t mx = 0;
#pragma unroll
    for (int m = 0; m < NPC; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(raw[m][j] & 0x7FFFu, (raw[m][j] >> 16) & 0x7FFFu));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 4));
    // 2^sh brings the largest |q| of the head into [2^14, 2^15), where fp16
    // keeps every bit of a bf16 value; bf16 subnormals count as exponent -126
    int ex = (int)((mx >> 7) & 0xFF) - 127;
    if (ex < -126) ex = -126;
    const int sh = mx == 0 ? 0 : min(120, max(-120, 14 - ex));
    const float up = __builtin_amdgcn_ldexpf(1.0f, sh);
    u32x4* qc = reinterpret_cast<u32x4*>(&sV[1][0][0]);
    const int k = hh >> 4, nn = hh & 15;
#pragma unroll
    for (int m = 0; m < NPC; ++m) {
      const int p = sub + 8 * m, t = p >> 2, gg = p & 3;
      u32x4 o;
      if (t < KSL) {
        f16x8 h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[2 * j] = (_Float16)(bf16_bits_to_f32(raw[m][j] & 0xFFFFu) * up);
          h[2 * j + 1] = (_Float16)(bf16_bits_to_f32(raw[m][j] >> 16) * up);
        }
        o = __builtin_bit_cast(u32x4, h);
      } else {
        bf16x8 h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[2 * j] = (__bf16)(bf16_bits_to_f32(raw[m][j] & 0xFFFFu) * up);
          h[2 * j + 1] = (__bf16)(bf16_bits_to_f32(raw[m][j] >> 16) * up);
        }
        o = __builtin_bit_cast(u32x4, h);
      }
      qc[(k * KS + t) * 64 + 16 * gg + nn] = o;
    }
    if (sub == 0) sFs[hh] = sm_scale_log2e * __builtin_amdgcn_ldexpf(1.0f, -sh);
    __syncthreads();  // the converted operands are in place
  }

  const int hl = lane & 31, kh = lane >> 5;  // A-operand row (head) and k-half of this lane
  float m_run = -INFINITY, l_run = 0.f;      // head hq0 + hl
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
  // transposing reads: lane group G = lane / 16 supplies channels 16 (G % 2) +
  // 0..15 of entries 8 (G / 2) + 0..7 of a 16-entry k-step; lane 4 tr_r + tr_c
  // points at 4 channels of one entry row
  const int G = lane >> 4, tr_r = (lane & 15) >> 2, tr_c = lane & 3;

  // wtile: a window tile, whose P enters the value products as P * sigma_j /
  // max sigma; the first one divides the accumulator by max sigma
  auto pv = [&](int buf, bool wtile, bool first_w) {
    _Float16 (*tk)[LDK] = sV[buf];
    // ---- softmax of head hl over the tile: this lane holds entries 16 u +
    // 8 kh + 0..7 (u < 4), its partner lane hl + 32 the other half
    f32x4 sv[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sv[2 * u] = *reinterpret_cast<const f32x4*>(&sS[buf][hl][16 * u + 8 * kh]);
      sv[2 * u + 1] = *reinterpret_cast<const f32x4*>(&sS[buf][hl][16 * u + 8 * kh + 4]);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) mt = fmaxf(mt, fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3])));
    mt = fmaxf(mt, xor32f(mt));
    // the reference moves only when the tile's maximum passes it by more
    // than RESCALE_SLACK (the first finite logit always moves it), so the
    // exponentials stay below 2^RESCALE_SLACK and most tiles leave the
    // accumulator unscaled; softmax is unchanged by the choice of reference
    const bool move = mt > m_run + RESCALE_SLACK;
    const float m_new = move ? mt : m_run;
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // nothing valid yet: O = l = 0
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.f;
    f16x8 a[4];
    float ps = 0.f;
    if (wtile) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sFw[buf][16 * u + 8 * kh]);
        const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sFw[buf][16 * u + 8 * kh + 4]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(sv[2 * u + (j >> 2)][j & 3] - m_ref);
          ps += p;
          a[u][j] = (_Float16)(p * (j < 4 ? f0[j & 3] : f1[j & 3]));
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(sv[2 * u + (j >> 2)][j & 3] - m_ref);
          ps += p;
          a[u][j] = (_Float16)p;
        }
      }
    }
    ps += xor32f(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // alpha of the heads whose output rows this lane holds: 8 q + 4 kh + 0..3
    // (skipped, wave-uniformly, when no head of the wave moved its reference)
    if (__any(move) || (first_w && sig_max > 0.f)) {
      if (kh == 0) sHd[r][0][hl] = alpha;
      f32x4 al[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) al[qq] = *reinterpret_cast<const f32x4*>(&sHd[r][0][8 * qq + 4 * kh]);
      if (first_w && sig_max > 0.f) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) al[qq] *= inv_sig_max;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[k][i] *= al[i >> 2][i & 3];
    }
#pragma unroll
    for (int u = 0; u < AT_TILE / 16; ++u) {
      const int r0 = 16 * u + 8 * (G >> 1) + tr_r, r1 = r0 + 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ch = 32 * (4 * r + k) + 16 * (G & 1) + 4 * tr_c;
        const f16x4 v0 = tr16_read(&tk[r0][tile_col(r0, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
        const f16x4 v1 = tr16_read(&tk[r1][tile_col(r1, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
        const f16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[k] = mfma32x32x16_f16(a[u], bv, acc[k]);
      }
    }
  };

  for (int i = 0; i < n_iter; i += 2) {
    if (i >= 1 && i - 1 < n_tiles) pv(1, false, false);
    __syncthreads();
    if (i < n_tiles) pv(0, false, false);
    __syncthreads();
  }
  for (int i = 0; i < n_iter_w; i += 2) {
    if (i >= 1 && i - 1 < n_wt) pv(1, true, false);
    __syncthreads();
    if (i < n_wt) pv(0, true, i == 0);
    __syncthreads();
  }
  const float tail = (n_wt > 0 && sig_max > 0.f) ? sig_max : 1.f;

  // ---- epilogue: element i of acc[k] is head 8 (i / 4) + 4 kh + i % 4,
  // channel 32 (4 r + k) + hl
  if (kh == 0) {
    sHd[r][0][hl] = m_run;
    sHd[r][1][hl] = l_run;
  }
  f32x4 lv[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) lv[qq] = *reinterpret_cast<const f32x4*>(&sHd[r][1][8 * qq + 4 * kh]);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int hh = 8 * (i >> 2) + 4 * kh + (i & 3);
    const int h = hq0 + hh;
    if (h >= H) continue;
    const float l = lv[i >> 2][i & 3];
    if (n_split == 1) {
      const float inv = l > 0.f ? tail / l : 0.f;
      float* orow = out + (b * H + h) * DC + 128 * r + hl;
#pragma unroll
      // final outputs are streamed past the caches (non-temporal stores):
      // nothing here reads them again, and L2 lines left dirty would have to
      // be written back before the kernel counts as finished (measured:
      // reuse-128k attention 23.8 -> 23.1 us); the split partials, which the
      // merge kernel reads on the same XCD, keep ordinary stores
      for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(acc[k][i] * inv, &orow[32 * k]);
    } else {
      float* orow = ws_o + ((b * H + h) * n_split + split) * DC + 128 * r + hl;
#pragma unroll
      for (int k = 0; k < 4; ++k) orow[32 * k] = acc[k][i] * tail;
    }
  }
  if (r == 0 && kh == 0 && hq0 + hl < H) {
    const int64_t row = b * H + hq0 + hl;
    if (n_split == 1) {
      if (lse) lse[row] = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
    } else {
      ws_ml[2 * (row * n_split + split)] = m_run;
      ws_ml[2 * (row * n_split + split) + 1] = l_run;
    }
  }
}

// The 32-head kernel as a persistent loop, for launches with more (query,
// 32-head) units than CUs and one slice per query (prefill chunks): workgroup
// x takes units x, x + G, x + 2G, ... (G workgroups, a multiple of eight, so
// every unit keeps the XCD of the one-unit-per-workgroup grid) and walks their
// tiles as one stream.  The score and value waves and the per-tile work are
// those of sparse_attn_role_kernel; what changes is the hand-over between
// units, which that kernel pays as a workgroup's start-up (ids, then the
// gathers; the query fetched and converted) and drain:
//  * one boundary step per unit: the value waves multiply the last tile of
//    the unit before and convert this unit's query, whose rows they fetched
//    one unit earlier, into the value buffer that no tile occupies at that
//    moment; the score waves take their operands from there after the step's
//    barrier, and score the unit's first tile while the value waves write
//    the outputs of the unit before;
//  * the score waves' look-ahead gathers run on across the boundary (the
//    first two tiles of a unit load during the last two of the unit before);
//  * the entry ids are double-buffered in LDS: the value waves fetch a unit's
//    ids two units ahead and store them during the boundary step before it.
// Tile j of unit u (T tiles per unit) uses value buffer X_u ^ (j & 1), with
// X_u = (T odd) ? 0 : u & 1, so the buffer the value waves read in a boundary
// step (the unit before's last tile) is X_u and the converted query goes to
// X_u ^ 1, which the unit's tile 1 overwrites only after every score wave has
// read it.  Needs T >= 2 (the look-ahead reaches one unit ahead only).
template <int DR>
__global__ __launch_bounds__(512) void sparse_attn_role_stream_kernel(
    const uint16_t* __restrict__ q, const CacheRef cache, const int32_t* __restrict__ idx, int K, int B, int H,
    int64_t N_cap, int qps, float sm_scale_log2e, int n_hp, int64_t n_units, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int DC = 512;
  constexpr int KSL = DC / 32;
  constexpr int KSR = DR / 32;
  constexpr int KS = KSL + KSR;
  constexpr int LDK = DC + 16;
  constexpr int SP = AT_TILE + 4;
  using GR = GatherRegs<DC, DR>;
  constexpr int NCW = GR::NCW, RW = GR::RW;
  static_assert(4 * NCW == KSL && (DR == 0 || RW == KSR), "gather layout = MFMA k-steps");
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][AT_TILE][LDK];
  __shared__ __attribute__((aligned(16))) float sS[2][32][SP];
  __shared__ __attribute__((aligned(16))) float sHd[4][2][32];
  __shared__ float sFs[32];
  __shared__ int32_t sIdx[2][AT_IDS];
  static_assert(2 * KS * 64 * 16 <= (int)sizeof(sV[1]), "converted query fits one value buffer");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int T = (K + AT_TILE - 1) / AT_TILE;  // 2 .. 8 (checked by the host)
  // this workgroup's units: v = blockIdx.x + k G for k < n_my; unit v is query
  // b = (v / 8 / n_hp) * 8 + v % 8, heads 32 ((v / 8) % n_hp) ..; units with
  // b >= B (the padding of the batch to eight) come last in every sequence
  // (n_units < 2^31, checked by the host: unit numbers are 32-bit)
  const uint32_t G = gridDim.x, nhp = (uint32_t)n_hp;
  auto unit_b = [&](int k) -> int64_t {
    const uint32_t v = blockIdx.x + (uint32_t)k * G;
    return (int64_t)(((v >> 3) / nhp) * 8 + (v & 7));
  };
  auto unit_h0 = [&](int k) -> int {
    const uint32_t v = blockIdx.x + (uint32_t)k * G;
    return (int)((v >> 3) % nhp) * 32;
  };
  int n_my = 0;
  {
    const int cnt = n_units > (int64_t)blockIdx.x ? (int)((n_units - 1 - blockIdx.x) / G) + 1 : 0;
    int lo = 0, hi = cnt;  // the first k whose query is padding
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (unit_b(mid) < B) lo = mid + 1;
      else hi = mid;
    }
    n_my = lo;
  }
  if (n_my == 0) return;
  const uint32_t cs32 = (uint32_t)cache.codes_stride, ss32 = (uint32_t)cache.scales_stride;
  const uint32_t rs32 = (uint32_t)cache.rope_stride, ncap32 = (uint32_t)min<int64_t>(N_cap, INT32_MAX);

  // ---- unit 0's entry ids to LDS (one per thread, -1 past K)
  {
    const int64_t b0 = unit_b(0);
    const int32_t id = idx[b0 * K + min(tid, K - 1)];
    sIdx[0][tid] = tid < K ? id : -1;
  }
  constexpr int NPC = KS * 4 / 8;
  const int hh = 8 * (wave & 3) + (lane >> 3), sub = lane & 7;

  if (wave < 4) {
    // ================= score waves
    const int w = wave;
    // gather tile j of unit k (k >= n_my: a masked load of row 0)
    auto gather = [&](GR& gr, int k, int j) {
      __builtin_amdgcn_sched_barrier(0);
      const bool uok = k < n_my;
      const int64_t sq = unit_b(uok ? k : n_my - 1) / qps;
      const uint8_t* seq_codes = cache.codes + sq * N_cap * cache.codes_stride;
      const uint8_t* seq_scales = cache.scales + sq * N_cap * cache.scales_stride;
      const uint8_t* seq_rope = reinterpret_cast<const uint8_t*>(cache.rope) + sq * N_cap * cache.rope_stride;
      const uint32_t id = uok ? (uint32_t)sIdx[k & 1][j * AT_TILE + 16 * w + n] : 0xFFFFFFFFu;
      gr.valid = id < ncap32;
      const uint32_t r = gr.valid ? id : 0u;
      const uint32_t oc = r * cs32 + 16 * g, os = r * ss32 + 2 * g, orp = r * rs32 + 32 * g;
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        gr.cw[i] = *reinterpret_cast<const u32x4*>(seq_codes + (oc + 64 * i));
        gr.sb[i] = *reinterpret_cast<const uint16_t*>(seq_scales + (os + 8 * i));
      }
      if constexpr (DR > 0) {
#pragma unroll
        for (int t = 0; t < RW; ++t) gr.rw[t] = *reinterpret_cast<const u32x4*>(seq_rope + (orp + 16 * t));
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    f16x8 Bq[2][KSL];
    bf16x8 Br[2][KSR > 0 ? KSR : 1];
    float fscale[2];
    auto process = [&](GR& gr, int buf) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NCW; ++i) asm volatile("" : "+v"(gr.sb[i]));
      _Float16 (*tk)[LDK] = sV[buf];
      const int e = 16 * w + n;
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(gr.valid ? (uint32_t)gr.sb[i] : 0u, 1.0f, false);
        const f16x2 s_lo = {sc[0], sc[0]}, s_hi = {sc[1], sc[1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t word = gr.cw[i][j];
          const f16x2 sv = j < 2 ? s_lo : s_hi;
          const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sv;
          const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sv;
          const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sv;
          const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sv;
          const f16x8 a = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          *reinterpret_cast<f16x8*>(&tk[e][tile_col(e, 4 * i + g, j)]) = a;
          c0 = mfma16x16x32_f16(a, Bq[0][4 * i + j], c0);
          c1 = mfma16x16x32_f16(a, Bq[1][4 * i + j], c1);
        }
      }
#pragma unroll
      for (int t = 0; t < KSR; ++t) {
        const bf16x8 rv = __builtin_bit_cast(bf16x8, gr.rw[t]);
        c0 = mfma16x16x32_bf16(rv, Br[0][t], c0);
        c1 = mfma16x16x32_bf16(rv, Br[1][t], c1);
      }
      const uint64_t vb = __ballot(g == 0 && gr.valid);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x4 c = k ? c1 : c0;
        f32x4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = ((vb >> (4 * g + i)) & 1u) ? c[i] * fscale[k] : -INFINITY;
        *reinterpret_cast<f32x4*>(&sS[buf][16 * k + n][16 * w + 4 * g]) = sv;
      }
    };

    __syncthreads();  // unit 0's ids are in place
    GR ga, gb;
    gather(ga, 0, 0);
    gather(gb, 0, 1);
    // one step per tile: (k, j) is the tile processed, (nk, nj) the one two
    // tiles later whose gather follows; gathers alternate between ga and gb
    // along the stream (tile s of the stream in ga when s is even)
    int k = 0, j = 0;
    const int total = n_my * T;
    auto step = [&](GR& gr) {
      const int X = (T & 1) ? 0 : (k & 1);
      if (j == 0) {
        __syncthreads();  // boundary step: the value waves convert unit k's query into buffer X ^ 1
        const u32x4* qcv = reinterpret_cast<const u32x4*>(&sV[X ^ 1][0][0]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int t = 0; t < KSL; ++t) Bq[kk][t] = __builtin_bit_cast(f16x8, qcv[(kk * KS + t) * 64 + lane]);
#pragma unroll
          for (int t = 0; t < KSR; ++t) Br[kk][t] = __builtin_bit_cast(bf16x8, qcv[(kk * KS + KSL + t) * 64 + lane]);
          fscale[kk] = sFs[16 * kk + n];
        }
      }
      process(gr, X ^ (j & 1));
      int nj = j + 2, nk = k;
      if (nj >= T) {
        nj -= T;
        ++nk;
      }
      gather(gr, nk, nj);
      __syncthreads();
      if (++j == T) {
        j = 0;
        ++k;
      }
    };
    int s = 0;
    for (; s + 2 <= total; s += 2) {
      step(ga);
      step(gb);
    }
    if (s < total) step(ga);
    // the look-ahead gathers past the last tile are never used: wait for them
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // ================= value waves: channels 128 r .. + 127 of all 32 heads
  const int r = wave - 4;
  // the query rows of unit k (8 heads per wave, 8 lanes per head; pieces in
  // the order the gather lays out the latent) and the ids of unit k (two per
  // lane), fetched one and two units ahead of their use
  u32x4 raw[NPC];
  auto fetch_query = [&](int k) {
    const int h = unit_h0(k) + hh;
    const bool hok = h < H;
    const uint16_t* qrow = q + (unit_b(k) * H + (hok ? h : 0)) * (DC + DR);
#pragma unroll
    for (int m = 0; m < NPC; ++m) {
      const int p = sub + 8 * m, t = p >> 2, gg = p & 3;
      const int off = t < KSL ? 128 * (t >> 2) + 32 * gg + 8 * (t & 3) : DC + 16 * gg + 8 * (t - KSL);
      raw[m] = hok ? *reinterpret_cast<const u32x4*>(qrow + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  const int tv = tid - 256;  // 0 .. 255
  int32_t nid[2];
  auto fetch_ids = [&](int k) {
    const int64_t bk = unit_b(k < n_my ? k : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) nid[i] = idx[bk * K + min(tv + 256 * i, K - 1)];
  };
  auto store_ids = [&](int k) {
#pragma unroll
    for (int i = 0; i < 2; ++i) sIdx[k & 1][tv + 256 * i] = tv + 256 * i < K ? nid[i] : -1;
  };
  // converts raw into the score waves' operands in value buffer `buf`
  auto convert_query = [&](int buf) {
    uint32_t mx = 0;
#pragma unroll
    for (int m = 0; m < NPC; ++m)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) mx = max(mx, max(raw[m][jj] & 0x7FFFu, (raw[m][jj] >> 16) & 0x7FFFu));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 4));
    // 2^sh brings the largest |q| of the head into [2^14, 2^15), where fp16
    // keeps every bit of a bf16 value; bf16 subnormals count as exponent -126
    int ex = (int)((mx >> 7) & 0xFF) - 127;
    if (ex < -126) ex = -126;
    const int sh = mx == 0 ? 0 : min(120, max(-120, 14 - ex));
    const float up = __builtin_amdgcn_ldexpf(1.0f, sh);
    u32x4* qc = reinterpret_cast<u32x4*>(&sV[buf][0][0]);
    const int kq = hh >> 4, nn = hh & 15;
#pragma unroll
    for (int m = 0; m < NPC; ++m) {
      const int p = sub + 8 * m, t = p >> 2, gg = p & 3;
      u32x4 o;
      if (t < KSL) {
        f16x8 h;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          h[2 * jj] = (_Float16)(bf16_bits_to_f32(raw[m][jj] & 0xFFFFu) * up);
          h[2 * jj + 1] = (_Float16)(bf16_bits_to_f32(raw[m][jj] >> 16) * up);
        }
        o = __builtin_bit_cast(u32x4, h);
      } else {
        bf16x8 h;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          h[2 * jj] = (__bf16)(bf16_bits_to_f32(raw[m][jj] & 0xFFFFu) * up);
          h[2 * jj + 1] = (__bf16)(bf16_bits_to_f32(raw[m][jj] >> 16) * up);
        }
        o = __builtin_bit_cast(u32x4, h);
      }
      qc[(kq * KS + t) * 64 + 16 * gg + nn] = o;
    }
    if (sub == 0) sFs[hh] = sm_scale_log2e * __builtin_amdgcn_ldexpf(1.0f, -sh);
  };

  const int hl = lane & 31, kh = lane >> 5;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[kk][i] = 0.f;
  const int G4 = lane >> 4, tr_r = (lane & 15) >> 2, tr_c = lane & 3;

  auto pv = [&](int buf) {
    _Float16 (*tk)[LDK] = sV[buf];
    f32x4 sv[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sv[2 * u] = *reinterpret_cast<const f32x4*>(&sS[buf][hl][16 * u + 8 * kh]);
      sv[2 * u + 1] = *reinterpret_cast<const f32x4*>(&sS[buf][hl][16 * u + 8 * kh + 4]);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) mt = fmaxf(mt, fmaxf(fmaxf(sv[jj][0], sv[jj][1]), fmaxf(sv[jj][2], sv[jj][3])));
    mt = fmaxf(mt, xor32f(mt));
    const bool move = mt > m_run + RESCALE_SLACK;
    const float m_new = move ? mt : m_run;
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.f;
    f16x8 a[4];
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = __builtin_amdgcn_exp2f(sv[2 * u + (jj >> 2)][jj & 3] - m_ref);
        ps += p;
        a[u][jj] = (_Float16)p;
      }
    }
    ps += xor32f(ps);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(move)) {
      if (kh == 0) sHd[r][0][hl] = alpha;
      f32x4 al[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) al[qq] = *reinterpret_cast<const f32x4*>(&sHd[r][0][8 * qq + 4 * kh]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[kk][i] *= al[i >> 2][i & 3];
    }
#pragma unroll
    for (int u = 0; u < AT_TILE / 16; ++u) {
      const int r0 = 16 * u + 8 * (G4 >> 1) + tr_r, r1 = r0 + 4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = 32 * (4 * r + kk) + 16 * (G4 & 1) + 4 * tr_c;
        const f16x4 v0 = tr16_read(&tk[r0][tile_col(r0, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
        const f16x4 v1 = tr16_read(&tk[r1][tile_col(r1, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
        const f16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[kk] = mfma32x32x16_f16(a[u], bv, acc[kk]);
      }
    }
  };
  // outputs of unit k: element i of acc[kk] is head 8 (i / 4) + 4 kh + i % 4,
  // channel 32 (4 r + kk) + hl; the state is reset for the next unit
  auto epilogue = [&](int k) {
    const int64_t bk = unit_b(k);
    const int h0 = unit_h0(k);
    if (kh == 0) sHd[r][1][hl] = l_run;
    f32x4 lv[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) lv[qq] = *reinterpret_cast<const f32x4*>(&sHd[r][1][8 * qq + 4 * kh]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = h0 + 8 * (i >> 2) + 4 * kh + (i & 3);
      if (h >= H) continue;
      const float l = lv[i >> 2][i & 3];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float* orow = out + (bk * H + h) * DC + 128 * r + hl;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) __builtin_nontemporal_store(acc[kk][i] * inv, &orow[32 * kk]);
    }
    if (r == 0 && kh == 0 && h0 + hl < H && lse)
      lse[bk * H + h0 + hl] = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[kk][i] = 0.f;
  };

  fetch_query(0);
  fetch_ids(1);
  __syncthreads();  // unit 0's ids are in place
  for (int k = 0; k < n_my; ++k) {
    // boundary step of unit k (the score waves wait at its barrier): the
    // last tile of unit k - 1, whose buffer tile 0 of unit k overwrites next,
    // and unit k's query
    const int X = (T & 1) ? 0 : (k & 1);
    if (k > 0) pv(X);
    convert_query(X ^ 1);
    if (k + 1 < n_my) store_ids(k + 1);
    __syncthreads();
    // while tile 0 of unit k is scored: the outputs of unit k - 1, then the
    // fetches for the next units (after the stores, so that the query rows
    // are not held in registers beside the accumulators)
    if (k > 0) epilogue(k - 1);
    if (k + 1 < n_my) fetch_query(k + 1);
    if (k + 2 < n_my) fetch_ids(k + 2);
    __syncthreads();
    for (int jt = 1; jt < T; ++jt) {
      pv(X ^ ((jt - 1) & 1));
      __syncthreads();
    }
  }
  {
    const int X = (T & 1) ? 0 : (n_my & 1);  // the last tile's buffer
    pv(X);
    epilogue(n_my - 1);
  }
}

// Merge the per-slice partial results of one (b, h) row by log-sum-exp; each
// of the 128 threads owns 4 consecutive channels (d_c <= 512).  The slices are
// taken 8 at a time with every load of a round issued together (one memory
// round trip per 8 slices), merged online.  Unless the attention spread its
// slices (`spread`: block x merges row x), block x runs on XCD x % 8 like the
// attention workgroups of its query, whose partials sit in that XCD's L2.
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ ws_o,
                                                           const float* __restrict__ ws_ml,
                                                           int B, int H, int n_split, int DC, int spread,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse) {
  constexpr int R = 8;
  int64_t row;
  if (spread) {
    row = blockIdx.x;
  } else {
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int64_t b = (int64_t)(slot / H) * 8 + xcd;
    if (b >= B) return;
    row = b * H + slot % H;
  }
  const float* ml = ws_ml + row * n_split * 2;
  const int c = 4 * threadIdx.x;
  const bool has = c < DC;
  const float* po = ws_o + row * n_split * DC + (has ? c : 0);
  float m = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += R) {
    float mm[R], ll[R];
    f32x4 v[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const bool ok = s0 + j < n_split;
      mm[j] = ok ? ml[2 * (s0 + j)] : -INFINITY;
      ll[j] = ok ? ml[2 * (s0 + j) + 1] : 0.f;
      v[j] = ok && has ? *reinterpret_cast<const f32x4*>(po + (int64_t)(s0 + j) * DC) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mn = m;
#pragma unroll
    for (int j = 0; j < R; ++j) mn = fmaxf(mn, mm[j]);
    const float a = mn == -INFINITY ? 1.f : exp2f(m - mn);
    L *= a;
    o *= a;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float w = mm[j] == -INFINITY ? 0.f : exp2f(mm[j] - mn);
      L += w * ll[j];
      o += v[j] * w;
    }
    m = mn;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  if (has) __builtin_nontemporal_store(o * inv, reinterpret_cast<f32x4*>(out + row * DC + c));
  if (lse && threadIdx.x == 0) lse[row] = L > 0.f ? (m + __log2f(L)) * LN2 : -INFINITY;
}

// Heads per workgroup: 32 (score waves and value waves) for the 512-channel
// latent when the batch gives at least 64 (query, head group) units, i.e. at
// most four slices per query, else 16.  Measured: the 32-head kernel is
// faster unsplit (batch 128: 25.6 vs 34.7 us) and with four slices (batch
// 32: 16.9 vs 19.1 us) but slower with eight or more (batch 8: 12.4 vs 11.8
// us; batch 1: 12.1 vs 10.8 us), where the per-workgroup latency path rather
// than the CU's throughput sets the time.
static int attn_heads_per_wg(int B, int H, int d_c) {
  return (d_c == 512 && H > 16 && (int64_t)B * ((H + 31) / 32) >= 64) ? 32 : 16;
}

// Slices per query: enough workgroups for 256 CUs, whole 64-entry tiles.
static void attn_plan(int B, int H, int K, int d_c, int* n_split, int* per_split) {
  const int hpw = attn_heads_per_wg(B, H, d_c);
  const int n_hg = (H + hpw - 1) / hpw;
  const int tiles = (int)(((int64_t)K + AT_TILE - 1) / AT_TILE);
  const int64_t base = (int64_t)B * n_hg;
  // at most one workgroup per CU: measured, splitting further (two per CU)
  // costs more in partials and contention than it gains in parallelism, and
  // a second, partial round of workgroups costs a whole workgroup lifetime
  int s = base >= 256 ? 1 : (int)(256 / (base > 1 ? base : 1));
  s = max(s, (tiles + AT_IDS / AT_TILE - 1) / (AT_IDS / AT_TILE));  // <= 8 tiles per split
  s = max(1, min(s, tiles));
  const int tps = (tiles + s - 1) / s;
  s = (tiles + tps - 1) / tps;
  *n_split = s;
  *per_split = tps * AT_TILE;
}

// The persistent 32-head kernel: one workgroup per CU walking several units
// each, when the query is unsplit, has 2 to 8 tiles, and the units outnumber
// the workgroups.
constexpr int AT_STREAM_WG = 256;
static bool attn_streamed(int hpw, int n_split, int K, int64_t n_units) {
  return hpw == 32 && n_split == 1 && K > AT_TILE && K <= AT_IDS && n_units > AT_STREAM_WG &&
         n_units < ((int64_t)1 << 31);
}

// The attention grid (and the combine's, when the query is split).
int64_t attn_launch_items(int B, int H, int d_c, int K) {
  if (B <= 0) return 0;
  int s, ps;
  attn_plan(B, H, K, d_c, &s, &ps);
  const int hpw = attn_heads_per_wg(B, H, d_c);
  const int n_hg = (H + hpw - 1) / hpw;
  const bool spread = B < 8;
  const int64_t groups = spread ? ((int64_t)B * s + 7) / 8 : ((int64_t)B + 7) / 8 * s;
  const int64_t items = groups * 8 * n_hg * (hpw == 32 ? 512 : 256);
  const int64_t comb = s > 1 ? (spread ? (int64_t)B * H : ((int64_t)B + 7) / 8 * 8 * H) * 128 : 0;
  return items > comb ? items : comb;
}

int64_t swa_launch_items(int B, int H) { return ((int64_t)B + 7) / 8 * 8 * ((H + 15) / 16) * 256; }

// Workspace: partial outputs f32 [B, H, s, d_c], then (max, sum) f32 [B, H, s, 2].
size_t attn_workspace_bytes(int B, int H, int d_c, int K) {
  int s, ps;
  attn_plan(B, H, K, d_c, &s, &ps);
  if (s <= 1) return 0;
  return (size_t)B * H * s * ((size_t)d_c + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const uint16_t* q, CacheRef cache, const int32_t* idx, int K, int B, int H,
                              int d_c, int d_r, int64_t N_cap, int qps, float sm_scale, float* out, float* lse,
                              void* workspace, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  int s, ps;
  attn_plan(B, H, K, d_c, &s, &ps);
  const int hpw = attn_heads_per_wg(B, H, d_c);
  const int n_hg = (H + hpw - 1) / hpw;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = s > 1 ? ws_o + (size_t)B * H * s * d_c : nullptr;
  // slices of a small batch spread over the XCDs; else one query per XCD
  const int spread = B < 8 ? 1 : 0;
  const int64_t groups = spread ? ((int64_t)B * s + 7) / 8 : ((int64_t)B + 7) / 8 * s;
  const dim3 grid((unsigned)(groups * 8 * n_hg));
  const float sl = sm_scale * LOG2E;
#define CSA2_ATTN(KERNEL, THREADS, DCV, DRV)                                                          \
  hipLaunchKernelGGL((KERNEL<DCV, DRV>), grid, dim3(THREADS), 0, stream, q, cache, idx, K, B, H, N_cap, qps, sl, \
                     n_hg, s, ps, spread, out, lse, ws_o, ws_ml)
  const WinRef no_win{nullptr, 0, nullptr, nullptr, 0, nullptr, 0};
  const int64_t n_units = groups * 8 * n_hg;
  if (attn_streamed(hpw, s, K, n_units)) {
    const dim3 sgrid((unsigned)AT_STREAM_WG);
    if (d_r == 64)
      hipLaunchKernelGGL((sparse_attn_role_stream_kernel<64>), sgrid, dim3(512), 0, stream, q, cache, idx, K, B, H,
                         N_cap, qps, sl, n_hg, n_units, out, lse);
    else if (d_r == 0)
      hipLaunchKernelGGL((sparse_attn_role_stream_kernel<0>), sgrid, dim3(512), 0, stream, q, cache, idx, K, B, H,
                         N_cap, qps, sl, n_hg, n_units, out, lse);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (hpw == 32) {
    if (d_r == 64)
      hipLaunchKernelGGL((sparse_attn_role_kernel<64, false>), grid, dim3(512), 0, stream, q, cache, idx, K, B, H, N_cap,
                         qps, sl, n_hg, s, ps, spread, out, lse, ws_o, ws_ml, no_win);
    else if (d_r == 0)
      hipLaunchKernelGGL((sparse_attn_role_kernel<0, false>), grid, dim3(512), 0, stream, q, cache, idx, K, B, H, N_cap,
                         qps, sl, n_hg, s, ps, spread, out, lse, ws_o, ws_ml, no_win);
    else return hipErrorInvalidValue;
  } else if (d_c == 512 && d_r == 64) CSA2_ATTN(sparse_attn_kernel, 256, 512, 64);
  else if (d_c == 512 && d_r == 0) CSA2_ATTN(sparse_attn_kernel, 256, 512, 0);
  else if (d_c == 128 && d_r == 0) CSA2_ATTN(sparse_attn_kernel, 256, 128, 0);
  else if (d_c == 128 && d_r == 64) CSA2_ATTN(sparse_attn_kernel, 256, 128, 64);
  else return hipErrorInvalidValue;
#undef CSA2_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  const int64_t cblocks = spread ? (int64_t)B * H : ((int64_t)B + 7) / 8 * 8 * H;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)cblocks), dim3(128), 0, stream, ws_o, ws_ml, B, H,
                     s, d_c, spread, out, lse);
  return hipGetLastError();
}

// The sparse attention and the query's sliding window as one softmax over the
// union of their keys ([P4] CSA2 paragraph: the SWA branch beside the sparse
// one).  The 32-head kernel attends to the window rows as more tiles after the
// selected entries' (in the query's first slice); batches it does not serve
// run the sparse kernels and then the window kernel, which merges into their
// (out, lse).
bool sparse_swa_fused(int B, int H, int d_c) { return attn_heads_per_wg(B, H, d_c) == 32; }

size_t sparse_swa_workspace_bytes(int B, int H, int d_c, int K) {
  const size_t a = (attn_workspace_bytes(B, H, d_c, K) + 15) & ~(size_t)15;
  return sparse_swa_fused(B, H, d_c) ? a : a + (size_t)B * H * sizeof(float);
}

hipError_t launch_sparse_swa_attn(const uint16_t* q, CacheRef cache, const int32_t* idx, int K, int B, int H,
                                  int d_r, int64_t N_cap, WinRef win, float sm_scale, float* out, float* lse,
                                  void* workspace, hipStream_t stream) {
  constexpr int d_c = 512;
  if (B == 0) return hipSuccess;
  if (!sparse_swa_fused(B, H, d_c)) {
    const size_t a = (attn_workspace_bytes(B, H, d_c, K) + 15) & ~(size_t)15;
    float* l = lse ? lse : reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + a);
    hipError_t e = launch_sparse_attn(q, cache, idx, K, B, H, d_c, d_r, N_cap, 1, sm_scale, out, l, workspace, stream);
    if (e != hipSuccess) return e;
    return launch_swa_attn(q, win.codes, win.codes_stride, win.sigma, win.rope, win.rope_stride, win.n_win, B, H,
                           d_r, win.W_cap, sm_scale, out, l, out, lse, stream);
  }
  int s, ps;
  attn_plan(B, H, K, d_c, &s, &ps);
  const int n_hg = (H + 31) / 32;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = s > 1 ? ws_o + (size_t)B * H * s * d_c : nullptr;
  const int spread = B < 8 ? 1 : 0;
  const int64_t groups = spread ? ((int64_t)B * s + 7) / 8 : ((int64_t)B + 7) / 8 * s;
  const dim3 grid((unsigned)(groups * 8 * n_hg));
  const float sl = sm_scale * LOG2E;
  if (d_r == 64)
    hipLaunchKernelGGL((sparse_attn_role_kernel<64, true>), grid, dim3(512), 0, stream, q, cache, idx, K, B, H, N_cap,
                       1, sl, n_hg, s, ps, spread, out, lse, ws_o, ws_ml, win);
  else if (d_r == 0)
    hipLaunchKernelGGL((sparse_attn_role_kernel<0, true>), grid, dim3(512), 0, stream, q, cache, idx, K, B, H, N_cap,
                       1, sl, n_hg, s, ps, spread, out, lse, ws_o, ws_ml, win);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s == 1) return e;
  const int64_t cblocks = spread ? (int64_t)B * H : ((int64_t)B + 7) / 8 * 8 * H;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)cblocks), dim3(128), 0, stream, ws_o, ws_ml, B, H, s, d_c,
                     spread, out, lse);
  return hipGetLastError();
}

// Sliding-window branch: softmax attention of 16 query heads over the window
// rows of one sequence (the last tokens, one FP8 entry per token: E4M3 latent
// with a power-of-two scale per row, bf16 RoPE part), optionally merged with
// the sparse branch's (out, lse) into one softmax over the union of both key
// sets ([P4] CSA2 paragraph: the SWA branch beside the sparse one, SWA KV in
// FP8; [P1] section 效率组件四件, item 4).
//
// Same wave layout as the 16-head sparse kernel: wave w scores window rows
// 16w .. 16w + 15 of a 64-row tile, lane (n, g) holding channels 128 g .. + 127
// of row n as 8 words of 16 E4M3 values; each word is two score k-steps after
// an exact E4M3 -> fp16 conversion.  The latent products and the RoPE
// products go to separate accumulators so that the row scale multiplies only
// the latent part; the value products use the unscaled E4M3 values with P
// scaled by sigma_j / max sigma (a power of two, <= 1), and max sigma is
// applied once in the epilogue.  The window is at most 256 rows (4 tiles),
// loaded tile by tile.
struct SwaRegs {
  u32x4 cw[8];  // 128 E4M3 latent values of the lane's quarter row
  u32x4 rw[2];  // 16 RoPE channels (bf16)
};

template <int DR>
__global__ __launch_bounds__(256) void swa_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, int64_t codes_stride,
    const float* __restrict__ sigma, const uint16_t* __restrict__ rope, int64_t rope_stride,
    const int32_t* __restrict__ n_win, int B, int H, int W_cap, float sm_scale_log2e, int n_hg,
    const float* in_out, const float* __restrict__ in_lse, float* out, float* __restrict__ lse) {
  constexpr int DC = 512;
  constexpr int KSL = DC / 32;            // latent k-steps
  constexpr int KSR = DR / 32;            // RoPE k-steps
  constexpr int LDK = DC + 16;
  constexpr int NDB = DC / 4 / 16;        // PV d-blocks per wave (128 channels)
  __shared__ __attribute__((aligned(16))) _Float16 sK[AT_TILE][LDK];
  __shared__ __attribute__((aligned(16))) _Float16 sP[16][AT_TILE + 8];
  __shared__ float sMax[4][16], sSum[4][16], sAlpha[16], sFinM[16], sFinL[16];
  __shared__ float sSig[256];
  __shared__ float sRed[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // workgroup x runs on XCD x % 8: the head groups of one query, which read
  // the same window rows, share that XCD's L2
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int64_t b = (int64_t)(slot / n_hg) * 8 + xcd;
  if (b >= B) return;  // padding of the grid to whole groups of eight queries
  const int h0 = (slot % n_hg) * 16;
  const int nw = n_win ? min(max(n_win[b], 0), W_cap) : W_cap;
  const int n_tiles = (nw + AT_TILE - 1) / AT_TILE;

  // ---- row scales of the window and their maximum
  float sg = 0.f;
  if (tid < nw) sg = sigma[b * W_cap + tid];
  sSig[tid] = sg;
  float smax = sg;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) smax = fmaxf(smax, __shfl_xor(smax, o));
  if (lane == 0) sRed[wave] = smax;

  // ---- window rows: row 64 tile + 16 wave + n, channels 128 g .. + 127 as
  // 8 words of 16 E4M3 values, and 16 channels of the RoPE part per word
  auto gather = [&](SwaRegs& gr, int tile) {
    __builtin_amdgcn_sched_barrier(0);
    const int row = tile * AT_TILE + 16 * wave + n;
    const int64_t rr = b * W_cap + (row < nw ? row : 0);
    const uint8_t* crow = codes + rr * codes_stride + 128 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) gr.cw[i] = *reinterpret_cast<const u32x4*>(crow + 16 * i);
    if constexpr (DR > 0) {
      const uint8_t* rrow = reinterpret_cast<const uint8_t*>(rope) + rr * rope_stride + 32 * g;
#pragma unroll
      for (int t = 0; t < KSR; ++t) gr.rw[t] = *reinterpret_cast<const u32x4*>(rrow + 16 * t);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  SwaRegs ra0;
  if (n_tiles > 0) gather(ra0, 0);

  // ---- query heads h0 + n as B operands: latent k-step t -> channels
  // 128 g + 8 t .. + 7, RoPE k-step t -> channels d_c + 16 g + 8 t .. + 7
  u32x4 qraw[KSL + KSR];
  {
    // the 16 query rows, fetched once per workgroup as contiguous 16-byte
    // pieces into the value tile (free until the first tile), then read in
    // the operand layout (rows of heads >= H are zero)
    constexpr int QP = (DC + DR) / 8, QPITCH = DC + DR + 8, QN = (16 * QP + 255) / 256;
    static_assert(16 * QPITCH * 2 <= (int)sizeof(sK), "query staging fits the value tile");
    uint16_t* qs = reinterpret_cast<uint16_t*>(&sK[0][0]);
    u32x4 qv[QN];
#pragma unroll
    for (int k = 0; k < QN; ++k) {
      const int pc = tid + 256 * k, row = pc / QP, col = pc - row * QP;
      const bool ok = pc < 16 * QP && h0 + row < H;
      qv[k] = ok ? *reinterpret_cast<const u32x4*>(q + (b * H + h0 + row) * (DC + DR) + 8 * col)
                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < QN; ++k) {
      const int pc = tid + 256 * k, row = pc / QP, col = pc - row * QP;
      if (pc < 16 * QP) *reinterpret_cast<u32x4*>(qs + row * QPITCH + 8 * col) = qv[k];
    }
    __syncthreads();
    const uint16_t* qrow = qs + n * QPITCH;
#pragma unroll
    for (int t = 0; t < KSL + KSR; ++t) {
      const int off = t < KSL ? 128 * g + 8 * t : DC + 16 * g + 8 * (t - KSL);
      qraw[t] = *reinterpret_cast<const u32x4*>(qrow + off);
    }
  }
  f16x8 Bq[KSL];
  bf16x8 Br[KSR > 0 ? KSR : 1];
  float fscale;
  {
    uint32_t mx = 0;
#pragma unroll
    for (int t = 0; t < KSL + KSR; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(qraw[t][j] & 0x7FFFu, (qraw[t][j] >> 16) & 0x7FFFu));
    mx = max(mx, xor16(mx));
    mx = max(mx, xor32(mx));
    // 2^sh brings the largest |q| of the head into [2^14, 2^15), where fp16
    // keeps every bit of a bf16 value
    int ex = (int)((mx >> 7) & 0xFF) - 127;
    if (ex < -126) ex = -126;
    const int sh = mx == 0 ? 0 : min(120, max(-120, 14 - ex));
    const float up = __builtin_amdgcn_ldexpf(1.0f, sh);
    fscale = sm_scale_log2e * __builtin_amdgcn_ldexpf(1.0f, -sh);
#pragma unroll
    for (int t = 0; t < KSL; ++t) {
      f16x8 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = (_Float16)(bf16_bits_to_f32(qraw[t][j] & 0xFFFFu) * up);
        o[2 * j + 1] = (_Float16)(bf16_bits_to_f32(qraw[t][j] >> 16) * up);
      }
      Bq[t] = o;
    }
#pragma unroll
    for (int t = 0; t < KSR; ++t) {
      bf16x8 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = (__bf16)(bf16_bits_to_f32(qraw[KSL + t][j] & 0xFFFFu) * up);
        o[2 * j + 1] = (__bf16)(bf16_bits_to_f32(qraw[KSL + t][j] >> 16) * up);
      }
      Br[t] = o;
    }
  }
  __syncthreads();  // row scales and their per-wave maxima
  const float s_max = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
  const float inv_smax = s_max > 0.f ? 1.0f / s_max : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const SwaRegs& gr, int tile) {
    const u32x4* cw = gr.cw;
    const u32x4* rw = gr.rw;
    const int row = tile * AT_TILE + 16 * wave + n;
    const bool valid = row < nw;
    // ---- exact E4M3 -> fp16, latent scores, value tile
    const int e = 16 * wave + n;
    f32x4 cl = {0.f, 0.f, 0.f, 0.f}, cr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[i][2 * h], 1.0f, false);
        const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[i][2 * h], 1.0f, true);
        const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[i][2 * h + 1], 1.0f, false);
        const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cw[i][2 * h + 1], 1.0f, true);
        f16x8 a = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        if (!valid) a = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        const int t = 2 * i + h;  // channels 128 g + 8 t .. + 7
        *reinterpret_cast<f16x8*>(&sK[e][tile_col(e, 4 * g + (t >> 2), t & 3)]) = a;
        cl = mfma16x16x32_f16(a, Bq[t], cl);
      }
    }
#pragma unroll
    for (int t = 0; t < KSR; ++t) cr = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, rw[t]), Br[t], cr);
    // cl[i], cr[i]: row 16 wave + 4 g + i, head n
    const uint64_t vb = __ballot(g == 0 && valid);
    float s2[4], rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sgi = sSig[tile * AT_TILE + 16 * wave + 4 * g + i];
      rs[i] = sgi * inv_smax;
      s2[i] = ((vb >> (4 * g + i)) & 1u) ? (cl[i] * sgi + cr[i]) * fscale : -INFINITY;
    }
    // ---- online softmax (base 2), maxima exchanged through LDS
    float mt = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mt = fmaxf(mt, xor16f(mt));
    mt = fmaxf(mt, xor32f(mt));
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
    ps += xor16f(ps);
    ps += xor32f(ps);
    if (g == 0) sSum[wave][n] = ps;
    if (wave == 0 && g == 0) sAlpha[n] = alpha;
    *reinterpret_cast<f16x4*>(&sP[n][16 * wave + 4 * g]) =
        f16x4{(_Float16)(p[0] * rs[0]), (_Float16)(p[1] * rs[1]), (_Float16)(p[2] * rs[2]), (_Float16)(p[3] * rs[3])};
    __syncthreads();
    l_run = l_run * alpha + (sSum[0][n] + sSum[1][n] + sSum[2][n] + sSum[3][n]);
    m_run = m_new;
    // ---- O = alpha O + P' . V (V: the unscaled E4M3 values of the tile)
    {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = sAlpha[4 * g + i];
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[d][i] *= al[i];
      const int tr_r = n >> 2, tr_c = n & 3;
#pragma unroll
      for (int u = 0; u < AT_TILE / 32; ++u) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&sP[n][32 * u + 8 * g]);
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
          const int ch = 32 * pv_chunk<DC>(wave, d >> 1) + 16 * (d & 1) + 4 * tr_c;
          const int r0 = 32 * u + 8 * g + tr_r, r1 = r0 + 4;
          const f16x4 v0 = tr16_read(&sK[r0][tile_col(r0, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
          const f16x4 v1 = tr16_read(&sK[r1][tile_col(r1, ch >> 5, (ch >> 3) & 3) + (ch & 7)]);
          const f16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[d] = mfma16x16x32_f16(a, bv, acc[d]);
        }
      }
    }
    __syncthreads();  // the tile buffers are rewritten by the next tile
  };
  // two register sets: the loads of tile t + 1 are in flight while tile t is
  // processed (past the last tile they read row 0 again, unconditionally)
  if (n_tiles > 0) {
    SwaRegs& ra = ra0;
    SwaRegs rb;
    int t = 0;
    gather(rb, 1);
    for (; t + 2 <= n_tiles; t += 2) {
      process(ra, t);
      gather(ra, t + 2);
      process(rb, t + 1);
      gather(rb, t + 3);
    }
    if (t < n_tiles) process(ra, t);
    __builtin_amdgcn_s_waitcnt(0);  // no load may land after the wave ends
  }

  // ---- epilogue: lane (channel n of each d-block, k-group g) holds heads
  // h0 + 4 g + i; window result o_w = acc * max sigma / l, merged with the
  // sparse branch when given: weights e^(lse - max lse) of the two branches
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
    const float lw = l > 0.f ? (m + __log2f(l)) * LN2 : -INFINITY;  // window lse (natural log)
    const float ow = l > 0.f ? s_max / l : 0.f;                        // scale of acc -> o_w
    float wa = 0.f, wb = 1.f, den = 1.f, lo = lw;
    if (in_lse) {
      const float ls = in_lse[b * H + h];
      const float mm = fmaxf(ls, lw);
      const float ref = mm == -INFINITY ? 0.f : mm;
      wa = ls == -INFINITY ? 0.f : __expf(ls - ref);
      wb = lw == -INFINITY ? 0.f : __expf(lw - ref);
      den = wa + wb;
      lo = den > 0.f ? ref + __logf(den) : -INFINITY;
      den = den > 0.f ? den : 1.f;
    }
    const int64_t orow = (b * H + h) * DC;
    float mi[NDB];  // the sparse branch's values, all read before any write (out may be in_out)
#pragma unroll
    for (int d = 0; d < NDB; ++d)
      mi[d] = in_lse ? in_out[orow + 32 * pv_chunk<DC>(wave, d >> 1) + 16 * (d & 1) + n] : 0.f;
    const float inv_den = 1.0f / den;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int64_t c = orow + 32 * pv_chunk<DC>(wave, d >> 1) + 16 * (d & 1) + n;
      const float v = acc[d][i] * ow;
      __builtin_nontemporal_store(in_lse ? (wa * mi[d] + wb * v) * inv_den : v, &out[c]);
    }
    if (lse && wave == 0 && n == 0) lse[b * H + h] = lo;
  }
}

hipError_t launch_swa_attn(const uint16_t* q, const uint8_t* codes, int64_t codes_stride, const float* sigma,
                           const uint16_t* rope, int64_t rope_stride, const int32_t* n_win, int B, int H, int d_r,
                           int W_cap, float sm_scale, const float* in_out, const float* in_lse, float* out,
                           float* lse, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int n_hg = (H + 15) / 16;
  const dim3 grid((unsigned)(((int64_t)B + 7) / 8 * 8 * n_hg));
  const float sl = sm_scale * LOG2E;
  if (d_r == 64)
    hipLaunchKernelGGL(swa_attn_kernel<64>, grid, dim3(256), 0, stream, q, codes, codes_stride, sigma, rope,
                       rope_stride, n_win, B, H, W_cap, sl, n_hg, in_out, in_lse, out, lse);
  else if (d_r == 0)
    hipLaunchKernelGGL(swa_attn_kernel<0>, grid, dim3(256), 0, stream, q, codes, codes_stride, sigma, rope,
                       rope_stride, n_win, B, H, W_cap, sl, n_hg, in_out, in_lse, out, lse);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace csa2
