// INT4 weight-only decode GEMV for gfx950: y[m][n] = sum_k x[m][k] * q[n][k]
// * s[n][k / 128], x and y BF16, q signed 4-bit, s BF16, M <= 64.
//
// Decode streams every weight once per step, so with 4-bit weights the step
// moves half the bytes of FP8 weights (source pages: "ترفندهای کلادفلر برای
// جا دادن مدل‌های غول‌پیکر تو GPU", the second technique; "更小、更快、更安全：
// 大规模运行Kimi和GLM", section "压缩模型权重").  The kernel is bound by HBM:
// 0.5 byte per weight + 2 bytes of scale per 128 weights.
//
// Storage (the layout is part of the interface; int4_pack_weights builds it
// from the common row layout).  Rows are cut into tiles of 16 rows x 128
// weights: tile t, group g is 1 KiB of 32-bit words at ((t*G + g)*16 + r)*16
// + j (G = K/128, row r = n - 16t, word j holds k = 128g + 8j .. +7) and its
// 16 scales are 32 contiguous bytes at (t*G + g)*16 + r.  A wave's load of
// one tile-group is one contiguous KiB and consecutive groups are adjacent,
// so every wave streams sequential memory: with rows 4 KiB apart instead,
// each DRAM page was reopened for every 64 bytes and the stream ran at half
// the rate.  Within a word, nibble i holds k = 8j + 2i (i < 4) or
// 8j + 2(i-4) + 1 (i >= 4): a shift and one three-input bit operation per
// pair then turn a word into four bf16 pairs in natural k order, which is
// what an MFMA operand register holds.
//
// Dequantization without arithmetic: u = q + 8 (each nibble's top bit
// flipped) placed in the top four mantissa bits of 1.0 gives the bf16 value
// 1 + u/16 = 1.5 + q/16 exactly.  The MFMA contracts x with those values,
// and four more MFMAs with the constant -1.5 on the same x remove the
// offset: sum_k x (1.5 + q/16) - 1.5 sum_k x = (sum_k x q) / 16.  The
// group's scale (times 16) is applied to the fp32 group sum, once per group.
//
// Work: a workgroup owns NS tiles (16*NS rows) and all of K; its four waves
// split K into equal runs of groups and meet in LDS at the end (fixed order:
// the result does not depend on timing).  Each wave keeps a ring of D
// stages, one group's codes, scales (and activations) per stage, loaded
// D - 1 groups ahead of their use.  MFMA v_mfma_f32_16x16x32_bf16: A = 16
// activation rows x 32 k, B = 32 k x 16 weight rows; lane l supplies
// k = 8*(l/16)..+7 of activation row / weight row l%16 and receives outputs
// for activation rows 4*(l/16)..+3 of weight row l%16.  Activation rows past
// M read row 0 and are discarded (M = 1 uses one row of 16; the matrix unit
// has the throughput to spare).
#include "common.hpp"
#include "internal.hpp"

namespace fp8kv {
namespace {

constexpr int kI4Waves = 4;
constexpr int kI4Threads = 64 * kI4Waves;
constexpr int kI4LdsX = 32 * 1024;  // activations staged in LDS up to this many bytes
constexpr int kI4RingLds = 4;       // ring depth when the activations sit in LDS (<= 128 VGPRs)
// Activations read from registers: per 128-weight group a wave loads 16 * MB
// activation rows (4 KiB per 16 rows) against NS KiB of codes, from L2, with
// a two-stage ring (deeper rings measured slower).  NS is chosen per call
// (pick_tiles): these workgroups run about one per CU, so a call takes
// ceil(workgroups / CUs) rounds of NS tiles each; the NS with the fewest
// tile-times wins, the larger on a tie (each activation block then feeds
// more weight rows).  At 28,672 rows (1,792 tiles), 7 tiles per workgroup
// make 256 workgroups and one round where 4 made 448 and two: M = 16 went
// from 36 to 28 us and M = 64 from 84 to 60 us.  The CU count is the
// device's own (device_compute_units).

// One word of 8 weights -> 8 bf16 values 1 + (q + 8)/16 in natural k order.
// Each pair: shift the two nibbles to bits 3..6 / 19..22, keep them, and
// xor with 0x3FC0: that sets the exponent bits of 1.0 (0x3F80) and flips
// the nibble's top bit, turning two's complement q into offset binary
// q + 8.  Shift plus one three-input bit operation per pair on gfx950.
__device__ __forceinline__ bf16x8_t i4x8_to_offset_bf16(uint32_t w) {
  u32x4_t r;
  r[0] = ((w << 3) & 0x00780078u) ^ 0x3FC03FC0u;  // nibbles 0, 4 -> k0, k1
  r[1] = ((w >> 1) & 0x00780078u) ^ 0x3FC03FC0u;  // nibbles 1, 5 -> k2, k3
  r[2] = ((w >> 5) & 0x00780078u) ^ 0x3FC03FC0u;  // nibbles 2, 6 -> k4, k5
  r[3] = ((w >> 9) & 0x00780078u) ^ 0x3FC03FC0u;  // nibbles 3, 7 -> k6, k7
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int MB, int NS, bool XL>
struct Stage {
  u32x4_t w[NS];                  // 32 codes of weight row 16*ns + lane%16, k = 32*(lane/16)..+31 of the group
  uint32_t s[NS];                 // that row's scale for the group (bf16 bits)
  bf16x8_t a[XL ? 1 : MB][4];     // activations of row 16*mb + lane%16, k = 32*(lane/16) + 8*i..+7 (unused
                                  // when the activations sit in LDS)
};

template <int MB, int NS, bool XL>
__device__ __forceinline__ void issue_stage(Stage<MB, NS, XL>& S, const u32x4_t* const (&wrow)[NS],
                                            const uint16_t* const (&srow)[NS], const bf16x8_t* const (&xrow)[MB],
                                            int g) {
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    // non-temporal: the codes are read once; keeping them out of the
    // caches leaves room for the activations, which every workgroup rereads
    S.w[ns] = __builtin_nontemporal_load(&wrow[ns][64 * (int64_t)g]);
    S.s[ns] = __builtin_nontemporal_load(&srow[ns][16 * (int64_t)g]);
  }
  if constexpr (!XL) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) S.a[mb][i] = xrow[mb][16 * (int64_t)g + i];
  }
}

template <int MB, int NS, bool XL>
__device__ __forceinline__ void compute_stage(const Stage<MB, NS, XL>& S, f32x4_t (&acc)[NS][MB], bf16x8_t neg15,
                                              const bf16x8_t* xl, int g) {
  if constexpr (MB > 1) {
    // Tiles outside, activation blocks inside: one tile's unpacked codes are
    // live at a time instead of all NS (at MB = 4, NS = 7 this keeps the
    // kernel within its registers; 58 us vs 60.5 us at 64 x 28,672 x 8,192).
    // Every output sees the same operations in the same order either way.
    f32x4_t corr[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      corr[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        corr[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.a[mb][i], neg15, corr[mb], 0, 0, 0);
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      bf16x8_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = i4x8_to_offset_bf16(S.w[ns][i]);
      const float sc = 16.f * bf16_bits_to_f32(S.s[ns]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t t = corr[mb];
#pragma unroll
        for (int i = 0; i < 4; ++i) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(S.a[mb][i], b[i], t, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[ns][mb][v] += sc * t[v];
      }
    }
    return;
  }
  bf16x8_t b[NS][4];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns)
#pragma unroll
    for (int i = 0; i < 4; ++i) b[ns][i] = i4x8_to_offset_bf16(S.w[ns][i]);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    bf16x8_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XL)
        a[i] = xl[16 * g + i];
      else
        a[i] = S.a[mb][i];
    }
    f32x4_t corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], neg15, corr, 0, 0, 0);
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      f32x4_t t = corr;
#pragma unroll
      for (int i = 0; i < 4; ++i) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[ns][i], t, 0, 0, 0);
      const float sc = 16.f * bf16_bits_to_f32(S.s[ns]);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[ns][mb][v] += sc * t[v];
    }
  }
}

template <int MB, int NS, int D, bool XL>
__global__ __launch_bounds__(kI4Threads) void int4_gemv_kernel(Int4GemvParams p) {
  __shared__ f32x4_t red[kI4Waves - 1][NS * MB][64];
  __shared__ bf16x8_t xs[XL ? kI4LdsX / 16 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int groups = p.k >> 7;
  const int g0 = (int)((int64_t)groups * wave / kI4Waves);
  const int g1 = (int)((int64_t)groups * (wave + 1) / kI4Waves);

  // Tiles past the last one and activation rows past M read a valid one
  // instead (tile 0, row 0); their outputs are never stored, so no load needs
  // a predicate.  Rows past N inside the last tile are the caller's padding.
  const int64_t tiles = (p.n + 15) / 16;
  const u32x4_t* wrow[NS];
  const uint16_t* srow[NS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    const int64_t t = (int64_t)blockIdx.x * NS + ns;
    const int64_t tt = t < tiles ? t : 0;
    wrow[ns] = reinterpret_cast<const u32x4_t*>(p.w + tt * groups * 256) + 4 * r + c;  // + 64 per group
    srow[ns] = p.s + tt * groups * 16 + r;                                            // + 16 per group
  }
  const bf16x8_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * mb + r;
    xrow[mb] = reinterpret_cast<const bf16x8_t*>(p.x + (int64_t)(m < p.m ? m : 0) * p.k) + 4 * c;  // + 16 per group
  }

  // Small activations (m * k * 2 <= kI4LdsX bytes, so MB == 1) are copied to
  // LDS once per workgroup: the ring then carries only weights and scales
  // and can be deeper for the same registers.
  const bf16x8_t* xl = nullptr;
  if constexpr (XL) {
    const int64_t n16 = (int64_t)p.m * p.k / 8;
    const bf16x8_t* xg = reinterpret_cast<const bf16x8_t*>(p.x);
    for (int64_t t = threadIdx.x; t < n16; t += kI4Threads) xs[t] = xg[t];
    __syncthreads();
    xl = xs + (int64_t)(r < p.m ? r : 0) * (p.k / 8) + 4 * c;  // + 16 per group
  }

  const bf16x8_t neg15 = __builtin_bit_cast(bf16x8_t, u32x4_t{0xBFC0BFC0u, 0xBFC0BFC0u, 0xBFC0BFC0u, 0xBFC0BFC0u});
  f32x4_t acc[NS][MB];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[ns][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A ring of D stages, each holding one group's weights, scales and
  // activations, loaded together: D - 1 groups are in flight while one is
  // computed.  Loads complete in issue order, so the stage consumed is always
  // the oldest one outstanding and waiting for it leaves the others in
  // flight.
  // The loads are issued without branches (past the end they repeat the
  // last group, which is in cache), so every stage is issued exactly D - 1
  // stages before its use on every path.
  if (g0 < g1) {
    Stage<MB, NS, XL> st[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      issue_stage(st[j], wrow, srow, xrow, min(g0 + j, g1 - 1));
      __builtin_amdgcn_sched_barrier(0);  // keep the stages' loads in ring order
    }
    for (int g = g0; g < g1; g += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (g + j < g1) compute_stage(st[j], acc, neg15, xl, g + j);
        issue_stage(st[j], wrow, srow, xrow, min(g + j + D, g1 - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // split-K: waves 1..3 hand their sums to wave 0, which adds them in order
  if (wave > 0) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red[wave - 1][ns * MB + mb][lane] = acc[ns][mb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    const int64_t n = ((int64_t)blockIdx.x * NS + ns) * 16 + r;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t s = acc[ns][mb];
#pragma unroll
      for (int w = 0; w < kI4Waves - 1; ++w) {
        const f32x4_t o = red[w][ns * MB + mb][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) s[v] += o[v];
      }
      if (n < p.n) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 16 * mb + 4 * c + v;
          if (m < p.m) p.y[(int64_t)m * p.n + n] = (uint16_t)f32_to_bf16_bits(s[v]);
        }
      }
    }
  }
}

template <int MB, int NS, int D, bool XL>
hipError_t launch_cfg(const Int4GemvParams& p, hipStream_t stream) {
  const int64_t blocks = ((p.n + 15) / 16 + NS - 1) / NS;
  hipLaunchKernelGGL((int4_gemv_kernel<MB, NS, D, XL>), dim3((unsigned)blocks), dim3(kI4Threads), 0, stream, p);
  return hipGetLastError();
}

// Row layout -> tile layout, one thread per tile word: gathers the word's
// even-k nibbles into its low half-word and the odd-k ones into the high
// half-word; padding rows get code 0 and scale 0.
__global__ __launch_bounds__(256) void int4_pack_kernel(const uint32_t* wr, const uint16_t* sr, uint32_t* wt,
                                                        uint16_t* st, int32_t n, int32_t k) {
  const int64_t groups = k >> 7;
  const int64_t total = (int64_t)((n + 15) / 16) * groups * 256;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int j = (int)(idx & 15), r = (int)((idx >> 4) & 15);
  const int64_t tg = idx >> 8;  // t * groups + g
  const int64_t t = tg / groups, g = tg - t * groups;
  const int64_t row = 16 * t + r;
  const uint32_t in = row < n ? wr[row * (k >> 3) + 16 * g + j] : 0u;
  uint32_t e = in & 0x0F0F0F0Fu, o = (in >> 4) & 0x0F0F0F0Fu;  // k = 8j + {0,2,4,6} / {1,3,5,7}, one per byte
  e = (e | (e >> 4)) & 0x00FF00FFu;
  o = (o | (o >> 4)) & 0x00FF00FFu;
  e = (e | (e >> 8)) & 0x0000FFFFu;
  o = (o | (o >> 8)) & 0x0000FFFFu;
  wt[idx] = e | (o << 16);
  if (j == 0) st[tg * 16 + r] = row < n ? sr[row * groups + g] : (uint16_t)0;
}

}  // namespace

hipError_t launch_int4_pack(const uint32_t* w_rows, const uint16_t* s_rows, uint32_t* w_tiles, uint16_t* s_tiles,
                            int32_t n, int32_t k, hipStream_t stream) {
  const int64_t total = (int64_t)((n + 15) / 16) * (k >> 7) * 256;
  if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;  // more blocks than a grid holds
  hipLaunchKernelGGL(int4_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, w_rows, s_rows,
                     w_tiles, s_tiles, n, k);
  return hipGetLastError();
}

namespace {

// Tiles per workgroup on the register path (see the register-path comment above).
int pick_tiles(int64_t tiles) {
  const int64_t cus = device_compute_units();
  int best = 7;
  int64_t best_cost = INT64_MAX;
  for (const int ns : {7, 4, 2}) {
    const int64_t rounds = ((tiles + ns - 1) / ns + cus - 1) / cus;
    if (rounds * ns < best_cost) {
      best_cost = rounds * ns;
      best = ns;
    }
  }
  return best;
}

template <int MB>
hipError_t launch_reg(const Int4GemvParams& p, hipStream_t stream) {
  switch (pick_tiles((p.n + 15) / 16)) {
    case 7: return launch_cfg<MB, 7, 2, false>(p, stream);
    case 4: return launch_cfg<MB, 4, 2, false>(p, stream);
    default: return launch_cfg<MB, 2, 2, false>(p, stream);
  }
}

}  // namespace

hipError_t launch_int4_gemv(const Int4GemvParams& p, hipStream_t stream) {
  if (p.m <= 16 && (int64_t)p.m * p.k * 2 <= kI4LdsX) {
    // Activations in LDS.  When 7 tiles per workgroup take the fewest
    // tile-times, one workgroup per CU with a two-stage ring (at 28,672
    // rows: 24.6 us vs 25.9 us with 2 tiles per workgroup, four workgroups
    // per CU and a four-stage ring).
    if (pick_tiles((p.n + 15) / 16) == 7) return launch_cfg<1, 7, 2, true>(p, stream);
    return launch_cfg<1, 2, kI4RingLds, true>(p, stream);
  }
  switch ((p.m + 15) / 16) {
    case 1: return launch_reg<1>(p, stream);
    case 2: return launch_reg<2>(p, stream);
    case 3: return launch_reg<3>(p, stream);
    case 4: return launch_reg<4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8kv
