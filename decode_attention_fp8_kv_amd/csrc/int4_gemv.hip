// INT4 weight-only decode GEMV for gfx950: y[m][n] = sum_k x[m][k] * q[n][k]
// * s[n][k / 128], x and y BF16, q signed 4-bit, s BF16, M <= 64.
//
// Decode streams every weight once per step, so with 4-bit weights the step
// moves half the bytes of FP8 weights (source pages: "ترفندهای کلادفلر برای
// جا دادن مدل‌های غول‌پیکر تو GPU", the second technique; "更小、更快、更安全：
// 大规模运行Kimi和GLM", section "压缩模型权重").  The kernel is bound by HBM:
// 0.5 byte per weight + 2 bytes of scale per 128 weights.
//
// Storage (the layout is part of the interface): row n is K/8 32-bit words;
// word j holds k = 8j..8j+7 with nibble i at bits 4i..4i+3 holding
// k = 8j + 2i (i < 4) or 8j + 2(i-4) + 1 (i >= 4).  With that order one
// shift and one and-or per pair turn a word into four bf16 pairs in natural
// k order, which is what an MFMA operand register holds.
//
// Dequantization without arithmetic: u = q + 8 (flip each nibble's top bit)
// placed in the top four mantissa bits of 1.0 gives the bf16 value
// 1 + u/16 = 1.5 + q/16 exactly.  The MFMA contracts x with those values,
// and four more MFMAs with the constant -1.5 on the same x remove the
// offset: sum_k x (1.5 + q/16) - 1.5 sum_k x = (sum_k x q) / 16.  The
// group's scale (times 16) is applied to the fp32 group sum, once per group.
//
// Work: a workgroup owns 16*NS rows and all of K; its four waves split K
// into equal runs of 128-weight groups and meet in LDS at the end (fixed
// order: the result does not depend on timing).  Per group a wave issues one
// 16-byte weight load per lane and subtile -- 16 rows x 64 bytes -- one group
// ahead of its use.  MFMA v_mfma_f32_16x16x32_bf16: A = 16 activation rows x
// 32 k, B = 32 k x 16 weight rows; lane l supplies k = 8*(l/16)..+7 of
// activation row / weight row l%16 and receives outputs for activation rows
// 4*(l/16)..+3 of weight row l%16.  Rows past M read as zero (M = 1 uses one
// row of 16; the matrix unit has the throughput to spare).
#include "common.hpp"
#include "internal.hpp"

namespace fp8kv {
namespace {

constexpr int kI4Waves = 4;
constexpr int kI4Threads = 64 * kI4Waves;

// One word of 8 weights -> 8 bf16 values 1 + (q + 8)/16 in natural k order.
__device__ __forceinline__ bf16x8_t i4x8_to_offset_bf16(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;  // two's complement -> offset binary
  u32x4_t r;
  r[0] = ((u << 3) & 0x00780078u) | 0x3F803F80u;  // nibbles 0, 4 -> k0, k1
  r[1] = ((u >> 1) & 0x00780078u) | 0x3F803F80u;  // nibbles 1, 5 -> k2, k3
  r[2] = ((u >> 5) & 0x00780078u) | 0x3F803F80u;  // nibbles 2, 6 -> k4, k5
  r[3] = ((u >> 9) & 0x00780078u) | 0x3F803F80u;  // nibbles 3, 7 -> k6, k7
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int MB, int NS>
__global__ __launch_bounds__(kI4Threads) void int4_gemv_kernel(Int4GemvParams p) {
  __shared__ f32x4_t red[kI4Waves - 1][NS * MB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int groups = p.k >> 7;
  const int g0 = (int)((int64_t)groups * wave / kI4Waves);
  const int g1 = (int)((int64_t)groups * (wave + 1) / kI4Waves);
  const int64_t words_per_row = p.k >> 3;

  // Rows past N and activation rows past M read a valid row instead (row 0);
  // their outputs are never stored, so no load needs a predicate.
  const u32x4_t* wrow[NS];
  const uint16_t* srow[NS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    const int64_t n = (int64_t)blockIdx.x * (16 * NS) + 16 * ns + r;
    const int64_t nn = n < p.n ? n : 0;
    wrow[ns] = reinterpret_cast<const u32x4_t*>(p.w + nn * words_per_row) + c;  // + 4 per group
    srow[ns] = p.s + nn * groups;
  }
  const bf16x8_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * mb + r;
    xrow[mb] = reinterpret_cast<const bf16x8_t*>(p.x + (int64_t)(m < p.m ? m : 0) * p.k) + 4 * c;  // + 16 per group
  }

  const bf16x8_t neg15 = __builtin_bit_cast(bf16x8_t, u32x4_t{0xBFC0BFC0u, 0xBFC0BFC0u, 0xBFC0BFC0u, 0xBFC0BFC0u});
  f32x4_t acc[NS][MB];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[ns][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Weights and scales are loaded one group ahead.  Each iteration issues
  // this group's activation loads (L2-resident) before the next group's
  // weight loads: memory loads complete in issue order, so waiting for the
  // activations leaves the weight stream in flight.
  u32x4_t wcur[NS];
  uint32_t scur[NS];
  if (g0 < g1) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      wcur[ns] = wrow[ns][4 * (int64_t)g0];
      scur[ns] = srow[ns][g0];
    }
  }
  for (int g = g0; g < g1; ++g) {
    bf16x8_t a[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) a[mb][i] = xrow[mb][16 * (int64_t)g + i];
    const int gn = g + 1 < g1 ? g + 1 : g;  // the last iteration reloads its own group
    u32x4_t wnext[NS];
    uint32_t snext[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      wnext[ns] = wrow[ns][4 * (int64_t)gn];
      snext[ns] = srow[ns][gn];
    }
    bf16x8_t b[NS][4];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int i = 0; i < 4; ++i) b[ns][i] = i4x8_to_offset_bf16(wcur[ns][i]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][i], neg15, corr, 0, 0, 0);
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        f32x4_t t = corr;
#pragma unroll
        for (int i = 0; i < 4; ++i) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][i], b[ns][i], t, 0, 0, 0);
        const float sc = 16.f * bf16_bits_to_f32(scur[ns]);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[ns][mb][v] += sc * t[v];
      }
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      wcur[ns] = wnext[ns];
      scur[ns] = snext[ns];
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
    const int64_t n = (int64_t)blockIdx.x * (16 * NS) + 16 * ns + r;
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

template <int MB>
hipError_t launch_mb(const Int4GemvParams& p, hipStream_t stream) {
  constexpr int NS = 2;
  const int64_t blocks = (p.n + 16 * NS - 1) / (16 * NS);
  hipLaunchKernelGGL((int4_gemv_kernel<MB, NS>), dim3((unsigned)blocks), dim3(kI4Threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_int4_gemv(const Int4GemvParams& p, hipStream_t stream) {
  switch ((p.m + 15) / 16) {
    case 1: return launch_mb<1>(p, stream);
    case 2: return launch_mb<2>(p, stream);
    case 3: return launch_mb<3>(p, stream);
    case 4: return launch_mb<4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8kv
