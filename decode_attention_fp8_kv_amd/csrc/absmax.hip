// Per-tensor scale for the prefill -> decode hand-off: amax over the finite
// elements of a BF16 tensor, and scale = amax / 448 (1 if amax is 0).
//
// Prefill keeps K/V in BF16 and decode reads an FP8 cache (source pages:
// "Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa
// KV cache"; "更小、更快、更安全：大规模运行Kimi和GLM", section "量化 KV 缓存"), so
// a prefill's K/V are converted once on hand-off; the scale that maps its
// largest finite magnitude onto e4m3's largest value 448 is computed on the
// device, and kv_quant_append_dscale reads it from there, so the whole
// hand-off needs no host round trip.  Two kernels: a grid-stride reduction
// (four 16-byte loads in flight per thread, wave and block maxima, each
// block's maximum stored to its own word of a work buffer), then one block
// that reduces those words and writes amax and scale.  Per-block words
// instead of one atomic max: device-scope atomics on a single address are
// serviced one at a time, which with thousands of blocks costs more than
// the reads themselves.
#include "common.hpp"
#include "internal.hpp"

namespace fp8kv {
namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxMaxBlocks = kAmaxWorkFloats;  // one work word per block

__device__ __forceinline__ float finite_abs_max(float m, uint32_t bf16_bits) {
  const float a = __builtin_fabsf(__builtin_bit_cast(float, bf16_bits << 16));
  return a <= 3.40282347e38f ? __builtin_fmaxf(m, a) : m;  // NaN and infinity fail the test
}

// Block y of the grid reduces tensor y (x0 or x1) into its own
// kAmaxWorkFloats work words.
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const uint16_t* x0, const uint16_t* x1, int64_t n,
                                                            float* work) {
  __shared__ float wmax[kAmaxThreads / 64];
  const uint16_t* x = blockIdx.y == 0 ? x0 : x1;
  work += (int64_t)blockIdx.y * kAmaxWorkFloats;
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  const int64_t n8 = n >> 3;  // 16-byte words
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    u32x4_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const u32x4_t*>(x + 8 * (i + u * stride));
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = finite_abs_max(m, w[u][j] & 0xFFFFu);
        m = finite_abs_max(m, w[u][j] >> 16);
      }
  }
  for (; i < n8; i += stride) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(x + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = finite_abs_max(m, w[j] & 0xFFFFu);
      m = finite_abs_max(m, w[j] >> 16);
    }
  }
  for (int64_t t = 8 * n8 + (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; t < n; t += stride)
    m = finite_abs_max(m, x[t]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int k = 1; k < kAmaxThreads / 64; ++k) b = __builtin_fmaxf(b, wmax[k]);
    work[blockIdx.x] = b;
  }
}

// Block t finishes tensor t: out[2t] = amax, out[2t + 1] = scale.
__global__ __launch_bounds__(kAmaxThreads) void amax_finish_kernel(const float* work, int nb, float* out) {
  __shared__ float wmax[kAmaxThreads / 64];
  work += (int64_t)blockIdx.x * kAmaxWorkFloats;
  out += 2 * blockIdx.x;
  float m = 0.f;
  for (int i = threadIdx.x; i < nb; i += kAmaxThreads) m = __builtin_fmaxf(m, work[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = wmax[0];
#pragma unroll
    for (int k = 1; k < kAmaxThreads / 64; ++k) a = __builtin_fmaxf(a, wmax[k]);
    out[0] = a;
    out[1] = a > 0.f ? a / 448.0f : 1.0f;
  }
}

}  // namespace

hipError_t launch_absmax_scale(const uint16_t* x0, const uint16_t* x1, int tensors, int64_t n, float* out,
                               float* work, hipStream_t stream) {
  const int64_t blocks =
      std::max<int64_t>(1, std::min<int64_t>(kAmaxMaxBlocks, (n / 8 + 4 * kAmaxThreads - 1) / (4 * kAmaxThreads)));
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks, (unsigned)tensors), dim3(kAmaxThreads), 0, stream, x0, x1, n,
                     work);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_finish_kernel, dim3((unsigned)tensors), dim3(kAmaxThreads), 0, stream, work, (int)blocks,
                     out);
  return hipGetLastError();
}

}  // namespace fp8kv
