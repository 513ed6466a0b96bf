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
// (four 16-byte loads in flight per thread, wave and block maxima, one
// relaxed atomic max of the block's result into a scratch word -- for
// non-negative floats the bit order is the value order), then one thread
// that writes amax and scale and zeroes the scratch word for the next call
// (the kernel boundary orders it after every block's atomic).
#include "common.hpp"
#include "internal.hpp"

namespace fp8kv {
namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxMaxBlocks = 2048;

__device__ __forceinline__ float finite_abs_max(float m, uint32_t bf16_bits) {
  const float a = __builtin_fabsf(__builtin_bit_cast(float, bf16_bits << 16));
  return a <= 3.40282347e38f ? __builtin_fmaxf(m, a) : m;  // NaN and infinity fail the test
}

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const uint16_t* x, int64_t n, uint32_t* out) {
  __shared__ float wmax[kAmaxThreads / 64];
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
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = xor_max(m, off);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int k = 1; k < kAmaxThreads / 64; ++k) b = __builtin_fmaxf(b, wmax[k]);
    // out: [0] amax, [1] scale, [2] running max (bits), [3] unused
    __hip_atomic_fetch_max(out + 2, __builtin_bit_cast(uint32_t, b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ __launch_bounds__(1) void amax_finish_kernel(uint32_t* out) {
  const uint32_t bits = out[2];
  const float a = __builtin_bit_cast(float, bits);
  out[0] = bits;
  out[1] = __builtin_bit_cast(uint32_t, a > 0.f ? a / 448.0f : 1.0f);
  out[2] = 0u;
}

}  // namespace

hipError_t launch_absmax_scale(const uint16_t* x, int64_t n, float* out, hipStream_t stream) {
  const int64_t blocks =
      std::max<int64_t>(1, std::min<int64_t>(kAmaxMaxBlocks, (n / 8 + 4 * kAmaxThreads - 1) / (4 * kAmaxThreads)));
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream, x, n,
                     reinterpret_cast<uint32_t*>(out));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_finish_kernel, dim3(1), dim3(1), 0, stream, reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace fp8kv
