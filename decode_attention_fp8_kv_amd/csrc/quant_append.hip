// kv_quant_append kernel: BF16 K/V rows -> e4m3 (or BF16) bytes scattered
// into cache pages through the page table.
//
// The cache holds e4m3 values with one fp32 scale per tensor (source pages:
// "Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa
// KV cache"; "更小、更快、更安全：大规模运行Kimi和GLM", section "量化 KV 缓存").
// Each element x becomes e4m3(fp32(x) / scale): an IEEE fp32 division, then
// round-to-nearest-even with saturation at +-448.
//
// One thread moves 8 consecutive elements of one (row, KV head) for both K
// and V: a 16-byte BF16 load each, 8-byte (FP8) or 16-byte (BF16) stores.
// Consecutive threads cover consecutive elements of a row, so loads and
// stores are fully coalesced; a row of one head is one contiguous run of
// head_dim elements in its page.
#include "common.hpp"
#include "internal.hpp"

namespace fp8kv {
namespace {

template <int KV>
__global__ __launch_bounds__(256) void quant_append_kernel(AppendParams p) {
  const int chunks_per_row = (p.num_kv_heads * p.head_dim) >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.n_rows * chunks_per_row) return;
  const int row = (int)(idx / chunks_per_row);
  const int e0 = (int)(idx - (int64_t)row * chunks_per_row) << 3;  // element within the row
  const int head = e0 / p.head_dim;
  const int d0 = e0 - head * p.head_dim;

  const int seq = p.row_seq[row];
  const int pos = p.row_pos[row];
  const int page_size = 1 << p.log2_page_size;
  if (seq < 0 || seq >= p.batch || pos < 0 || pos >= p.max_pages * page_size) return;
  const int page = p.page_table[(int64_t)seq * p.max_pages + (pos >> p.log2_page_size)];
  if (page < 0 || page >= p.num_pages) return;
  const int slot = pos & (page_size - 1);
  const int64_t dst = (((int64_t)page * p.num_kv_heads + head) * page_size + slot) * p.head_dim + d0;
  const int64_t src = (int64_t)row * p.num_kv_heads * p.head_dim + e0;

  const u32x4_t kin = *reinterpret_cast<const u32x4_t*>(p.k_new + src);
  const u32x4_t vin = *reinterpret_cast<const u32x4_t*>(p.v_new + src);
  if constexpr (KV == 0) {
    u32x2_t kout, vout;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t kb[2], vb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t kw = kin[2 * half + j], vw = vin[2 * half + j];
        // element 2j+0 is the low half-word, 2j+1 the high one
        const float k0 = __builtin_bit_cast(float, kw << 16) / p.k_scale;
        const float k1 = __builtin_bit_cast(float, kw & 0xFFFF0000u) / p.k_scale;
        const float v0 = __builtin_bit_cast(float, vw << 16) / p.v_scale;
        const float v1 = __builtin_bit_cast(float, vw & 0xFFFF0000u) / p.v_scale;
        kb[j] = e4m3_encode_pair(k0, k1);
        vb[j] = e4m3_encode_pair(v0, v1);
      }
      kout[half] = kb[0] | (kb[1] << 16);
      vout[half] = vb[0] | (vb[1] << 16);
    }
    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(p.k_cache) + dst) = kout;
    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(p.v_cache) + dst) = vout;
  } else {
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.k_cache) + dst) = kin;
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.v_cache) + dst) = vin;
  }
}

}  // namespace

hipError_t launch_quant_append(const AppendParams& p, int kv_dtype, hipStream_t stream) {
  const int64_t threads = (int64_t)p.n_rows * ((p.num_kv_heads * p.head_dim) >> 3);
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (kv_dtype == 0)
    hipLaunchKernelGGL(quant_append_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(quant_append_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8kv
