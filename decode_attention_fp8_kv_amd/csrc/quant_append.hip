// kv_quant_append kernel: BF16 K/V rows -> e4m3 (or BF16) bytes scattered
// into cache pages through the page table.
//
// The cache holds e4m3 values with one fp32 scale per tensor (source pages:
// "Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa
// KV cache"; "更小、更快、更安全：大规模运行Kimi和GLM", section "量化 KV 缓存").
// Each element x becomes e4m3(fp32(x) / scale): an IEEE fp32 division, then
// round-to-nearest-even with saturation at +-448.
//
// One thread moves 16 consecutive elements of one (row, KV head) for both K
// and V: two 16-byte BF16 loads each, one 16-byte (FP8) or two (BF16)
// stores.  Consecutive threads cover consecutive elements of a row, so loads
// and stores are fully coalesced; a row of one head is one contiguous run
// of head_dim elements in its page.  Sixteen independent divisions per
// tensor and thread keep the IEEE division's dependency chains overlapped.
//
// A decode step's first kernel (append_check_kernel) runs these rows and the
// page check of the step's decode in one launch: the append writes only
// cache bytes and the check reads only the page table, lengths and tags, so
// the two are independent, and the check's blocks run beside the append's
// instead of costing a launch of their own.
#include "common.hpp"
#include "internal.hpp"
#include "page_check.hpp"

namespace fp8kv {
namespace {

constexpr int kChunk = 16;  // elements per thread

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// 16 BF16 elements (two 16-byte words) -> 16 e4m3 codes of fp32(x) / s.
__device__ __forceinline__ u32x4_t quant16(const u32x4_t (&in)[2], float s) {
  u32x4_t out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // output word q = elements 4q .. 4q+3
    const uint32_t w0 = in[q >> 1][2 * (q & 1)], w1 = in[q >> 1][2 * (q & 1) + 1];
    out[q] = e4m3_encode_pair(bf16_lo(w0) / s, bf16_hi(w0) / s) |
             (e4m3_encode_pair(bf16_lo(w1) / s, bf16_hi(w1) / s) << 16);
  }
  return out;
}

// Thread idx of the append: elements [16 c, 16 c + 16) of one row's
// num_kv_heads * head_dim, c = idx % (num_kv_heads * head_dim / 16).
template <int KV>
__device__ __forceinline__ void append_chunk(const AppendParams& p, int64_t idx) {
  const int chunks_per_row = (p.num_kv_heads * p.head_dim) / kChunk;
  if (idx >= (int64_t)p.n_rows * chunks_per_row) return;
  const int row = (int)(idx / chunks_per_row);
  const int e0 = (int)(idx - (int64_t)row * chunks_per_row) * kChunk;  // element within the row
  const int head = e0 / p.head_dim;
  const int d0 = e0 - head * p.head_dim;

  const int seq = p.row_seq[row];
  const int pos = p.row_pos[row];
  const int page_size = 1 << p.log2_page_size;
  const bool reports = p.row_status != nullptr && e0 == 0;  // the row's first thread reports its status
  if (seq < 0 || seq >= p.batch || pos < 0 || pos >= p.max_pages * page_size) {
    if (reports) p.row_status[row] = 2;
    return;
  }
  const int64_t at = (int64_t)seq * p.max_pages + (pos >> p.log2_page_size);
  const int page = p.page_table[at];
  if (page < 0 || page >= p.num_pages) {
    if (reports) p.row_status[row] = 2;
    return;
  }
  // Checked append: the page must still belong to the generation the
  // sequence recorded for this slot.
  if (p.page_tags != nullptr && p.page_tags[page] != p.expected_tags[at]) {
    if (reports) p.row_status[row] = 1;
    return;
  }
  if (reports) p.row_status[row] = 0;
  const int slot = pos & (page_size - 1);
  const int64_t dst = (((int64_t)page * p.num_kv_heads + head) * page_size + slot) * p.head_dim + d0;
  const int64_t src = (int64_t)row * p.num_kv_heads * p.head_dim + e0;

  u32x4_t kin[2], vin[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    kin[h] = *reinterpret_cast<const u32x4_t*>(p.k_new + src + 8 * h);
    vin[h] = *reinterpret_cast<const u32x4_t*>(p.v_new + src + 8 * h);
  }
  if constexpr (KV == 0) {
    // Device-scale append: the scales come from device memory (a scale that
    // is not finite and positive writes nothing).
    const float ks = p.k_scale_dev != nullptr ? *p.k_scale_dev : p.k_scale;
    const float vs = p.v_scale_dev != nullptr ? *p.v_scale_dev : p.v_scale;
    if (!(ks > 0.f && ks <= 3.40282347e38f && vs > 0.f && vs <= 3.40282347e38f)) return;
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(p.k_cache) + dst) = quant16(kin, ks);
    *reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(p.v_cache) + dst) = quant16(vin, vs);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.k_cache) + dst + 8 * h) = kin[h];
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.v_cache) + dst + 8 * h) = vin[h];
    }
  }
}

template <int KV>
__global__ __launch_bounds__(256) void quant_append_kernel(AppendParams p) {
  append_chunk<KV>(p, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Blocks [0, append_blocks): the append; then one block per (chunk c,
// sequence b) of the page check, c fastest.  The branch is uniform per block,
// as check_block's block-wide reductions require.
template <int KV>
__global__ __launch_bounds__(256) void append_check_kernel(AppendParams a, DecodeParams d, int64_t append_blocks) {
  const int64_t blk = blockIdx.x;
  if (blk < append_blocks) {
    append_chunk<KV>(a, blk * 256 + threadIdx.x);
    return;
  }
  const int64_t cb = blk - append_blocks;
  check_block(d, (int)(cb % d.check_chunks), (int)(cb / d.check_chunks));
}

static_assert(kBlockThreads == 256, "the append and the check share a block size");

int64_t append_blocks(const AppendParams& p) {
  const int64_t threads = (int64_t)p.n_rows * ((p.num_kv_heads * p.head_dim) / kChunk);
  return (threads + 255) / 256;
}

}  // namespace

hipError_t launch_quant_append(const AppendParams& p, int kv_dtype, hipStream_t stream) {
  const int64_t blocks = append_blocks(p);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (kv_dtype == 0)
    hipLaunchKernelGGL(quant_append_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(quant_append_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append_check(const AppendParams& a, const DecodeParams& d, int kv_dtype, hipStream_t stream) {
  const int64_t na = append_blocks(a);
  const int64_t total = na + (int64_t)d.check_chunks * d.batch;
  if (total > 0x7FFFFFFF) {  // too many blocks for one 1-D grid: two launches
    const hipError_t e = launch_quant_append(a, kv_dtype, stream);
    if (e != hipSuccess) return e;
    return launch_page_check(d, stream);
  }
  if (kv_dtype == 0)
    hipLaunchKernelGGL(append_check_kernel<0>, dim3((unsigned)total), dim3(256), 0, stream, a, d, na);
  else
    hipLaunchKernelGGL(append_check_kernel<1>, dim3((unsigned)total), dim3(256), 0, stream, a, d, na);
  return hipGetLastError();
}

}  // namespace fp8kv
