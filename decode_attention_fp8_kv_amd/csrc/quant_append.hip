// kv_quant_append kernel: BF16 K/V rows -> e4m3 (or BF16) bytes scattered
// into cache pages through the page table.
//
// The cache holds e4m3 values with one fp32 scale per tensor (source pages:
// "Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa
// KV cache"; "更小、更快、更安全：大规模运行Kimi和GLM", section "量化 KV 缓存").
// Each element x becomes e4m3(fp32(x) / scale): an IEEE fp32 division, then
// round-to-nearest-even with saturation at +-448.
//
// One thread moves 16 elements of one (row, KV head) for both K and V, two
// 16-byte BF16 loads each: 16 consecutive elements and one 16-byte store
// with an FP8 cache; with a BF16 cache two runs of 8 half a head apart and
// two 16-byte stores, so that each store instruction of a wave writes whole
// lines.  Consecutive threads cover consecutive elements of a row, so loads
// and stores are fully coalesced; a row of one head is one contiguous run
// of head_dim elements in its page.  The cache is written with non-temporal
// stores: the kernel is bound by HBM's mixed read/write rate.
//
// The division without dividing: with an IEEE division per element the kernel
// was bound by its ALU work (the division's scale/fma/fixup sequence and its
// quarter-rate reciprocal cost ~27 lane operations per element), so each
// element is first computed as q1 = fl32(x * r) with r = fl32(1 / s), one
// multiply.  Two correctly rounded operations put q1 within 2 fp32 ulps of the
// wanted fl32(x / s) (r normal), and rounding to e4m3 is monotone, so the two
// give the same code unless an e4m3 rounding midpoint lies within 2 ulps of q1.
// For quotients of at least 2^-6 (e4m3's normal range; also the saturation
// range, where no midpoint exists above 432) the midpoints are the fp32 values
// whose 20 mantissa bits below e4m3's 3 are exactly 1000...0, a fixed-position
// bit test; quotients in [2^-11, 2^-6), where the e4m3 quantum is the subnormal
// 2^-9, are not tested and always divided, and below 2^-11 both round to 0.
// Only flagged elements (a window of +-3 ulps, with a margin) take the IEEE
// division.  When s is a power of two both quotients are exact products and
// equal; when r is not a normal fp32 every element is divided.  Checked
// bit-exact against division on every BF16 pattern at many scales.
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

// The reciprocal of a scale and whether fl32(x * r) may stand in for
// fl32(x / s): kNoShortcut when r is not a normal fp32, kExact when s is a
// power of two (every product is the exact quotient), else kTested.
enum Shortcut { kTested = 0, kExact = 1, kNoShortcut = 2 };
struct Recip {
  float r;
  Shortcut mode;
};
__device__ __forceinline__ Recip reciprocal(float s) {
  Recip c;
  c.r = 1.0f / s;  // IEEE, correctly rounded
  const uint32_t sb = __builtin_bit_cast(uint32_t, s);
  if (!(c.r >= 1.17549435e-38f && c.r <= 3.40282347e38f))
    c.mode = kNoShortcut;
  else if ((sb & 0x7FFFFFu) == 0u && (sb & 0x7F800000u) != 0u)
    c.mode = kExact;
  else
    c.mode = kTested;
  return c;
}

constexpr uint32_t kMidWindow = 3;  // fp32 ulps around an e4m3 midpoint that take the division

// fp32 -> e4m3 of a pair known not to hold a NaN: clamp to +-448, then the
// hardware's round-to-nearest-even conversion.
__device__ __forceinline__ uint32_t e4m3_encode_pair_finite(float a, float b) {
  const float ca = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  const float cb = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}

// 16 BF16 elements (two 16-byte words) -> 16 e4m3 codes of fl32(x / s).
__device__ __forceinline__ u32x4_t quant16(const u32x4_t (&in)[2], float s, const Recip& rc) {
  float x[16], q[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = in[i >> 2][i & 3];
    x[2 * i] = bf16_lo(w);
    x[2 * i + 1] = bf16_hi(w);
  }
  const bool tested = rc.mode == kTested, all = rc.mode == kNoShortcut;  // uniform
  bool any_nan = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    q[i] = x[i] * rc.r;
    const float a = __builtin_fabsf(q[i]);
    const bool normal = a >= 0x1p-6f;  // e4m3 normal or saturated range: test the midpoint bits
    const bool small = a >= 0x1p-11f;  // with !normal: e4m3 subnormal range, always divided
    const bool near_mid =
        ((__builtin_bit_cast(uint32_t, q[i]) & 0xFFFFFu) - (0x80000u - kMidWindow)) <= 2u * kMidWindow;
    // normal implies small: divide iff small and (not normal, or near a midpoint)
    const bool flag = small & (near_mid | !normal);
    if (all | (tested & flag)) q[i] = x[i] / s;  // rare: a masked branch
    if (i & 1) any_nan |= __builtin_isunordered(q[i - 1], q[i]);
  }
  u32x4_t out;
#pragma unroll
  for (int w = 0; w < 4; ++w)  // output word w = elements 4w .. 4w+3
    out[w] = e4m3_encode_pair_finite(q[4 * w], q[4 * w + 1]) |
             (e4m3_encode_pair_finite(q[4 * w + 2], q[4 * w + 3]) << 16);
  if (any_nan) {  // NaN inputs (rare): every NaN becomes 0x7F
#pragma unroll
    for (int w = 0; w < 4; ++w)
      out[w] = e4m3_encode_pair(q[4 * w], q[4 * w + 1]) | (e4m3_encode_pair(q[4 * w + 2], q[4 * w + 3]) << 16);
  }
  return out;
}

// Thread `threadIdx.x` of append block `blk`: flattened chunk idx = 256 blk +
// threadIdx.x, i.e. elements [16 c, 16 c + 16) of row idx / cpr's
// num_kv_heads * head_dim, c = idx % cpr, cpr = num_kv_heads * head_dim / 16.
// The 64-bit division is done once per block on uniform values; each thread
// adds its offset and divides a small number (< cpr + 256) by cpr through the
// fp32 reciprocal, corrected to the exact quotient.
template <int KV>
__device__ __forceinline__ void append_chunk(const AppendParams& p, int64_t blk) {
  const int cpr = (p.num_kv_heads * p.head_dim) / kChunk;
  const int64_t base = blk * 256;
  const int64_t row0 = base / cpr;
  const int t = (int)(base - row0 * cpr) + (int)threadIdx.x;
  int extra = (int)((float)t * (1.0f / (float)cpr));
  extra -= extra * cpr > t ? 1 : 0;
  extra += (extra + 1) * cpr <= t ? 1 : 0;
  if (row0 + extra >= p.n_rows) return;
  const int row = (int)(row0 + extra);
  const int e0 = (t - extra * cpr) * kChunk;  // element within the row
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

  // FP8: the thread's 16 elements are contiguous (one 16-byte store).  BF16:
  // elements [8c, 8c + 8) and [D/2 + 8c, +8) of its head (c = d0 / 16), so
  // that each of its two 16-byte stores lines up with its neighbours' into
  // whole lines.  The cache is written with non-temporal stores (streamed
  // past the caches: the append's rows are not read back by this kernel);
  // with two adjacent 16-byte stores per thread each store instruction
  // covered half of every line and the non-temporal BF16 append ran at 4.1
  // TB/s instead of 5.5.
  const int64_t piece = KV == 0 ? 8 : p.head_dim / 2;
  const int64_t shift = KV == 0 ? 0 : -(d0 / 2);
  u32x4_t kin[2], vin[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    kin[h] = *reinterpret_cast<const u32x4_t*>(p.k_new + src + shift + piece * h);
    vin[h] = *reinterpret_cast<const u32x4_t*>(p.v_new + src + shift + piece * h);
  }
  if constexpr (KV == 0) {
    // Device-scale append: the scales come from device memory (a scale that
    // is not finite and positive writes nothing).
    const float ks = p.k_scale_dev != nullptr ? *p.k_scale_dev : p.k_scale;
    const float vs = p.v_scale_dev != nullptr ? *p.v_scale_dev : p.v_scale;
    if (!(ks > 0.f && ks <= 3.40282347e38f && vs > 0.f && vs <= 3.40282347e38f)) return;
    __builtin_nontemporal_store(quant16(kin, ks, reciprocal(ks)),
                                reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(p.k_cache) + dst));
    __builtin_nontemporal_store(quant16(vin, vs, reciprocal(vs)),
                                reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(p.v_cache) + dst));
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __builtin_nontemporal_store(kin[h], reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.k_cache) + dst + shift +
                                                                     piece * h));
      __builtin_nontemporal_store(vin[h], reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.v_cache) + dst + shift +
                                                                     piece * h));
    }
  }
}

template <int KV>
__global__ __launch_bounds__(256) void quant_append_kernel(AppendParams p) {
  append_chunk<KV>(p, blockIdx.x);
}

// Blocks [0, append_blocks): the append; then one block per (chunk c,
// sequence b) of the page check, c fastest.  The branch is uniform per block,
// as check_block's block-wide reductions require.
template <int KV>
__global__ __launch_bounds__(256) void append_check_kernel(AppendParams a, DecodeParams d, int64_t append_blocks) {
  const int64_t blk = blockIdx.x;
  if (blk < append_blocks) {
    append_chunk<KV>(a, blk);
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
