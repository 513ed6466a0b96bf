// C-ABI entry points declared in include/fp8kv.h: host-side argument checks,
// the work plan, and launches on the caller's stream.  No entry point
// allocates, synchronizes or reads device memory.
#include "fp8kv.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.hpp"

namespace fp8kv {
namespace {

thread_local char g_last_hip_error[256] = "";

int record_hip(hipError_t e) {
  if (e == hipSuccess) return FP8KV_OK;
  std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return FP8KV_ERR_LAUNCH;
}

bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }

int log2_page_size(int32_t ps) {
  if (ps < 16 || ps > 256 || (ps & (ps - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < ps) ++l;
  return l;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool finite_positive(float x) { return std::isfinite(x) && x > 0.0f; }

constexpr int32_t kDefaultComputeUnits = 256;  // MI355X's count, if the device cannot be queried
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_compute_units[kMaxDevices];  // 0 = not queried yet
constexpr int32_t kBlocksPerCu = 1;        // 4 waves per CU stream as fast as 8 and split the work less
constexpr int64_t kMinTilesPerWave = 4;   // below this, fewer waves: merge cost beats parallelism
constexpr int64_t kMaxBlocks = 65535;
constexpr int64_t kMaxTotalTiles = int64_t(1) << 40;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t max_total_tiles(int32_t batch, int32_t num_kv_heads, int32_t page_size, int32_t max_pages) {
  const int64_t max_tiles = ((int64_t)max_pages * page_size + kTileTokens - 1) / kTileTokens;
  return (int64_t)batch * num_kv_heads * max_tiles;
}

}  // namespace

// The default grids keep every block resident: one workgroup per compute unit.  A partitioned device
// (e.g. a CPX-mode MI355X that shows 32 CUs) gets a grid of its own size.
int32_t device_compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultComputeUnits;
  }
  int32_t cus = g_compute_units[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = kDefaultComputeUnits;
  }
  g_compute_units[dev].store(n, std::memory_order_relaxed);
  return n;
}

int32_t plan_blocks(int32_t batch, int32_t num_kv_heads, int32_t page_size, int32_t max_pages, int32_t num_blocks,
                    int32_t blocks_per_cu) {
  int64_t nb = num_blocks;
  if (nb <= 0) {
    const int64_t bound = max_total_tiles(batch, num_kv_heads, page_size, max_pages);
    const int64_t per_block = kMinTilesPerWave * kWavesPerBlock;
    nb = std::min((int64_t)device_compute_units() * blocks_per_cu, (bound + per_block - 1) / per_block);
  }
  return (int32_t)std::max<int64_t>(1, std::min(nb, kMaxBlocks));
}

WorkspaceLayout workspace_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_pages, int32_t num_blocks) {
  const size_t group = (size_t)(num_q_heads / num_kv_heads);
  const size_t segs = (size_t)batch * num_kv_heads;
  const size_t slots = 2 * (size_t)num_blocks * kWavesPerBlock;  // two partial slots per wave
  WorkspaceLayout w;
  w.check_bits = 0;
  w.seg_desc = round_up((size_t)batch * check_chunks(max_pages), 256);
  w.part_ml = w.seg_desc + round_up(segs * sizeof(uint64_t), 256);
  w.part_acc = w.part_ml + round_up(slots * group * 2 * sizeof(float), 256);
  w.total = w.part_acc + round_up(slots * group * head_dim * sizeof(float), 256);
  return w;
}

}  // namespace fp8kv

using namespace fp8kv;

extern "C" {

int fp8kv_abi_version(void) { return FP8KV_ABI_VERSION; }

const char* fp8kv_status_string(int status) {
  switch (status) {
    case FP8KV_OK: return "ok";
    case FP8KV_ERR_NULL: return "a required pointer is NULL";
    case FP8KV_ERR_SHAPE: return "invalid size (non-positive, heads not divisible, or too large)";
    case FP8KV_ERR_UNSUPPORTED: return "unsupported head_dim, page_size, GQA group or kv_dtype";
    case FP8KV_ERR_WORKSPACE: return "workspace too small";
    case FP8KV_ERR_SCALE: return "scale not finite and positive";
    case FP8KV_ERR_TAGS: return "page_tags and expected_tags must both be NULL or both be set";
    case FP8KV_ERR_LAUNCH: return "HIP launch failed (see fp8kv_last_hip_error)";
    case FP8KV_ERR_ALIGN: return "a pointer is not aligned as required";
    case FP8KV_ERR_SCRATCH: return "the sizes need more workspace than the fixed scratch of the no-allocation call holds";
    default: return "unknown status";
  }
}

const char* fp8kv_last_hip_error(void) { return g_last_hip_error; }

namespace {
// Argument checks and parameters of an append; FP8KV_OK or the status to return (nothing launched).
int append_setup(const uint16_t* k_new, const uint16_t* v_new, const int32_t* row_seq, const int32_t* row_pos,
                 const int32_t* page_table, int32_t batch, int32_t max_pages, float k_scale, float v_scale,
                 void* k_cache, void* v_cache, int32_t num_pages, int32_t n_rows, int32_t num_kv_heads,
                 int32_t head_dim, int32_t page_size, int32_t kv_dtype, const uint32_t* page_tags,
                 const uint32_t* expected_tags, uint8_t* row_status, const float* k_scale_dev,
                 const float* v_scale_dev, AppendParams& p) {
  if (kv_dtype != FP8KV_KV_FP8_E4M3 && kv_dtype != FP8KV_KV_BF16) return FP8KV_ERR_UNSUPPORTED;
  if (n_rows < 0 || batch <= 0 || max_pages <= 0 || num_pages <= 0 || num_kv_heads <= 0 || num_kv_heads > 65535)
    return FP8KV_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return FP8KV_ERR_UNSUPPORTED;
  const int l2ps = log2_page_size(page_size);
  if (l2ps < 0) return FP8KV_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * page_size > INT32_MAX) return FP8KV_ERR_SHAPE;
  if (n_rows == 0) return FP8KV_OK;
  if (!k_new || !v_new || !row_seq || !row_pos || !page_table || !k_cache || !v_cache) return FP8KV_ERR_NULL;
  if (kv_dtype == FP8KV_KV_FP8_E4M3 && !k_scale_dev && (!finite_positive(k_scale) || !finite_positive(v_scale)))
    return FP8KV_ERR_SCALE;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return FP8KV_ERR_ALIGN;

  p.k_scale_dev = k_scale_dev;
  p.v_scale_dev = v_scale_dev;
  p.k_new = k_new;
  p.v_new = v_new;
  p.row_seq = row_seq;
  p.row_pos = row_pos;
  p.page_table = page_table;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.page_tags = page_tags;
  p.expected_tags = expected_tags;
  p.row_status = row_status;
  p.batch = batch;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.n_rows = n_rows;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.log2_page_size = l2ps;
  return FP8KV_OK;
}

int quant_append_impl(const uint16_t* k_new, const uint16_t* v_new, const int32_t* row_seq, const int32_t* row_pos,
                      const int32_t* page_table, int32_t batch, int32_t max_pages, float k_scale, float v_scale,
                      void* k_cache, void* v_cache, int32_t num_pages, int32_t n_rows, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, int32_t kv_dtype, const uint32_t* page_tags,
                      const uint32_t* expected_tags, uint8_t* row_status, const float* k_scale_dev,
                      const float* v_scale_dev, void* stream) {
  AppendParams p{};
  const int st = append_setup(k_new, v_new, row_seq, row_pos, page_table, batch, max_pages, k_scale, v_scale,
                              k_cache, v_cache, num_pages, n_rows, num_kv_heads, head_dim, page_size, kv_dtype,
                              page_tags, expected_tags, row_status, k_scale_dev, v_scale_dev, p);
  if (st != FP8KV_OK || n_rows == 0) return st;
  return record_hip(launch_quant_append(p, kv_dtype, static_cast<hipStream_t>(stream)));
}

bool pool_sizes_ok(int32_t batch, int32_t max_pages, int32_t num_pages) {
  return batch > 0 && max_pages > 0 && num_pages > 0;
}
}  // namespace

int kv_quant_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* row_seq, const int32_t* row_pos,
                    const int32_t* page_table, int32_t batch, int32_t max_pages, float k_scale, float v_scale,
                    void* k_cache, void* v_cache, int32_t num_pages, int32_t n_rows, int32_t num_kv_heads,
                    int32_t head_dim, int32_t page_size, int32_t kv_dtype, void* stream) {
  return quant_append_impl(k_new, v_new, row_seq, row_pos, page_table, batch, max_pages, k_scale, v_scale, k_cache,
                           v_cache, num_pages, n_rows, num_kv_heads, head_dim, page_size, kv_dtype, nullptr,
                           nullptr, nullptr, nullptr, nullptr, stream);
}

int kv_quant_append_checked(const uint16_t* k_new, const uint16_t* v_new, const int32_t* row_seq,
                            const int32_t* row_pos, const int32_t* page_table, int32_t batch, int32_t max_pages,
                            float k_scale, float v_scale, void* k_cache, void* v_cache, int32_t num_pages,
                            int32_t n_rows, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t kv_dtype, const uint32_t* page_tags, const uint32_t* expected_tags,
                            uint8_t* row_status, void* stream) {
  if (n_rows > 0 && (!page_tags || !expected_tags || !row_status)) return FP8KV_ERR_NULL;
  return quant_append_impl(k_new, v_new, row_seq, row_pos, page_table, batch, max_pages, k_scale, v_scale, k_cache,
                           v_cache, num_pages, n_rows, num_kv_heads, head_dim, page_size, kv_dtype, page_tags,
                           expected_tags, row_status, nullptr, nullptr, stream);
}

int kv_quant_append_dscale(const uint16_t* k_new, const uint16_t* v_new, const int32_t* row_seq,
                           const int32_t* row_pos, const int32_t* page_table, int32_t batch, int32_t max_pages,
                           const float* k_scale_dev, const float* v_scale_dev, void* k_cache, void* v_cache,
                           int32_t num_pages, int32_t n_rows, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, void* stream) {
  if (n_rows > 0 && (!k_scale_dev || !v_scale_dev)) return FP8KV_ERR_NULL;
  if (n_rows > 0 && (!aligned(k_scale_dev, 4) || !aligned(v_scale_dev, 4))) return FP8KV_ERR_ALIGN;
  return quant_append_impl(k_new, v_new, row_seq, row_pos, page_table, batch, max_pages, 1.0f, 1.0f, k_cache,
                           v_cache, num_pages, n_rows, num_kv_heads, head_dim, page_size, FP8KV_KV_FP8_E4M3,
                           nullptr, nullptr, nullptr, k_scale_dev, v_scale_dev, stream);
}

int kv_absmax_scale(const uint16_t* x, int64_t n, float* out, float* work, void* stream) {
  static_assert(kAmaxWorkFloats == FP8KV_AMAX_WORK_FLOATS, "work buffer size");
  if (n < 0) return FP8KV_ERR_SHAPE;
  if (!out || !work || (n > 0 && !x)) return FP8KV_ERR_NULL;
  if ((n > 0 && !aligned(x, 16)) || !aligned(out, 4) || !aligned(work, 4)) return FP8KV_ERR_ALIGN;
  return record_hip(launch_absmax_scale(x, x, 1, n, out, work, static_cast<hipStream_t>(stream)));
}

int kv_absmax_scale_kv(const uint16_t* k, const uint16_t* v, int64_t n, float* out, float* work, void* stream) {
  if (n < 0) return FP8KV_ERR_SHAPE;
  if (!out || !work || (n > 0 && (!k || !v))) return FP8KV_ERR_NULL;
  if ((n > 0 && (!aligned(k, 16) || !aligned(v, 16))) || !aligned(out, 4) || !aligned(work, 4))
    return FP8KV_ERR_ALIGN;
  return record_hip(launch_absmax_scale(k, v, 2, n, out, work, static_cast<hipStream_t>(stream)));
}

int page_pool_init(int32_t* free_pages, int32_t* free_count, int32_t num_pages, void* stream) {
  if (num_pages <= 0) return FP8KV_ERR_SHAPE;
  if (!free_pages || !free_count) return FP8KV_ERR_NULL;
  return record_hip(launch_pool_init(free_pages, free_count, num_pages, static_cast<hipStream_t>(stream)));
}

int page_alloc(const int32_t* n_new, int32_t* page_counts, int32_t* page_table, uint32_t* expected_tags,
               uint32_t* page_tags, int32_t* free_pages, int32_t* free_count, uint8_t* status, int32_t batch,
               int32_t max_pages, int32_t num_pages, void* stream) {
  if (!pool_sizes_ok(batch, max_pages, num_pages)) return FP8KV_ERR_SHAPE;
  if (!n_new || !page_counts || !page_table || !expected_tags || !page_tags || !free_pages || !free_count ||
      !status)
    return FP8KV_ERR_NULL;
  PoolParams p{};
  p.n_new = n_new;
  p.page_counts = page_counts;
  p.page_table = page_table;
  p.expected_tags = expected_tags;
  p.page_tags = page_tags;
  p.free_pages = free_pages;
  p.free_count = free_count;
  p.status = status;
  p.batch = batch;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  return record_hip(launch_pool_alloc(p, static_cast<hipStream_t>(stream)));
}

int page_free(const uint8_t* release, int32_t* page_counts, const int32_t* page_table, int32_t* free_pages,
              int32_t* free_count, uint8_t* status, int32_t batch, int32_t max_pages, int32_t num_pages,
              void* stream) {
  if (!pool_sizes_ok(batch, max_pages, num_pages)) return FP8KV_ERR_SHAPE;
  if (!release || !page_counts || !page_table || !free_pages || !free_count || !status) return FP8KV_ERR_NULL;
  PoolParams p{};
  p.release = release;
  p.page_counts = page_counts;
  p.page_table = const_cast<int32_t*>(page_table);  // only read by the free kernel
  p.free_pages = free_pages;
  p.free_count = free_count;
  p.status = status;
  p.batch = batch;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  return record_hip(launch_pool_free(p, static_cast<hipStream_t>(stream)));
}

int int4_gemv(const uint16_t* x, const uint32_t* w_tiles, const uint16_t* s_tiles, uint16_t* y, int32_t m, int32_t n,
              int32_t k, void* stream) {
  if (m < 1 || m > FP8KV_INT4_MAX_M || n < 1 || k < FP8KV_INT4_GROUP || k % FP8KV_INT4_GROUP != 0)
    return FP8KV_ERR_SHAPE;
  if (!x || !w_tiles || !s_tiles || !y) return FP8KV_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_tiles, 16) || !aligned(s_tiles, 2) || !aligned(y, 2)) return FP8KV_ERR_ALIGN;
  Int4GemvParams p{};
  p.x = x;
  p.w = w_tiles;
  p.s = s_tiles;
  p.y = y;
  p.m = m;
  p.n = n;
  p.k = k;
  return record_hip(launch_int4_gemv(p, static_cast<hipStream_t>(stream)));
}

int int4_pack_weights(const uint32_t* w_rows, const uint16_t* s_rows, uint32_t* w_tiles, uint16_t* s_tiles, int32_t n,
                      int32_t k, void* stream) {
  if (n < 1 || k < FP8KV_INT4_GROUP || k % FP8KV_INT4_GROUP != 0) return FP8KV_ERR_SHAPE;
  if (!w_rows || !s_rows || !w_tiles || !s_tiles) return FP8KV_ERR_NULL;
  if (!aligned(w_rows, 4) || !aligned(s_rows, 2) || !aligned(w_tiles, 16) || !aligned(s_tiles, 2))
    return FP8KV_ERR_ALIGN;
  return record_hip(launch_int4_pack(w_rows, s_rows, w_tiles, s_tiles, n, k, static_cast<hipStream_t>(stream)));
}

size_t paged_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t page_size, int32_t max_pages, int32_t num_blocks) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_pages <= 0 || num_blocks < 0) return 0;
  if (num_q_heads % num_kv_heads != 0 || !supported_head_dim(head_dim) || log2_page_size(page_size) < 0) return 0;
  const int32_t nb = plan_blocks(batch, num_kv_heads, page_size, max_pages, num_blocks, kBlocksPerCu);
  return workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, max_pages, nb).total;
}

int paged_decode_attn_path(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
  const char* force = std::getenv("FP8KV_FORCE_PATH");
  if (force && std::strcmp(force, "mfma") == 0) return 1;
  if (force && std::strcmp(force, "valu") == 0 && num_q_heads / num_kv_heads <= 4) return 0;
  return num_q_heads / num_kv_heads >= 5 ? 1 : 0;
}

namespace {
// Argument checks and parameters of a decode call; FP8KV_OK or the status to return (nothing launched).
int decode_setup(const uint16_t* q, const void* k_cache, const void* v_cache, int32_t kv_dtype, float k_scale,
                 float v_scale, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                 const uint32_t* page_tags, const uint32_t* expected_tags, uint16_t* out, uint8_t* abort_flags,
                 void* workspace, size_t workspace_bytes, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t page_size, int32_t num_pages, float softmax_scale, int32_t num_blocks,
                 DecodeParams& p, bool& mfma) {
  if (kv_dtype != FP8KV_KV_FP8_E4M3 && kv_dtype != FP8KV_KV_BF16) return FP8KV_ERR_UNSUPPORTED;
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_pages <= 0 || num_pages <= 0 || num_blocks < 0)
    return FP8KV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return FP8KV_ERR_SHAPE;
  if (batch > 65535 || num_kv_heads > 65535 || (int64_t)batch * num_q_heads > INT32_MAX) return FP8KV_ERR_SHAPE;
  const int32_t group = num_q_heads / num_kv_heads;
  if (group > kMaxGroup || !supported_head_dim(head_dim)) return FP8KV_ERR_UNSUPPORTED;
  const int l2ps = log2_page_size(page_size);
  if (l2ps < 0) return FP8KV_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * page_size > INT32_MAX) return FP8KV_ERR_SHAPE;
  if (max_total_tiles(batch, num_kv_heads, page_size, max_pages) > kMaxTotalTiles) return FP8KV_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out || !abort_flags || !workspace)
    return FP8KV_ERR_NULL;
  if ((page_tags == nullptr) != (expected_tags == nullptr)) return FP8KV_ERR_TAGS;
  if (kv_dtype == FP8KV_KV_FP8_E4M3 && (!finite_positive(k_scale) || !finite_positive(v_scale)))
    return FP8KV_ERR_SCALE;
  if (!std::isfinite(softmax_scale)) return FP8KV_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(out, 8) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(workspace, 256))
    return FP8KV_ERR_ALIGN;
  mfma = paged_decode_attn_path(num_q_heads, num_kv_heads) == 1;
  // one resident block (4 waves) per CU by default: every decode kernel runs one wave per SIMD
  const int32_t nb = plan_blocks(batch, num_kv_heads, page_size, max_pages, num_blocks, kBlocksPerCu);
  const WorkspaceLayout ws = workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, max_pages, nb);
  if (workspace_bytes < ws.total) return FP8KV_ERR_WORKSPACE;

  const double log2e = 1.4426950408889634;
  p.q = q;
  p.k_cache = static_cast<const uint8_t*>(k_cache);
  p.v_cache = static_cast<const uint8_t*>(v_cache);
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.page_tags = page_tags;
  p.expected_tags = expected_tags;
  p.out = out;
  p.abort_flags = abort_flags;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  p.check_bits = base + ws.check_bits;
  p.check_chunks = check_chunks(max_pages);
  p.checked = page_tags != nullptr ? 1 : 0;
  p.seg_desc = reinterpret_cast<uint64_t*>(base + ws.seg_desc);
  p.part_ml = reinterpret_cast<float*>(base + ws.part_ml);
  p.part_acc = reinterpret_cast<float*>(base + ws.part_acc);
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.log2_page_size = l2ps;
  p.num_blocks = nb;
  if (kv_dtype == FP8KV_KV_FP8_E4M3) {
    p.qk_scale_log2 = (float)((double)softmax_scale * (double)k_scale * log2e);
    p.v_scale = v_scale;
  } else {
    p.qk_scale_log2 = (float)((double)softmax_scale * log2e);
    p.v_scale = 1.0f;
  }
  return FP8KV_OK;
}
}  // namespace

int paged_decode_attn(const uint16_t* q, const void* k_cache, const void* v_cache, int32_t kv_dtype, float k_scale,
                      float v_scale, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                      const uint32_t* page_tags, const uint32_t* expected_tags, uint16_t* out, uint8_t* abort_flags,
                      void* workspace, size_t workspace_bytes, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
                      float softmax_scale, int32_t num_blocks, void* stream) {
  DecodeParams p{};
  bool mfma = false;
  const int st = decode_setup(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_table, max_pages, seq_lens,
                              page_tags, expected_tags, out, abort_flags, workspace, workspace_bytes, batch,
                              num_q_heads, num_kv_heads, head_dim, page_size, num_pages, softmax_scale, num_blocks,
                              p, mfma);
  if (st != FP8KV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.checked) {
    const int e = record_hip(launch_page_check(p, s));
    if (e != FP8KV_OK) return e;
  }
  return record_hip(launch_decode(p, kv_dtype, head_dim, mfma, s));
}

}  // extern "C"

// ------------------------------------------------------------------------
// The no-allocation variant of paged_decode_attn.  Its workspace is this
// file-scope device array: one copy on every device the library runs on,
// held until the process ends, shared by every call on that device (so
// calls that overlap on one device race).  Host code never uses the array's
// name as an address: the device address of the current device's copy is
// looked up once per device with hipGetSymbolAddress and kept.
// ------------------------------------------------------------------------
namespace fp8kv {
namespace {

constexpr size_t kScratchBytes = FP8KV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the workspace is 256-byte aligned");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch_address[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return record_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return record_hip(hipErrorInvalidDevice);
  void* a = g_scratch_address[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    a = g_scratch_address[dev].load(std::memory_order_relaxed);
    if (a == nullptr) {
      const hipError_t es = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (es != hipSuccess || a == nullptr) return record_hip(es != hipSuccess ? es : hipErrorInvalidSymbol);
      g_scratch_address[dev].store(a, std::memory_order_release);
    }
  }
  *out = a;
  return FP8KV_OK;
}

}  // namespace
}  // namespace fp8kv

extern "C" {

int paged_decode_attn_noalloc(const uint16_t* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                              float k_scale, float v_scale, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, const uint32_t* page_tags, const uint32_t* expected_tags,
                              uint16_t* out, uint8_t* abort_flags, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
                              float softmax_scale, int32_t num_blocks, void* stream) {
  // Every argument is checked first, against a stand-in workspace address (aligned, never used): a
  // workspace larger than the scratch is FP8KV_ERR_SCRATCH, and nothing touches the device on an error.
  DecodeParams p{};
  bool mfma = false;
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
  int st = decode_setup(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_table, max_pages, seq_lens, page_tags,
                        expected_tags, out, abort_flags, stand_in, kScratchBytes, batch, num_q_heads, num_kv_heads,
                        head_dim, page_size, num_pages, softmax_scale, num_blocks, p, mfma);
  if (st == FP8KV_ERR_WORKSPACE) return FP8KV_ERR_SCRATCH;
  if (st != FP8KV_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != FP8KV_OK) return st;
  st = decode_setup(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_table, max_pages, seq_lens, page_tags,
                    expected_tags, out, abort_flags, ws, kScratchBytes, batch, num_q_heads, num_kv_heads, head_dim,
                    page_size, num_pages, softmax_scale, num_blocks, p, mfma);
  if (st != FP8KV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.checked) {
    const int e = record_hip(launch_page_check(p, s));
    if (e != FP8KV_OK) return e;
  }
  return record_hip(launch_decode(p, kv_dtype, head_dim, mfma, s));
}

int paged_decode_step(const uint16_t* k_new, const uint16_t* v_new, const int32_t* row_seq, const int32_t* row_pos,
                      int32_t n_rows, const uint16_t* q, void* k_cache, void* v_cache, int32_t kv_dtype,
                      float k_scale, float v_scale, const int32_t* page_table, int32_t max_pages,
                      const int32_t* seq_lens, const uint32_t* page_tags, const uint32_t* expected_tags,
                      uint16_t* out, uint8_t* abort_flags, void* workspace, size_t workspace_bytes, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t num_pages, float softmax_scale, int32_t num_blocks, void* decode_begin_event,
                      void* decode_end_event, void* stream) {
  DecodeParams p{};
  bool mfma = false;
  int st = decode_setup(q, k_cache, v_cache, kv_dtype, k_scale, v_scale, page_table, max_pages, seq_lens, page_tags,
                        expected_tags, out, abort_flags, workspace, workspace_bytes, batch, num_q_heads, num_kv_heads,
                        head_dim, page_size, num_pages, softmax_scale, num_blocks, p, mfma);
  if (st != FP8KV_OK) return st;
  AppendParams a{};
  st = append_setup(k_new, v_new, row_seq, row_pos, page_table, batch, max_pages, k_scale, v_scale, k_cache, v_cache,
                    num_pages, n_rows, num_kv_heads, head_dim, page_size, kv_dtype, nullptr, nullptr, nullptr, nullptr,
                    nullptr, a);
  if (st != FP8KV_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int e = FP8KV_OK;
  if (p.checked)
    e = record_hip(launch_append_check(a, p, kv_dtype, s));
  else if (n_rows > 0)
    e = record_hip(launch_quant_append(a, kv_dtype, s));
  if (e != FP8KV_OK) return e;
  return record_hip(launch_decode(p, kv_dtype, head_dim, mfma, s, static_cast<hipEvent_t>(decode_begin_event),
                                  static_cast<hipEvent_t>(decode_end_event)));
}

}  // extern "C"
