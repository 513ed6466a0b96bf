// Internal interface between the C-ABI entry points (api.cpp) and the kernel
// translation units.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8kv {

constexpr int kTileTokens = 64;   // tokens per tile handled by one wave at a time
constexpr int kWavesPerBlock = 4; // waves per workgroup (independent workers)
constexpr int kBlockThreads = 64 * kWavesPerBlock;
constexpr int kMaxGroup = 16;     // query heads per KV head handled by one workgroup

struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const int32_t* page_table;
  void* k_cache;
  void* v_cache;
  float k_scale, v_scale;
  const float* k_scale_dev;         // device-scale append: scales read from device memory, or null
  const float* v_scale_dev;
  const uint32_t* page_tags;        // checked append: [num_pages], or null (no check)
  const uint32_t* expected_tags;    // checked append: [B][max_pages]
  uint8_t* row_status;              // checked append: [n_rows] 0 written, 1 tag mismatch, 2 bad destination
  int32_t batch, max_pages, num_pages, n_rows, num_kv_heads, head_dim, log2_page_size;
};

struct PoolParams {
  const int32_t* n_new;             // alloc: pages requested per sequence [B]
  const uint8_t* release;           // free: nonzero = return the sequence's pages [B]
  int32_t* page_counts;             // [B] pages each sequence holds
  int32_t* page_table;              // [B][max_pages]
  uint32_t* expected_tags;          // [B][max_pages]
  uint32_t* page_tags;              // [num_pages]
  int32_t* free_pages;              // [num_pages] stack of free page ids (top = last)
  int32_t* free_count;              // [1] number of free pages
  uint8_t* status;                  // [B]
  int32_t batch, max_pages, num_pages;
};

struct Int4GemvParams {
  const uint16_t* x;                // bf16 [m][k]
  const uint32_t* w;                // tile layout: [ceil(n/16)][k/128][16 rows][16 words]
  const uint16_t* s;                // tile layout: bf16 [ceil(n/16)][k/128][16 rows]
  uint16_t* y;                      // bf16 [m][n]
  int32_t m, n, k;
};

struct DecodeParams {
  const uint16_t* q;                // bf16 [B][Hq][D]
  const uint8_t* k_cache;           // [P][Hkv][PS][D] elements
  const uint8_t* v_cache;
  const int32_t* page_table;        // [B][max_pages]
  const int32_t* seq_lens;          // [B]
  const uint32_t* page_tags;        // [P] or null (check off)
  const uint32_t* expected_tags;    // [B][max_pages] or null
  uint16_t* out;                    // bf16 [B][Hq][D]
  uint8_t* abort_flags;             // [B]
  uint8_t* check_bits;              // [B][check_chunks] abort bits found by the page check
  uint64_t* seg_desc;               // [B*Hkv] first partial slot | number of partials << 32 (< 2: none);
                                    // bit 63: a page id failed the decode's range check
  float* part_ml;                   // [2*waves][G][2]  running max (log2 domain), sum
  float* part_acc;                  // [2*waves][G][D]  unnormalized output
  int32_t batch, num_q_heads, num_kv_heads, group, max_pages, num_pages;
  int32_t log2_page_size;
  int32_t num_blocks;               // grid size; each of its 4*num_blocks waves owns an equal share
  int32_t check_chunks;             // page-check blocks per sequence (1024 page slots each)
  int32_t checked;                  // 1: check_bits hold this call's page check (tags on); 0: no
                                    // check ran, lengths are checked in the decode's schedule and
                                    // page ids as each round of pages is loaded
  float qk_scale_log2;              // softmax_scale * k_scale * log2(e)
  float v_scale;                    // folded into the final normalization
};

// Grid size chosen on the host from sizes only (no device reads).
int32_t plan_blocks(int32_t batch, int32_t num_kv_heads, int32_t page_size, int32_t max_pages,
                    int32_t num_blocks, int32_t blocks_per_cu);

struct WorkspaceLayout {
  size_t check_bits, seg_desc, part_ml, part_acc, total;
};
WorkspaceLayout workspace_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_pages, int32_t num_blocks);
constexpr int32_t kCheckSlots = 1024;  // page-table slots per page-check block
inline int32_t check_chunks(int32_t max_pages) { return (max_pages + kCheckSlots - 1) / kCheckSlots; }

hipError_t launch_quant_append(const AppendParams& p, int kv_dtype, hipStream_t stream);
constexpr int32_t kAmaxWorkFloats = 512;  // equals FP8KV_AMAX_WORK_FLOATS
// tensors = 1 (x0) or 2 (x0 and x1, n elements each); work holds tensors * kAmaxWorkFloats floats
hipError_t launch_absmax_scale(const uint16_t* x0, const uint16_t* x1, int tensors, int64_t n, float* out,
                               float* work, hipStream_t stream);
hipError_t launch_pool_init(int32_t* free_pages, int32_t* free_count, int32_t num_pages, hipStream_t stream);
hipError_t launch_pool_alloc(const PoolParams& p, hipStream_t stream);
hipError_t launch_pool_free(const PoolParams& p, hipStream_t stream);
hipError_t launch_int4_gemv(const Int4GemvParams& p, hipStream_t stream);
hipError_t launch_int4_pack(const uint32_t* w_rows, const uint16_t* s_rows, uint32_t* w_tiles, uint16_t* s_tiles,
                            int32_t n, int32_t k, hipStream_t stream);
// Page check alone (one block per 1024-slot chunk of a sequence); writes check_bits.
hipError_t launch_page_check(const DecodeParams& p, hipStream_t stream);
// The append's rows and the page check in one launch (a decode step's first kernel): the append's
// blocks come first, then one block per (chunk, sequence) of the check.
hipError_t launch_append_check(const AppendParams& a, const DecodeParams& d, int kv_dtype, hipStream_t stream);
// Decode + merge.  Events, when not null, are recorded on the stream right before the decode kernel
// and right after it (before the merge).
hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int head_dim, bool mfma, hipStream_t stream,
                         hipEvent_t decode_begin = nullptr, hipEvent_t decode_end = nullptr);

// Compute units of the current device, queried once per device (256, MI355X's count, if the query
// fails, e.g. when no device is visible to a host-only caller).
int32_t device_compute_units();

}  // namespace fp8kv
