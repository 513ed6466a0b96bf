// The page check of paged_decode_attn, as a block-level device function that
// two launches share: the check kernel of a decode call with tags on, and the
// first kernel of a decode step, where the check's blocks run beside the
// append's.
//
// Source pages: "ترفندهای کلادفلر برای جا دادن مدل‌های غول‌پیکر تو GPU", third
// technique, and "Tối ưu hóa mô hình AI quy mô lớn", section "Bảo vệ tính toàn
// vẹn của KV Cache" -- every cache page carries a tag that changes when the
// page is reallocated; the tag is compared before the page is used and a
// mismatch aborts the request.
#pragma once

#include "internal.hpp"

namespace fp8kv {

constexpr uint32_t kAbortTag = 1u;   // a used page's tag differs from the expected tag
constexpr uint32_t kAbortMeta = 2u;  // bad length, or a used page id out of range

constexpr int kCheckUnroll = 4;                             // slots per thread
constexpr int kCheckChunk = kCheckUnroll * kBlockThreads;   // slots per block
static_assert(kCheckChunk == kCheckSlots, "the host sizes the check grid with kCheckSlots");

// One block (kBlockThreads threads, every one of them calling this) checks
// page-table slots [c * 1024, (c + 1) * 1024) of sequence b.  Every slot j <
// ceil(L / page_size) is checked: the id must lie in [0, num_pages) (else
// kAbortMeta) and, when tags are on, the page's current tag must equal the tag
// the sequence recorded for that slot (else kAbortTag); a length outside
// [1, max_pages * page_size] is kAbortMeta.  The block's bits go to
// check_bits[b][c]; the decode ORs a sequence's chunks.  Page ids and expected
// tags are loaded for the whole chunk of the table row (in bounds of the row)
// while the length is still in flight, so the check costs two dependent loads.
__device__ __forceinline__ void check_block(const DecodeParams& p, int c, int b) {
  const int L = p.seq_lens[b];
  const int64_t row = (int64_t)b * p.max_pages;
  const bool tags_on = p.page_tags != nullptr;
  int pid[kCheckUnroll];
  uint32_t expected[kCheckUnroll];
#pragma unroll
  for (int u = 0; u < kCheckUnroll; ++u) {
    const int j = c * kCheckChunk + u * kBlockThreads + threadIdx.x;
    pid[u] = j < p.max_pages ? p.page_table[row + j] : 0;
    expected[u] = (tags_on && j < p.max_pages) ? p.expected_tags[row + j] : 0u;
  }
  const int max_tokens = p.max_pages << p.log2_page_size;
  uint32_t bits = 0;
  if (L < 1 || L > max_tokens) {
    bits = kAbortMeta;
  } else {
    const int n_pages = (L + (1 << p.log2_page_size) - 1) >> p.log2_page_size;
#pragma unroll
    for (int u = 0; u < kCheckUnroll; ++u) {
      const int j = c * kCheckChunk + u * kBlockThreads + threadIdx.x;
      if (j >= n_pages) continue;
      if (pid[u] < 0 || pid[u] >= p.num_pages)
        bits |= kAbortMeta;
      else if (tags_on && p.page_tags[pid[u]] != expected[u])
        bits |= kAbortTag;
    }
  }
  const int any_tag = __syncthreads_or((int)(bits & kAbortTag));
  const int any_meta = __syncthreads_or((int)(bits & kAbortMeta));
  if (threadIdx.x == 0)
    p.check_bits[(int64_t)b * p.check_chunks + c] = (uint8_t)((any_tag ? kAbortTag : 0u) | (any_meta ? kAbortMeta : 0u));
}

}  // namespace fp8kv
