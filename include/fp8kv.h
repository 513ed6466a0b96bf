/*
 * fp8kv.h -- C ABI of the MI355X (gfx950) paged decode-attention library
 * over an FP8 e4m3 KV cache with per-page generation tags.
 *
 * The method: a decode step's attention reads a paged KV cache that is held
 * as 8-bit e4m3 floating point instead of BF16, which halves its size, and
 * converts values as it reads them (page "Cloudflare tối ưu hóa Kimi và GLM
 * trên Workers AI", section "Lượng tử hóa KV cache"; page "更小、更快、更安全
 * ：大规模运行Kimi和GLM", section "量化 KV 缓存").  Every cache page of the
 * shared pool carries a tag that changes on each reallocation; the tag is
 * compared before the page is read and a mismatch aborts the request rather
 * than returning wrong data; the check is optional (page "ترفندهای کلادفلر
 * برای جا دادن مدل‌های غول‌پیکر تو GPU", third technique; page "Tối ưu hóa
 * mô hình AI quy mô lớn", section "Bảo vệ tính toàn vẹn của KV Cache").  The
 * e4m3 bit layout is the OCP OFP8 E4M3 encoding (bias 7, no infinities,
 * NaN = S.1111.111, largest finite magnitude 448).
 *
 * Conventions for every call below
 * --------------------------------
 *  - Pointers are DEVICE pointers (memory on the current HIP device) unless
 *    stated otherwise; the caller owns all memory, including the workspace.
 *  - BF16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous on that stream: they enqueue kernels and return.
 *    They never allocate memory, never synchronize and never read device
 *    memory from the host.
 *  - Argument checking happens on the host before anything is launched; a
 *    negative status means nothing was launched and no memory was touched.
 *  - Conditions found in device data (stale tags, bad page ids, bad lengths)
 *    are results, not errors: they are reported in `abort_flags`.
 *  - Calls are reentrant; different streams may run calls concurrently as
 *    long as they do not share output or workspace buffers.
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8KV_ABI_VERSION 2

/* KV cache element types. */
#define FP8KV_KV_FP8_E4M3 0 /* 1 byte per element, value = e4m3(code) * scale */
#define FP8KV_KV_BF16 1     /* 2 bytes per element, raw BF16, no scale       */

/* Status codes (return values). */
#define FP8KV_OK 0
#define FP8KV_ERR_NULL (-1)        /* a required pointer is NULL                      */
#define FP8KV_ERR_SHAPE (-2)       /* a size is <= 0, or heads do not divide          */
#define FP8KV_ERR_UNSUPPORTED (-3) /* head_dim / page_size / group / dtype not built  */
#define FP8KV_ERR_WORKSPACE (-4)   /* workspace smaller than the size function says   */
#define FP8KV_ERR_SCALE (-5)       /* a scale is not finite or not > 0                */
#define FP8KV_ERR_TAGS (-6)        /* exactly one of page_tags / expected_tags given  */
#define FP8KV_ERR_LAUNCH (-7)      /* the HIP runtime rejected a launch               */
#define FP8KV_ERR_ALIGN (-8)       /* q/k_new/v_new/caches not 16-byte aligned, out not
                                      8-byte aligned, or workspace not 256-byte aligned */
#define FP8KV_ERR_SCRATCH (-9)     /* paged_decode_attn_noalloc: the sizes need more
                                      workspace than FP8KV_NOALLOC_SCRATCH_BYTES       */

/* Abort-flag bits written per sequence by paged_decode_attn. */
#define FP8KV_ABORT_TAG_MISMATCH 1u /* a used page's tag differs from the expected one */
#define FP8KV_ABORT_BAD_METADATA 2u /* seq_len outside [1, max_pages*page_size], or a
                                       used page id outside [0, num_pages)            */

/* Supported shapes (kernels are compiled for these). */
#define FP8KV_MAX_GROUP 16 /* num_q_heads / num_kv_heads                      */
/* head_dim in {64, 128}; page_size a power of two in [16, 256].               */

/* ABI version of the loaded library (FP8KV_ABI_VERSION it was built with). */
int fp8kv_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* fp8kv_status_string(int status);

/* Text of the last HIP runtime error seen by this thread ("" if none). */
const char* fp8kv_last_hip_error(void);

/*
 * kv_quant_append -- write new K/V rows into the paged caches.
 *
 * The decode pool keeps its KV cache as e4m3 bytes instead of BF16, so each
 * new token's K and V are converted once as they enter the cache ("Cloudflare
 * tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa KV cache";
 * "更小、更快、更安全：大规模运行Kimi和GLM", section "量化 KV 缓存").
 *
 * Row r (of n_rows) belongs to sequence row_seq[r] at token position
 * row_pos[r]; it is written to physical page
 *     page = page_table[row_seq[r] * max_pages + row_pos[r] / page_size]
 * at slot row_pos[r] % page_size, for every KV head h and element d:
 *     cache[((page * num_kv_heads + h) * page_size + slot) * head_dim + d].
 *
 * kv_dtype FP8KV_KV_FP8_E4M3: each element x becomes the e4m3 code of the
 *   fp32 quotient fp32(x) / scale (an IEEE, correctly rounded fp32 division),
 *   rounded to the nearest e4m3 value with ties to the even code, saturating
 *   at +-448 (+-inf too); every NaN becomes 0x7F; K uses
 *   k_scale and V uses v_scale (one fp32 scale per tensor).  Dequantized
 *   values are code * scale.
 * kv_dtype FP8KV_KV_BF16: the BF16 bits are copied; the scales are ignored.
 *
 *   k_new, v_new   uint16 BF16 [n_rows][num_kv_heads][head_dim]
 *   row_seq        int32 [n_rows]   sequence index of each row
 *   row_pos        int32 [n_rows]   token position of each row
 *   page_table     int32 [batch][max_pages]
 *   k_cache,
 *   v_cache        [num_pages][num_kv_heads][page_size][head_dim] of
 *                  uint8 (FP8) or uint16 (BF16)
 *   k_scale,
 *   v_scale        HOST fp32 values, finite and > 0 (FP8 mode only)
 *
 * A row whose sequence index is outside [0, batch), whose position is
 * outside [0, max_pages*page_size) or whose page id is outside
 * [0, num_pages) is skipped: nothing is ever written outside the pools.
 * Rows aimed at the same slot are a caller error (the winner is unspecified).
 * n_rows == 0 is valid and launches nothing.  num_kv_heads is at most 65535
 * (FP8KV_ERR_SHAPE beyond).
 */
int kv_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                    const int32_t* row_seq, const int32_t* row_pos,
                    const int32_t* page_table, int32_t batch, int32_t max_pages,
                    float k_scale, float v_scale,
                    void* k_cache, void* v_cache, int32_t num_pages,
                    int32_t n_rows, int32_t num_kv_heads, int32_t head_dim,
                    int32_t page_size, int32_t kv_dtype, void* stream);

/*
 * kv_quant_append_checked -- kv_quant_append that writes a row only while
 * its page still belongs to the generation the sequence recorded: a row is
 * written iff page_tags[p] == expected_tags[seq * max_pages + pos /
 * page_size] for its page p.  Same arguments as kv_quant_append plus
 *
 *   page_tags      uint32 [num_pages]              current page generations
 *   expected_tags  uint32 [batch][max_pages]       generations the sequences
 *                  recorded (written by page_alloc)
 *   row_status     uint8 [n_rows] (written): 0 written, 1 tag mismatch (not
 *                  written), 2 destination out of range (not written)
 *
 * For the writer side of the tag check: an append through a stale page
 * table (its pages freed and handed to another sequence) is refused instead
 * of overwriting the new owner's data ("ترفندهای کلادفلر برای جا دادن
 * مدل‌های غول‌پیکر تو GPU", third technique).  Errors: as kv_quant_append;
 * FP8KV_ERR_NULL if a tag or status pointer is NULL.
 */
int kv_quant_append_checked(const uint16_t* k_new, const uint16_t* v_new,
                            const int32_t* row_seq, const int32_t* row_pos,
                            const int32_t* page_table, int32_t batch, int32_t max_pages,
                            float k_scale, float v_scale,
                            void* k_cache, void* v_cache, int32_t num_pages,
                            int32_t n_rows, int32_t num_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t kv_dtype,
                            const uint32_t* page_tags, const uint32_t* expected_tags,
                            uint8_t* row_status, void* stream);

/*
 * Prefill -> decode hand-off ("Cloudflare tối ưu hóa Kimi và GLM trên
 * Workers AI", section "Lượng tử hóa KV cache": prefill keeps BF16, decode
 * reads the FP8 cache, so a prefill's K/V are converted once when handed
 * over).  Reading of the scale rule (the pages give none): one fp32 scale
 * per tensor that maps the largest finite magnitude onto e4m3's 448.
 *
 * kv_absmax_scale -- out[0] = max |x| over the finite elements of the BF16
 * tensor x [n] (NaNs and infinities ignored; 0 if there are none), out[1] =
 * out[0] / 448 (IEEE fp32 division), or 1 if out[0] is 0.  out is a device
 * buffer of 2 floats; work is device scratch of FP8KV_AMAX_WORK_FLOATS
 * floats whose contents do not matter before a call and are undefined after
 * it (no initialisation needed).  Calls sharing a work or out buffer must be
 * ordered (same stream).  x is 16-byte aligned, out and work 4-byte
 * aligned; all three are owned by the caller.  Two kernels on `stream`.
 * Errors: FP8KV_ERR_SHAPE (n < 0), FP8KV_ERR_NULL, FP8KV_ERR_ALIGN.
 *
 * kv_absmax_scale_kv -- kv_absmax_scale of a K and a V tensor of n
 * elements each in one call: out[0], out[1] for k and out[2], out[3] for v
 * (out is 4 floats), work is 2 * FP8KV_AMAX_WORK_FLOATS floats; each pair
 * is bit-identical to what kv_absmax_scale gives for that tensor alone.  Two
 * kernels on `stream` instead of four, which is what a prefill hand-off
 * needs (both scales before the conversion).  Errors as kv_absmax_scale.
 *
 * kv_quant_append_dscale -- kv_quant_append into an FP8 cache with the
 * scales read from device memory (e.g. out + 1 of kv_absmax_scale), so the
 * hand-off needs no host round trip.  A scale that is not finite and
 * positive writes nothing (there is no host check to reject it).  Errors as
 * kv_quant_append (no FP8KV_ERR_SCALE), plus FP8KV_ERR_NULL / _ALIGN for the
 * scale pointers (4-byte aligned).
 */
#define FP8KV_AMAX_WORK_FLOATS 512
int kv_absmax_scale(const uint16_t* x, int64_t n, float* out, float* work, void* stream);
int kv_absmax_scale_kv(const uint16_t* k, const uint16_t* v, int64_t n, float* out, float* work,
                       void* stream);
int kv_quant_append_dscale(const uint16_t* k_new, const uint16_t* v_new,
                           const int32_t* row_seq, const int32_t* row_pos,
                           const int32_t* page_table, int32_t batch, int32_t max_pages,
                           const float* k_scale_dev, const float* v_scale_dev,
                           void* k_cache, void* v_cache, int32_t num_pages,
                           int32_t n_rows, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, void* stream);

/*
 * Generation-tagged page pool ("ترفندهای کلادفلر برای جا دادن مدل‌های
 * غول‌پیکر تو GPU", third technique; "Tối ưu hóa mô hình AI quy mô lớn",
 * section "Bảo vệ tính toàn vẹn của KV Cache": a page's tag changes whenever
 * the page is handed to a new owner).  All state lives in device memory,
 * owned by the caller; every call is one kernel on `stream`, deterministic.
 *
 *   free_pages     int32 [num_pages]  stack of free page ids (top = the
 *                  entry at free_count - 1)
 *   free_count     int32 [1]          number of free pages
 *   page_counts    int32 [batch]      pages each sequence holds (its first
 *                  page_counts[b] table entries)
 *   page_table     int32 [batch][max_pages]
 *   expected_tags  uint32 [batch][max_pages]
 *   page_tags      uint32 [num_pages]
 *
 * page_pool_init: every page free, stacked so that pops return 0, 1, 2, ...
 * (tags are left as they are).
 *
 * page_alloc: sequence b asks for n_new[b] more pages.  Valid iff n_new[b]
 * >= 0 and 0 <= page_counts[b] <= page_counts[b] + n_new[b] <= max_pages
 * (else status 2, nothing changes for b).  Valid requests are served in
 * order of b while their running total fits: b is served iff (sum of the
 * valid requests before b) + n_new[b] <= free_count (else status 1); a
 * request for zero pages is always served (status 0).  A served request
 * pops its pages in order into its next table slots; each page's tag is
 * incremented (mod 2^32) and the new value recorded in expected_tags.  A
 * popped id outside [0, num_pages) (a corrupt stack) is recorded as is with
 * expected tag 0 and no tag write -- the decode's page check flags it.
 *
 * page_free: every sequence with release[b] != 0 pushes its pages back in
 * order of b, then slot, and then holds 0 pages (status 0); page_counts[b]
 * outside [0, max_pages] is status 2; pushes are served in order while they
 * fit in the stack (else status 1), so a double free cannot overflow it.
 * Tags do not change on free; the released rows of page_table and
 * expected_tags are left as they were, so a reader still using them fails
 * the tag check once a page has a new owner.  status[b] = 0 for sequences
 * not released.
 *
 * Errors: FP8KV_ERR_SHAPE (batch, max_pages or num_pages <= 0),
 * FP8KV_ERR_NULL; device-side conditions are status codes, never errors.
 * Calls that share a pool must be ordered (same stream).
 */
int page_pool_init(int32_t* free_pages, int32_t* free_count, int32_t num_pages, void* stream);
int page_alloc(const int32_t* n_new, int32_t* page_counts, int32_t* page_table,
               uint32_t* expected_tags, uint32_t* page_tags,
               int32_t* free_pages, int32_t* free_count, uint8_t* status,
               int32_t batch, int32_t max_pages, int32_t num_pages, void* stream);
int page_free(const uint8_t* release, int32_t* page_counts, const int32_t* page_table,
              int32_t* free_pages, int32_t* free_count, uint8_t* status,
              int32_t batch, int32_t max_pages, int32_t num_pages, void* stream);

/*
 * paged_decode_attn_workspace_size -- bytes of device workspace that
 * paged_decode_attn needs for these sizes (a multiple of 256; mostly
 * 2 * 4 * num_blocks partial slots of 4 * G * (head_dim + 2) bytes each,
 * G = num_q_heads / num_kv_heads: up to ~17 MiB with the automatic grid).
 * num_blocks has the meaning it has in paged_decode_attn.  Returns 0 if the
 * sizes are invalid.
 */
size_t paged_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t page_size, int32_t max_pages,
                                        int32_t num_blocks);

/*
 * paged_decode_attn -- one decode step of attention for a batch of
 * sequences, one query token each, over a paged FP8 (or BF16) KV cache.
 *
 * The attention reads the e4m3 cache and converts values as it reads them
 * ("Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section "Lượng tử hóa
 * KV cache"; "更小、更快、更安全：大规模运行Kimi和GLM", section "量化 KV 缓存");
 * each page's generation tag is compared before the page is used and a
 * mismatch aborts the request instead of returning wrong data ("ترفندهای
 * کلادفلر برای جا دادن مدل‌های غول‌پیکر تو GPU", third technique; "Tối ưu hóa
 * mô hình AI quy mô lớn", section "Bảo vệ tính toàn vẹn của KV Cache").
 *
 * For sequence b with L = seq_lens[b] cached tokens and query head h
 * (group size G = num_q_heads / num_kv_heads, KV head g = h / G):
 *   k_t  = dequantized K row of token t (t < L) of KV head g,
 *   s_t  = softmax_scale * <q[b][h], k_t>,
 *   out[b][h] = sum_t softmax(s)_t * v_t     (rounded to BF16, nearest-even),
 * where token t lives in page page_table[b*max_pages + t/page_size], slot
 * t % page_size.  FP8 values are code * k_scale (K) and code * v_scale (V);
 * BF16 values are used as stored and the scales are ignored.
 *
 *   q              uint16 BF16 [batch][num_q_heads][head_dim]
 *   k_cache,
 *   v_cache        [num_pages][num_kv_heads][page_size][head_dim]
 *   page_table     int32 [batch][max_pages]; only the entries of the used
 *                  pages (slots j < ceil(seq_lens[b] / page_size)) are used as
 *                  page ids (with tags on, the page check also loads the
 *                  other entries of the row, without using them)
 *   seq_lens       int32 [batch]
 *   page_tags      uint32 [num_pages]              current page generations
 *   expected_tags  uint32 [batch][max_pages]       generations each sequence
 *                  recorded; both NULL = tag check off (the default), both
 *                  non-NULL = on, one NULL = FP8KV_ERR_TAGS
 *   out            uint16 BF16 [batch][num_q_heads][head_dim], 8-byte aligned
 *   abort_flags    uint8 [batch]; always written: 0, or an OR of the
 *                  FP8KV_ABORT_* bits
 *   workspace      device buffer of at least
 *                  paged_decode_attn_workspace_size(...) bytes, 256-byte
 *                  aligned; its contents need no initialization (each call
 *                  writes what it reads).  It holds per-call partial
 *                  results, so calls sharing a workspace must be ordered
 *                  (same stream).
 *
 *   num_blocks     0 = choose automatically (one workgroup per CU, fewer
 *                  for small batches); n > 0 = use n workgroups of 4 waves
 *                  (at most 65535).  The batch's work -- every (sequence,
 *                  KV head, 64-token tile) -- is cut into min(4n, tiles)
 *                  equal contiguous shares, one per wave, so long sequences
 *                  are split across waves (flash-decoding) and merged
 *                  exactly; the result does not depend on n beyond
 *                  floating-point rounding, and repeated calls with the same
 *                  inputs and n give bit-identical outputs.
 *
 * Kernels enqueued on the stream: with tags on, a page check (one block per
 * 1024 page-table slots of a sequence), then the decode kernel, which reads
 * K/V only of the sequences that passed (an aborted sequence costs 12 bytes
 * per page) and writes abort_flags, then a merge kernel that combines the
 * partial results of segments split between waves -- three kernels.  With
 * tags off there is no page check: the decode checks the lengths and the
 * page ids of each round of pages before reading any of them -- two kernels.
 *
 * Tag rule: for every page slot j < ceil(L / page_size) (the partial last
 * page included), the page id p = page_table[b*max_pages + j] must lie in
 * [0, num_pages) (else bit FP8KV_ABORT_BAD_METADATA) and, when tags are on,
 * page_tags[p] must equal expected_tags[b*max_pages + j] (else bit
 * FP8KV_ABORT_TAG_MISMATCH).  Pages are checked before their contents are
 * used.  When abort_flags[b] != 0, out[b] is NOT WRITTEN (left as it was).
 * The caches are never written.  out must not alias q.
 *
 * Errors (nothing launched): FP8KV_ERR_UNSUPPORTED (kv_dtype, head_dim,
 * page_size, group > FP8KV_MAX_GROUP), FP8KV_ERR_SHAPE (a size <= 0,
 * num_q_heads not a multiple of num_kv_heads, batch or num_kv_heads above
 * 65535, max_pages * page_size above INT32_MAX), FP8KV_ERR_NULL,
 * FP8KV_ERR_TAGS, FP8KV_ERR_SCALE (FP8 scales not finite and positive,
 * softmax_scale not finite), FP8KV_ERR_ALIGN, FP8KV_ERR_WORKSPACE,
 * FP8KV_ERR_LAUNCH.
 */
int paged_decode_attn(const uint16_t* q, const void* k_cache, const void* v_cache,
                      int32_t kv_dtype, float k_scale, float v_scale,
                      const int32_t* page_table, int32_t max_pages,
                      const int32_t* seq_lens,
                      const uint32_t* page_tags, const uint32_t* expected_tags,
                      uint16_t* out, uint8_t* abort_flags,
                      void* workspace, size_t workspace_bytes,
                      int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                      float softmax_scale, int32_t num_blocks, void* stream);

/*
 * paged_decode_attn_noalloc -- paged_decode_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments and results as
 * paged_decode_attn without the workspace: the call uses the library's own
 * scratch, a fixed device array of FP8KV_NOALLOC_SCRATCH_BYTES (32 MiB) that
 * every device the library runs on holds until the process ends.  The call
 * allocates and frees nothing (no hipMalloc, no allocating library routine);
 * the first call on a device looks up that device's scratch address once.
 *
 * Sizes whose workspace (paged_decode_attn_workspace_size) exceeds the
 * scratch are rejected with FP8KV_ERR_SCRATCH before anything is launched:
 * with the automatic grid the decode needs at most ~17 MiB for groups up to
 * 16 and head_dim 128 on a 256-CU device, plus a few bytes per sequence.
 * The scratch needs no initialization (every call writes what it reads)
 * and keeps the last call's contents.  Every call on one device shares that
 * device's scratch: calls that overlap on one device -- on different
 * streams, or from different host threads without ordering -- race, so
 * order them (one stream, or events between streams).
 *
 * Errors: those of paged_decode_attn (never FP8KV_ERR_WORKSPACE), plus
 * FP8KV_ERR_SCRATCH; FP8KV_ERR_LAUNCH if the scratch address cannot be
 * looked up.
 */
#define FP8KV_NOALLOC_SCRATCH_BYTES (32u << 20)
int paged_decode_attn_noalloc(const uint16_t* q, const void* k_cache, const void* v_cache,
                              int32_t kv_dtype, float k_scale, float v_scale,
                              const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens,
                              const uint32_t* page_tags, const uint32_t* expected_tags,
                              uint16_t* out, uint8_t* abort_flags,
                              int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t num_pages,
                              float softmax_scale, int32_t num_blocks, void* stream);

/*
 * paged_decode_step -- one whole decode step: kv_quant_append of the step's
 * new rows (k_new, v_new, row_seq, row_pos, n_rows; n_rows may be 0)
 * followed by paged_decode_attn, on the same stream, with every argument
 * meaning what it means there (the append uses page_table, batch,
 * max_pages, the caches, the scales and kv_dtype of the decode).  The
 * results are bit-identical to those two calls made in that order.
 *
 * The difference is the launches: with tags on, the page check runs in the
 * append's launch, in blocks of its own beside the append's (the append
 * writes only cache bytes, the check reads only the page table, lengths
 * and tags), so a step is three kernels -- append + page check, decode,
 * merge -- where the two calls make four; with tags off, also three
 * (append, decode, merge).  The tag check then costs no launch of its own,
 * which is how a serving loop would run it when tags are on (the pages
 * give its cost as under 1% of throughput and p95 latency: "ترفندهای
 * کلادفلر برای جا دادن مدل‌های غول‌پیکر تو GPU", third technique).
 *
 *   decode_begin_event,
 *   decode_end_event   optional hipEvent_t handles (as void*; NULL = none):
 *                  recorded on `stream` right before the decode kernel and
 *                  right after it (before the merge), so a caller can time
 *                  the decode kernel alone.
 *
 * Errors: those of paged_decode_attn, then those of kv_quant_append (the
 * append's pointers are checked only when n_rows > 0).  Nothing is
 * launched on an error.
 */
int paged_decode_step(const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* row_seq, const int32_t* row_pos, int32_t n_rows,
                      const uint16_t* q, void* k_cache, void* v_cache,
                      int32_t kv_dtype, float k_scale, float v_scale,
                      const int32_t* page_table, int32_t max_pages,
                      const int32_t* seq_lens,
                      const uint32_t* page_tags, const uint32_t* expected_tags,
                      uint16_t* out, uint8_t* abort_flags,
                      void* workspace, size_t workspace_bytes,
                      int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                      float softmax_scale, int32_t num_blocks,
                      void* decode_begin_event, void* decode_end_event, void* stream);

/*
 * paged_decode_attn_path -- which kernel family paged_decode_attn uses for a
 * GQA group size: 1 = MFMA (groups of 5..16 query heads per KV head fill a
 * 16-column matrix-core tile enough to be a dense contraction), 0 = VALU
 * (groups of 1..4).  -1 for invalid sizes.  Setting FP8KV_FORCE_PATH=mfma
 * (any group) or =valu (groups up to 4) in the environment overrides the
 * choice, so tests can cross-check the two families on one shape.
 */
int paged_decode_attn_path(int32_t num_q_heads, int32_t num_kv_heads);

/*
 * INT4 weight-only decode GEMV ("ترفندهای کلادفلر برای جا دادن مدل‌های
 * غول‌پیکر تو GPU", the second technique; "更小、更快、更安全：大规模运行Kimi和
 * GLM", section "压缩模型权重": weights stored as 4-bit integers, which
 * decode streams at half the bytes of FP8 and unpacks before the multiply).
 *
 * Weights use a tile layout built for the GEMV's loads; int4_pack_weights
 * converts the common row layout into it.  Np = 16 * ceil(n / 16), G = k / 128.
 *
 *   row layout   codes uint32 [n][k/8]: word j of row r holds the signed
 *                two's-complement 4-bit codes of k = 8j + i in nibble i
 *                (bits 4i..4i+3); scales bf16 [n][G], one per 128 weights
 *                of a row (no zero point)
 *   tile layout  codes uint32 [Np/16][G][16][16]: tile t, group g, row
 *                r = n - 16t, word j holds k = 128g + 8j .. +7, nibble i
 *                holding k = 128g + 8j + 2i for i < 4 and 128g + 8j +
 *                2(i-4) + 1 for i >= 4; scales bf16 [Np/16][G][16].  Rows
 *                n..Np-1 are padding (int4_pack_weights writes code 0 and
 *                scale 0 there; int4_gemv never uses them for an output row
 *                < n).
 *
 * int4_pack_weights -- row layout (w_rows, s_rows) -> tile layout (w_tiles,
 * s_tiles).  n >= 1, k a positive multiple of 128; w_rows 4-byte aligned,
 * w_tiles 16-byte aligned, scales 2-byte aligned; outputs must not overlap
 * the inputs.  One kernel on `stream`, bit-exact permutation of the codes.
 * Errors: FP8KV_ERR_SHAPE, FP8KV_ERR_NULL, FP8KV_ERR_ALIGN.
 *
 * int4_gemv -- y[m][n] = sum_k x[m][k] * q[n][k] * s[n][k / 128], rounded
 * once to BF16 (nearest-even) from an fp32 evaluation.
 *
 *   x        bf16 [m][k]         activations, 16-byte aligned
 *   w_tiles  tile layout codes   16-byte aligned
 *   s_tiles  tile layout scales  2-byte aligned
 *   y        bf16 [m][n]         output, 2-byte aligned, must not alias the
 *                                inputs
 *
 * 1 <= m <= FP8KV_INT4_MAX_M, n >= 1, k a positive multiple of 128.  All
 * buffers are device memory owned by the caller; one kernel on `stream`,
 * nothing allocated, the result is deterministic.  Errors: FP8KV_ERR_SHAPE,
 * FP8KV_ERR_NULL, FP8KV_ERR_ALIGN (nothing is launched).
 */
#define FP8KV_INT4_GROUP 128
#define FP8KV_INT4_MAX_M 64
int int4_pack_weights(const uint32_t* w_rows, const uint16_t* s_rows, uint32_t* w_tiles,
                      uint16_t* s_tiles, int32_t n, int32_t k, void* stream);
int int4_gemv(const uint16_t* x, const uint32_t* w_tiles, const uint16_t* s_tiles, uint16_t* y,
              int32_t m, int32_t n, int32_t k, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_H */
