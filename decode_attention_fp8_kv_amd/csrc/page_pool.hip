// Generation-tagged page pool on the device: the write side of the page-tag
// check.
//
// Every cache page carries a generation tag that changes whenever the page
// is handed to a new owner; readers compare it with the generation they
// recorded (source pages: "ترفندهای کلادفلر برای جا دادن مدل‌های غول‌پیکر تو
// GPU", third technique; "Tối ưu hóa mô hình AI quy mô lớn", section "Bảo vệ
// tính toàn vẹn của KV Cache").  The free pages are a stack of page ids in
// device memory with its count beside it, so allocation needs no host round
// trip.  Both operations are deterministic functions of their inputs:
//
//   alloc: requests are served in order of sequence while the running total
//          of valid requests fits (a request for zero pages is always
//          served); each popped page's tag is incremented and the new tag is
//          recorded as the sequence's expected tag for the slot.
//   free:  released sequences push their pages back in order of sequence,
//          then slot, while they fit in the stack; tags do not change.
//
// One block of 1024 threads does a whole call: the requests are scanned 1024
// at a time and the chunk's pages are spread over all threads (each thread
// finds the owner of its page by a binary search over the chunk's scan).
#include "common.hpp"
#include "internal.hpp"

namespace fp8kv {
namespace {

constexpr int kPoolThreads = 1024;
constexpr int kPoolWaves = kPoolThreads / 64;

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive scan of v over the block; *total receives the sum.
__device__ int64_t block_excl_scan(int64_t v, int64_t* sh, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t incl = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int64_t x = lane < kPoolWaves ? sh[lane] : 0;
    const int64_t xi = wave_incl_scan(x, lane);
    if (lane < kPoolWaves) sh[lane] = xi - x;
    if (lane == kPoolWaves - 1) sh[kPoolWaves] = xi;
  }
  __syncthreads();
  const int64_t r = incl - v + sh[wave];
  *total = sh[kPoolWaves];
  __syncthreads();
  return r;
}

// Last t in [0, n) with start[t] <= g (start is non-decreasing; start[0] <= g).
__device__ __forceinline__ int owner_of(const int64_t* start, int n, int64_t g) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void pool_init_kernel(int32_t* free_pages, int32_t* free_count, int32_t num_pages) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < num_pages) free_pages[i] = num_pages - 1 - (int32_t)i;  // pops come out 0, 1, 2, ...
  if (i == 0) *free_count = num_pages;
}

__global__ __launch_bounds__(kPoolThreads) void alloc_kernel(PoolParams p) {
  __shared__ int64_t sh[kPoolWaves + 1];
  __shared__ int64_t s_start[kPoolThreads];
  __shared__ int32_t s_cnt[kPoolThreads];
  __shared__ uint8_t s_served[kPoolThreads];
  __shared__ int64_t s_taken;
  const int tid = threadIdx.x;
  const int64_t F = min(max((int64_t)*p.free_count, (int64_t)0), (int64_t)p.num_pages);
  if (tid == 0) s_taken = 0;
  int64_t carry = 0;  // valid requests of the chunks before
  for (int c = 0; c < p.batch; c += kPoolThreads) {
    const int b = c + tid;
    const int64_t r = b < p.batch ? p.n_new[b] : 0;
    const int64_t cnt = b < p.batch ? p.page_counts[b] : 0;
    const bool valid = b < p.batch && r >= 0 && cnt >= 0 && cnt + r <= p.max_pages;
    int64_t chunk_total;
    const int64_t start = carry + block_excl_scan(valid ? r : 0, sh, &chunk_total);
    const bool served = valid && (r == 0 || start + r <= F);
    if (b < p.batch) p.status[b] = !valid ? 2 : served ? 0 : 1;
    s_start[tid] = start;
    s_cnt[tid] = (int32_t)cnt;
    s_served[tid] = served && r > 0;
    if (served && r > 0) atomicAdd((unsigned long long*)&s_taken, (unsigned long long)r);
    __syncthreads();
    const int n = min(kPoolThreads, p.batch - c);
    for (int64_t g = carry + tid; g < min(carry + chunk_total, F); g += kPoolThreads) {
      const int t = owner_of(s_start, n, g);
      if (!s_served[t]) continue;
      const int bb = c + t;
      const int slot = s_cnt[t] + (int)(g - s_start[t]);
      const int32_t page = p.free_pages[F - 1 - g];
      const int64_t at = (int64_t)bb * p.max_pages + slot;
      p.page_table[at] = page;
      if (page >= 0 && page < p.num_pages) {
        const uint32_t tag = p.page_tags[page] + 1u;
        p.page_tags[page] = tag;
        p.expected_tags[at] = tag;
      } else {
        p.expected_tags[at] = 0u;
      }
    }
    if (served) p.page_counts[b] = (int32_t)(cnt + r);
    carry += chunk_total;
    __syncthreads();
  }
  if (tid == 0) *p.free_count = (int32_t)(F - s_taken);
}

__global__ __launch_bounds__(kPoolThreads) void free_kernel(PoolParams p) {
  __shared__ int64_t sh[kPoolWaves + 1];
  __shared__ int64_t s_start[kPoolThreads];
  __shared__ uint8_t s_pushed[kPoolThreads];
  __shared__ int64_t s_count;
  const int tid = threadIdx.x;
  const int64_t F = min(max((int64_t)*p.free_count, (int64_t)0), (int64_t)p.num_pages);
  if (tid == 0) s_count = 0;
  int64_t carry = 0;  // pages of the valid released sequences of the chunks before
  for (int c = 0; c < p.batch; c += kPoolThreads) {
    const int b = c + tid;
    const bool rel = b < p.batch && p.release[b] != 0;
    const int64_t cnt = rel ? p.page_counts[b] : 0;
    const bool valid = rel && cnt >= 0 && cnt <= p.max_pages;
    int64_t chunk_total;
    const int64_t start = carry + block_excl_scan(valid ? cnt : 0, sh, &chunk_total);
    const bool pushed = valid && F + start + cnt <= p.num_pages;
    if (b < p.batch) p.status[b] = !rel ? 0 : !valid ? 2 : pushed ? 0 : 1;
    s_start[tid] = start;
    s_pushed[tid] = pushed;
    if (pushed && cnt > 0) atomicAdd((unsigned long long*)&s_count, (unsigned long long)cnt);
    __syncthreads();
    const int n = min(kPoolThreads, p.batch - c);
    for (int64_t g = carry + tid; g < carry + chunk_total; g += kPoolThreads) {
      const int t = owner_of(s_start, n, g);
      if (!s_pushed[t]) continue;
      p.free_pages[F + g] = p.page_table[(int64_t)(c + t) * p.max_pages + (g - s_start[t])];
    }
    __syncthreads();  // every page of the chunk is read before its count is cleared
    if (pushed) p.page_counts[b] = 0;
    carry += chunk_total;
    __syncthreads();
  }
  if (tid == 0) *p.free_count = (int32_t)(F + s_count);
}

}  // namespace

hipError_t launch_pool_init(int32_t* free_pages, int32_t* free_count, int32_t num_pages, hipStream_t stream) {
  hipLaunchKernelGGL(pool_init_kernel, dim3((unsigned)((num_pages + 255) / 256)), dim3(256), 0, stream, free_pages,
                     free_count, num_pages);
  return hipGetLastError();
}

hipError_t launch_pool_alloc(const PoolParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(alloc_kernel, dim3(1), dim3(kPoolThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_pool_free(const PoolParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(free_kernel, dim3(1), dim3(kPoolThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8kv
