// page_alloc.hip -- device-resident page allocator and tag tracker: a stack of free physical page
// ids plus one live tag per page, changed whenever the page is handed out again, so that a request
// still holding the old (page, tag) pair fails kv_tag_verify.  Allocation and release are each one
// single-workgroup kernel: the workgroup reads the stack top once, orders the work with a
// workgroup-wide scan and writes the new top last, so the result is deterministic and no other
// workgroup ever sees a half-updated stack.
#include "common.hpp"

namespace dapf8 {

namespace {

constexpr int kAllocThreads = 1024;

// Inclusive scan of v over the workgroup (1024 threads, 16 waves): wave scans with shuffles, then
// a scan of the 16 wave totals.  sums needs 16 values of LDS.  64-bit: a batch of requests may ask
// for more than 2^31 pages in total, and a wrapped prefix would grant pages nobody has.
__device__ __forceinline__ int64_t block_inclusive_scan(int64_t v, int64_t* sums, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) sums[wave] = v;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < kAllocThreads / 64; ++w) {
    const int64_t s = sums[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();  // sums may be rewritten by the next call
  total = all;
  return v + before;
}

}  // namespace

__global__ void pages_init_kernel(int32_t* __restrict__ free_list, int32_t* __restrict__ free_count,
                                  uint32_t* __restrict__ live_tags, int32_t num_pages) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < num_pages) {
    free_list[i] = num_pages - 1 - i;  // the top of the stack holds page 0
    if (live_tags) live_tags[i] = 0u;
  }
  if (i == 0) *free_count = num_pages;
}

// Pop for requests in order.  Request b is valid when counts[b] >= 0 and its slot range
// [first_slot[b], first_slot[b] + counts[b]) lies inside its page-table row; it is granted when it is
// valid and the pages of every valid request up to and including it fit on the stack.  The granted
// requests are therefore the valid ones before the first valid request that does not fit; their
// pages, in request order, are the ones nearest the top of the stack.
__global__ __launch_bounds__(kAllocThreads) void pages_alloc_kernel(
    int32_t* __restrict__ free_list, int32_t* __restrict__ free_count, uint32_t* __restrict__ live_tags,
    int32_t num_pages, const int32_t* __restrict__ counts, const int32_t* __restrict__ first_slot, int32_t B,
    int32_t* __restrict__ page_table, uint32_t* __restrict__ expected_tags, int32_t pt_stride,
    uint8_t* __restrict__ granted) {
  __shared__ int excl[kMaxAllocRequests];  // exclusive prefix of the valid requests' page counts,
                                            // saturated at the stack top (exact for granted ones)
  __shared__ int64_t sums[kAllocThreads / 64];
  __shared__ int s_top, s_used;
  const int t = threadIdx.x;
  if (t == 0) {
    s_top = min(max(*free_count, 0), num_pages);
    s_used = 0;
  }
  __syncthreads();
  const int top = s_top;
  int64_t carry = 0;
  for (int base = 0; base < B; base += kAllocThreads) {
    const int b = base + t;
    int64_t c = 0;
    bool valid = false;
    if (b < B) {
      const int n = counts[b], f = first_slot[b];
      valid = n >= 0 && f >= 0 && (int64_t)f + n <= pt_stride;
      c = valid ? n : 0;
    }
    int64_t total;
    const int64_t incl = block_inclusive_scan(c, sums, total);
    if (b < B) {
      const bool ok = valid && carry + incl <= top;
      granted[b] = ok ? 1 : 0;
      // non-decreasing in b; below top wherever a granted page can be looked up
      excl[b] = (int)min(carry + incl - c, (int64_t)top);
      if (ok && c > 0) atomicMax(&s_used, (int)(carry + incl));  // LDS: pages handed out in total
    }
    carry += total;
  }
  __syncthreads();
  const int used = s_used;
  // granted page g (0 <= g < used) belongs to the request b with excl[b] <= g < excl[b + 1]:
  // the largest b with excl[b] <= g (binary search; excl never decreases)
  for (int g = t; g < used; g += kAllocThreads) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (excl[mid] <= g)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int b = lo, j = g - excl[b];
    const int page = free_list[top - 1 - g];
    const size_t at = (size_t)b * pt_stride + first_slot[b] + j;
    page_table[at] = page;
    if (live_tags) {
      uint32_t tag = 0u;
      if (page >= 0 && page < num_pages) {
        tag = live_tags[page] + 1u;  // a generation counter: wraps, compared for equality only
        live_tags[page] = tag;
      }
      if (expected_tags) expected_tags[at] = tag;
    }
  }
  __syncthreads();
  if (t == 0) *free_count = top - used;
}

// Push pages in order; ids outside [0, num_pages) and ids beyond the stack's room are rejected.
__global__ __launch_bounds__(kAllocThreads) void pages_free_kernel(int32_t* __restrict__ free_list,
                                                                    int32_t* __restrict__ free_count,
                                                                    const int32_t* __restrict__ pages, int32_t n,
                                                                    int32_t num_pages, int32_t* __restrict__ status) {
  __shared__ int64_t sums[kAllocThreads / 64];
  __shared__ int s_top;
  const int t = threadIdx.x;
  if (t == 0) s_top = min(max(*free_count, 0), num_pages);
  __syncthreads();
  const int top = s_top;
  int64_t pushed = 0;
  for (int base = 0; base < n; base += kAllocThreads) {
    const int i = base + t;
    const int id = i < n ? pages[i] : -1;
    const int64_t v = (id >= 0 && id < num_pages) ? 1 : 0;
    int64_t total;
    const int64_t incl = block_inclusive_scan(v, sums, total);
    const int64_t at = top + pushed + incl - 1;
    if (v && at < num_pages) free_list[at] = id;
    pushed += total;
  }
  __syncthreads();
  if (t == 0) {
    const int room = num_pages - top;
    const int kept = (int)min(pushed, (int64_t)room);
    *free_count = top + kept;
    status[0] = kept;
    status[1] = n - kept;
  }
}

int launch_pages_init(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages, hipStream_t s) {
  hipLaunchKernelGGL(pages_init_kernel, dim3((unsigned)((num_pages + 255) / 256)), dim3(256), 0, s, free_list,
                     free_count, live_tags, num_pages);
  return check_launch("kv_pages_init");
}

int launch_pages_alloc(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages,
                       const int32_t* counts, const int32_t* first_slot, int32_t B, int32_t* page_table,
                       uint32_t* expected_tags, int32_t pt_stride, uint8_t* granted, hipStream_t s) {
  hipLaunchKernelGGL(pages_alloc_kernel, dim3(1), dim3(kAllocThreads), 0, s, free_list, free_count, live_tags,
                     num_pages, counts, first_slot, B, page_table, expected_tags, pt_stride, granted);
  return check_launch("kv_pages_alloc");
}

int launch_pages_free(int32_t* free_list, int32_t* free_count, const int32_t* pages, int32_t n, int32_t num_pages,
                      int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(pages_free_kernel, dim3(1), dim3(kAllocThreads), 0, s, free_list, free_count, pages, n,
                     num_pages, status);
  return check_launch("kv_pages_free");
}

}  // namespace dapf8
