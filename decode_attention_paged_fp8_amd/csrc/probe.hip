// probe.hip -- a plain read-only streaming kernel: the attainable HBM read rate that the decode
// kernels are measured against (next to the 8 TB/s HBM3E specification).  It moves data and does
// nothing else: every byte of the chosen blocks is read once with 16-byte non-temporal loads (the
// load type the attention kernels use) and folded into an XOR so the loads cannot be dropped.
//
// Two access patterns: contiguous (block_ids == NULL: the buffer front to back) and scattered
// blocks (block i at buf + block_ids[i] * block_bytes), the page-block pattern of a paged cache.
// Persistent grid of `waves` wavefronts; wave w reads blocks w, w + waves, ... (a 64-lane wave
// reads 1 KiB per load instruction, four instructions in flight per block step).
#include "common.hpp"

namespace dapf8 {

typedef uint32_t p32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const uint8_t* __restrict__ buf, const int32_t* __restrict__ ids,
                                                         int64_t n_blocks, int32_t block_bytes,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int per = block_bytes >> 10;  // 1 KiB wave loads per block
  p32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = wave; i < n_blocks; i += waves) {
    const int64_t blk = ids ? (int64_t)ids[i] : i;
    const p32x4* p = reinterpret_cast<const p32x4*>(buf + blk * block_bytes) + lane;
    int j = 0;
    for (; j + 4 <= per; j += 4) {  // four loads in flight per step
      const p32x4 a = __builtin_nontemporal_load(p + 64 * j);
      const p32x4 b = __builtin_nontemporal_load(p + 64 * (j + 1));
      const p32x4 c = __builtin_nontemporal_load(p + 64 * (j + 2));
      const p32x4 d = __builtin_nontemporal_load(p + 64 * (j + 3));
      acc ^= (a ^ b) ^ (c ^ d);
    }
    for (; j < per; ++j) acc ^= __builtin_nontemporal_load(p + 64 * j);
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// Read-write streaming probe: the attainable rate of a stream that reads two bytes for every byte it
// writes (the byte mix of a BF16 -> FP8 page transcode).  Each thread step reads 32 contiguous bytes
// (two 16-byte non-temporal loads) and writes their 16-byte XOR fold (one non-temporal store);
// persistent grid, unit i at src + 32 i and dst + 16 i.
__global__ __launch_bounds__(256) void copy_probe_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                         int64_t n_units) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < n_units; i0 += 4 * stride) {
    p32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // four units in flight
      const int64_t i = min(i0 + u * stride, n_units - 1);
      a[u] = __builtin_nontemporal_load(reinterpret_cast<const p32x4*>(src + 32 * i));
      b[u] = __builtin_nontemporal_load(reinterpret_cast<const p32x4*>(src + 32 * i) + 1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n_units) __builtin_nontemporal_store(a[u] ^ b[u], reinterpret_cast<p32x4*>(dst + 16 * i));
    }
  }
}

int launch_copy_probe(const void* src, void* dst, int64_t dst_bytes, int32_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst,
                     dst_bytes / 16);
  return check_launch("hbm_copy_probe");
}

int launch_read_probe(const void* buf, const int32_t* block_ids, int64_t n_blocks, int32_t block_bytes,
                      uint32_t* sink, int32_t workgroups, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, (const uint8_t*)buf, block_ids,
                     n_blocks, block_bytes, sink);
  return check_launch("hbm_read_probe");
}

}  // namespace dapf8
