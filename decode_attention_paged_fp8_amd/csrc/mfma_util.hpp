// mfma_util.hpp -- device helpers shared by the matrix-core decode kernels (gfx950): operand
// types, FP8 -> bf16 conversion, wave reductions, bf16 term splitting, and the block-wide prefix
// over the sequences' work units that the persistent (stream-K) kernels and their merge use.
#pragma once

#include "common.hpp"

namespace dapf8 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, u);
}

// 8 e4m3 codes (two dwords, code i in byte i) -> bf16x8 (exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const uint2 lo = fp8x4_to_bf16x4(w0);
  const uint2 hi = fp8x4_to_bf16x4(w1);
  return as_bf16x8(lo.x, lo.y, hi.x, hi.y);
}

// reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Split fp32 values into NT bf16 terms (round to nearest even each time): p = t1 + t2 + ... to
// ~8 * NT bits.
template <int NT>
__device__ __forceinline__ void split_bf16(const float* p, bf16x8* out) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = p[i];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)r[i];
      out[t][i] = h;
      r[i] -= (float)h;
    }
  }
}

// The running softmax reference max is only raised when a window's max exceeds it by more than
// this many binades, so weights stay below 2^kRescaleSlack and the accumulators are rescaled
// rarely (exact either way: every term is relative to the same reference).
constexpr float kRescaleSlack = 8.0f;

// Work-unit prefix of a persistent decode kernel.  A sequence of attended length L owns
// ceil(L / 2^shift) units per KV head (32-token windows or 64-token pages) and
// ceil(units / upp) partitions of upp units.
constexpr int kSkMaxB = 1024;

struct SkPrefix {
  int unit[kSkMaxB + 1];  // exclusive prefix of units per sequence
  int part[kSkMaxB + 1];  // exclusive prefix of partitions per sequence
  int len[kSkMaxB];       // attended length (0 when aborted)
};

// Prefix over the batch (B <= kSkMaxB), computed by the workgroup's first wave alone: each lane
// loads its sequences (b = lane, lane + 64, ...) with all loads in flight at once, then 64-wide
// chunks are scanned with lane shuffles and carried from chunk to chunk; one workgroup barrier
// publishes the tables.  (A workgroup-wide scan would cost a barrier pair per step.)
template <int NT>
__device__ __forceinline__ void sk_prefix(SkPrefix& px, const AttnArgs& a, int shift, int upp) {
  constexpr int kChunks = kSkMaxB / 64;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int max_len = a.pt_stride * a.page_size;
    int L[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int b = 64 * c + lane;
      L[c] = 0;
      if (b < a.B) {
        const int raw = a.seq_lens[b];
        int v = min(max(raw, 0), max_len);
        if (a.abort_mask && a.abort_mask[b]) v = 0;
        // with the in-walk tag check a length the page table cannot hold aborts the request
        if (a.abort_out && (raw < 0 || raw > max_len)) v = 0;
        L[c] = v;
      }
    }
    int cw = 0, cp = 0;  // units and partitions of the chunks before
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (64 * c >= a.B) break;  // uniform
      const int b = 64 * c + lane;
      const int lw = (L[c] + (1 << shift) - 1) >> shift;
      const int lp = (lw + upp - 1) / upp;
      int iw = lw, ip = lp;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int tw = __shfl_up(iw, off), tp = __shfl_up(ip, off);
        if (lane >= off) {
          iw += tw;
          ip += tp;
        }
      }
      if (b < a.B) {
        px.len[b] = L[c];
        px.unit[b] = cw + iw - lw;
        px.part[b] = cp + ip - lp;
      }
      cw += __shfl(iw, 63);
      cp += __shfl(ip, 63);
    }
    if (lane == 0) {
      px.unit[a.B] = cw;
      px.part[a.B] = cp;
    }
  }
  __syncthreads();
}

// largest b in [0, B) with Hkv * unit[b] <= g (binary search in LDS)
__device__ __forceinline__ int sk_find_seq(const SkPrefix& px, int B, int Hkv, long g) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long)Hkv * px.unit[mid] <= g)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Publish the prefix for the merge kernel: ws[0..B] = unit prefix, ws[B+1..2B+1] = partitions.
__device__ __forceinline__ void sk_publish_prefix(const SkPrefix& px, const AttnArgs& a, int nthreads) {
  int* wsp = reinterpret_cast<int*>(a.ws_ml);
  for (int b = threadIdx.x; b <= a.B; b += nthreads) {
    wsp[b] = px.unit[b];
    wsp[a.B + 1 + b] = px.part[b];
  }
}

}  // namespace dapf8
