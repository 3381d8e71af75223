// w4_gemv.hip -- INT4 weight-only decode GEMV on the matrix cores (gfx950):
//   y[m][n] = sum_k x[m][k] * q[n][k] * s[n][k / 128],   q in [-8, 7], s fp32, x bf16, M <= 16.
// Decode multiplies a few activation rows by the whole weight matrix, so the weights' bytes bound
// it; four-bit weights halve them against eight-bit ones.
//
// Packed weights: tiles of 16 output columns x 128 k, 1 KiB each, [N/16][K/128][16 cols][64 B].
// Inside a column's 64 bytes, group g (16 bytes) holds k = 32g .. 32g+31 of the tile as four dwords
// (dword j: k = 32g + 8j .. +7), each dword's nibbles in the order k+0, k+2, k+4, k+6, k+1, k+3, k+5,
// k+7, every nibble u = q + 8.  That order lets one shift and one and-or turn a nibble pair into a
// bf16 pair 1 + u/16 (exponent 2^0; u lands in the top four of the seven mantissa bits, so the value
// is exact): ((w >> 4p) << 3) & 0x00780078 | 0x3F803F80 is (k+2p, k+2p+1).  Scales are packed
// k-block-major, [K/128][N], so a wave's 16 columns read 64 contiguous bytes.
//
// One wave owns kW4Tiles adjacent 16-column tiles and an eighth of K; the eight waves of a
// workgroup split K and meet in LDS (many waves per CU keep enough weight bytes in flight).  Per 128-k block and tile: one 16-byte weight load per lane and four
// 16x16x32 MFMAs with the offset weights 1 + u/16 = 1.5 + q/16, plus one MFMA per step against
// all-ones bf16 that gives sum_k x for the offset's correction: sum x*q = 16 (sum x*(1.5 + q/16) -
// 1.5 sum x), taken per 128-k group before its scale (times 16, exact) multiplies it.  Products of
// bf16 values are exact in fp32, and the offset (1.5 against |q|/16 <= 0.5) keeps the cancellation
// in the correction small: the fp32 error is about 2^-24 sum |x| (48 + |q|) s per group instead of
// the 2^-24 sum |x| |q| s of a direct product.
#include "common.hpp"

namespace dapf8 {

namespace {

typedef uint32_t w4_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kW4Tiles = 4;      // 16-column tiles per wave
constexpr int kW4Waves = 8;      // K split inside a workgroup

// nibble pair p of w (bits 4p..4p+3 and 16+4p..) -> bf16 pair 1 + u/16: u moves to mantissa bits 3..6
__device__ __forceinline__ bf16x8 w4_dequant_offset(uint32_t w) {
  w4_u32x4 r;
  r.x = ((w << 3) & 0x00780078u) | 0x3F803F80u;
  r.y = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
  r.z = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
  r.w = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace

template <bool OUT_BF16>
__global__ __launch_bounds__(64 * kW4Waves) void w4_gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ wp,
                                                      const float* __restrict__ sp, void* __restrict__ y, int M, int N,
                                                      int K) {
  __shared__ f32x4 red[kW4Waves - 1][kW4Tiles][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int nt0 = blockIdx.x * kW4Tiles;  // first 16-column tile
  const int KB = K >> 7;                  // 128-k blocks
  const int kb0 = wave * KB / kW4Waves, kb1 = (wave + 1) * KB / kW4Waves;  // may be empty
  const int m = c;                        // A operand row of this lane
  const bool row_ok = m < M;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, w4_u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  f32x4 tot[kW4Tiles];
#pragma unroll
  for (int t = 0; t < kW4Tiles; ++t) tot[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  struct Blk {
    w4_u32x4 w[kW4Tiles];
    w4_u32x4 xa[4];
    float s[kW4Tiles];
  };
  auto load = [&](Blk& b, int kb) __attribute__((always_inline)) {
    kb = min(kb, kb1 - 1);
#pragma unroll
    for (int t = 0; t < kW4Tiles; ++t) {
      const size_t tile = (size_t)(nt0 + t) * KB + kb;
      b.w[t] = __builtin_nontemporal_load(reinterpret_cast<const w4_u32x4*>(wp + tile * 1024 + c * 64 + g * 16));
      b.s[t] = sp[(size_t)kb * N + (nt0 + t) * 16 + c];
    }
    const uint16_t* xr = x + (size_t)(row_ok ? m : 0) * K + kb * 128 + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const w4_u32x4 v = *reinterpret_cast<const w4_u32x4*>(xr + 8 * j);
      b.xa[j] = row_ok ? v : w4_u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto compute = [&](const Blk& b) __attribute__((always_inline)) {
    f32x4 acc[kW4Tiles], xs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < kW4Tiles; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, b.xa[j]);
      xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, xs, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kW4Tiles; ++t) {
        const uint32_t wj = j == 0 ? b.w[t].x : j == 1 ? b.w[t].y : j == 2 ? b.w[t].z : b.w[t].w;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w4_dequant_offset(wj), acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < kW4Tiles; ++t) tot[t] += (acc[t] - 1.5f * xs) * (16.0f * b.s[t]);
  };

  if (kb0 < kb1) {
    Blk b0, b1;
    load(b0, kb0);
    for (int kb = kb0; kb < kb1; kb += 2) {
      // the next block's loads are issued before this block's products (the scheduler would
      // otherwise wait for them inside the products and keep fewer bytes in flight)
      load(b1, kb + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(b0);
      if (kb + 1 >= kb1) break;
      load(b0, kb + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b1);
    }
  }
  // the K quarters meet in LDS; wave 0 adds them and writes the rows m < M
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < kW4Tiles; ++t) red[wave - 1][t][lane] = tot[t];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < kW4Tiles; ++t) {
      f32x4 v = tot[t];
#pragma unroll
      for (int w = 0; w < kW4Waves - 1; ++w) v += red[w][t][lane];
      // D[row][col]: col = lane % 16 (output column), rows 4 * (lane / 16) + i (batch rows)
      const int n = (nt0 + t) * 16 + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row < M) {
          if (OUT_BF16)
            ((uint16_t*)y)[(size_t)row * N + n] = f32_to_bf16_rne(v[i]);
          else
            ((float*)y)[(size_t)row * N + n] = v[i];
        }
      }
    }
  }
}

// Packing: one thread per output dword (8 nibbles of one column).
__global__ void w4_pack_kernel(const int8_t* __restrict__ q, const float* __restrict__ s, int N, int K,
                               uint32_t* __restrict__ wp, float* __restrict__ sp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // dword index in packed order
  const int64_t total = (int64_t)N * K / 8;
  if (i < total) {
    // packed order: tile (nt, kb), column c, group g, dword j
    const int j = (int)(i & 3), g = (int)((i >> 2) & 3), c = (int)((i >> 4) & 15);
    const int64_t tile = i >> 8;
    const int KB = K >> 7;
    const int nt = (int)(tile / KB), kb = (int)(tile - (int64_t)nt * KB);
    const int n = nt * 16 + c, k0 = kb * 128 + 32 * g + 8 * j;
    const int8_t* src = q + (size_t)n * K + k0;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int v = min(max((int)src[e], -8), 7) + 8;
      const int pos = (e & 1) ? 4 + (e >> 1) : (e >> 1);  // nibble order k+0, 2, 4, 6, 1, 3, 5, 7
      w |= (uint32_t)v << (4 * pos);
    }
    wp[i] = w;
  }
  const int64_t ns = (int64_t)N * (K >> 7);
  if (i < ns) {  // scales [N][K/128] -> [K/128][N]
    const int KB = K >> 7;
    const int n = (int)(i / KB), kb = (int)(i - (int64_t)n * KB);
    sp[(size_t)kb * N + n] = s[i];
  }
}

int launch_w4_pack(const int8_t* q, const float* s, int32_t N, int32_t K, uint8_t* wp, float* sp, hipStream_t st) {
  const int64_t total = std::max((int64_t)N * K / 8, (int64_t)N * (K >> 7));
  hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, q, s, N, K,
                     (uint32_t*)wp, sp);
  return check_launch("w4_pack");
}

int launch_w4_gemv(const void* x, const uint8_t* wp, const float* sp, void* y, int out_dt, int32_t M, int32_t N,
                   int32_t K, hipStream_t st) {
  const dim3 grid((unsigned)(N / (16 * kW4Tiles)));
  if (out_dt == DAPF8_ACT_BF16)
    hipLaunchKernelGGL(w4_gemv_kernel<true>, grid, dim3(64 * kW4Waves), 0, st, (const uint16_t*)x, wp, sp, y, M, N,
                       K);
  else
    hipLaunchKernelGGL(w4_gemv_kernel<false>, grid, dim3(64 * kW4Waves), 0, st, (const uint16_t*)x, wp, sp, y, M, N,
                       K);
  return check_launch("w4a16_gemv");
}

}  // namespace dapf8
