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
// A workgroup owns TPW adjacent 16-column tiles, as many as spread the N / 16 tiles over one
// workgroup per compute unit (at most 8; more tiles than that take more workgroups), and its eight
// waves split K and meet in LDS.  Each wave keeps D 128-k blocks of its TPW tiles in flight (TPW
// KiB each), so a compute unit streams 8 * D * TPW KiB at a time from one workgroup, and one
// activation block serves TPW tiles.
//
// Per 128-k block and tile: one 16-byte weight load per lane and four 16x16x32 MFMAs with the
// offset weights 1 + u/16 = 1.5 + q/16, plus one MFMA per step against all-ones bf16 that gives
// sum_k x for the offset's correction: sum x*q = 16 (sum x*(1.5 + q/16) - 1.5 sum x), taken per
// 128-k group before its scale (times 16, exact) multiplies it.  Products of bf16 values are exact
// in fp32, and the offset (1.5 against |q|/16 <= 0.5) keeps the cancellation in the correction
// small: the fp32 error is about 2^-24 sum |x| (48 + |q|) s per group instead of the
// 2^-24 sum |x| |q| s of a direct product.
#include "common.hpp"

namespace dapf8 {

namespace {

typedef uint32_t w4_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kW4MaxTiles = 8;   // 16-column tiles per workgroup, at most
constexpr int kW4Waves = 8;      // K split inside a workgroup
constexpr int kW4Depth = 2;      // 128-k blocks in flight per wave
constexpr int kW4Chunk = 8;      // blocks per unrolled stretch of a wave's K range
constexpr int kW4BufferWord3 = 0x00020000;  // buffer resource word 3: 32-bit data format, raw
constexpr int kW4NonTemporal = 2;           // cache policy of the weight loads: streamed once

// nibble pair p of w (bits 4p..4p+3 and 16+4p..) -> bf16 pair 1 + u/16: u moves to mantissa bits 3..6.
// mask = 0x00780078 and one = 0x3F803F80 arrive in registers, so that the mask and the or fuse
// into one v_and_or_b32 per pair (with both as literal constants the instruction cannot encode
// them, and the compiler splits it into two).
__device__ __forceinline__ bf16x8 w4_dequant_offset(uint32_t w, uint32_t mask, uint32_t one) {
  w4_u32x4 r;
  r.x = ((w << 3) & mask) | one;
  r.y = ((w >> 1) & mask) | one;
  r.z = ((w >> 5) & mask) | one;
  r.w = ((w >> 9) & mask) | one;
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace

template <bool OUT_BF16, int TPW, int D>
__global__ __launch_bounds__(64 * kW4Waves) void w4_gemv_kernel(const uint16_t* __restrict__ x,
                                                                 const uint8_t* __restrict__ wp,
                                                                 const float* __restrict__ sp, void* __restrict__ y,
                                                                 int M, int N, int K) {
  __shared__ f32x4 red[kW4Waves - 1][TPW][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int NT = N >> 4;                  // 16-column tiles
  const int nt0 = blockIdx.x * TPW;       // first tile of this workgroup
  const int KB = K >> 7;                  // 128-k blocks
  const int kb0 = wave * KB / kW4Waves, kb1 = (wave + 1) * KB / kW4Waves;  // may be empty
  const int m = c;                        // A operand row of this lane
  const bool row_ok = m < M;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, w4_u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  // the packed weights as a buffer (fewer than 2^31 bytes, checked at the API)
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)wp, (short)0, (int)((size_t)NT * KB * 1024), kW4BufferWord3);
  uint32_t nib_mask, nib_one;  // the dequantisation's constants, held in vector registers
  asm volatile("v_mov_b32 %0, 0x780078" : "=v"(nib_mask));
  asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(nib_one));

  f32x4 tot[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) tot[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  struct Blk {
    w4_u32x4 w[TPW];
    w4_u32x4 xa[4];
    float s[TPW];
  };
  // block kb of every tile.  Past the wave's last block (pipeline tail) and past the last tile (the
  // last workgroup's spare tiles) nothing reads the values: the weight load then gets an offset
  // past the buffer's end, which a buffer load answers with zeros without touching memory, and
  // the small scale and activation loads repeat valid addresses (cache hits).
  auto load = [&](Blk& b, int kb) __attribute__((always_inline)) {
    const bool live = kb < kb1;
    kb = min(kb, kb1 - 1);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int nt = min(nt0 + t, NT - 1);
      const uint32_t off = (uint32_t)(((size_t)nt * KB + kb) * 1024) + c * 64 + g * 16;
      b.w[t] = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, live && nt0 + t < NT ? off : 0x80000000u, 0,
                                                     kW4NonTemporal);
      b.s[t] = sp[(size_t)kb * N + nt * 16 + c];
    }
    // rows m >= M repeat row 0: a product row depends on its own A row only, and those rows are
    // never stored (zeroing them here would make every load wait for its data at once)
    const uint16_t* xr = x + (size_t)(row_ok ? m : 0) * K + kb * 128 + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) b.xa[j] = *reinterpret_cast<const w4_u32x4*>(xr + 8 * j);
  };
  auto compute = [&](const Blk& b, bool valid) __attribute__((always_inline)) {
    f32x4 acc[TPW], xs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, b.xa[j]);
      xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, xs, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint32_t wj = j == 0 ? b.w[t].x : j == 1 ? b.w[t].y : j == 2 ? b.w[t].z : b.w[t].w;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w4_dequant_offset(wj, nib_mask, nib_one), acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const f32x4 part = (acc[t] - 1.5f * xs) * (16.0f * b.s[t]);
      if (valid) tot[t] += part;
    }
  };

  if (kb0 < kb1) {
    Blk ring[D];
#pragma unroll
    for (int i = 0; i < D; ++i) load(ring[i], kb0 + i);
    // chunks of kW4Chunk blocks, each unrolled straight through: inside a chunk the waits count
    // only the slot being consumed, so D blocks stay in flight (a loop head would make the
    // compiler wait for every load there, and so would a load under a condition).  Each slot is
    // refilled right after its products; past the wave's last block the refill reads nothing
    // (see load) and a block past the end is computed and discarded, which keeps every load and
    // product unconditional.  The barrier keeps the scheduler from sinking the refill into the
    // next products.
    for (int base = kb0; base < kb1; base += kW4Chunk) {
#pragma unroll
      for (int i = 0; i < kW4Chunk; ++i) {
        compute(ring[i % D], base + i < kb1);
        load(ring[i % D], base + i + D);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // the K eighths meet in LDS; wave 0 adds them and writes the rows m < M of the real tiles
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) red[wave - 1][t][lane] = tot[t];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (nt0 + t >= NT) break;
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
  // one workgroup per compute unit when the tiles allow: TPW = ceil(tiles / CUs), at most 8
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return check_launch("w4a16_gemv");
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  const int nt = N / 16;
  const int tpw = std::min(kW4MaxTiles, std::max(1, (nt + cus[dev] - 1) / cus[dev]));
  const dim3 grid((unsigned)((nt + tpw - 1) / tpw)), block(64 * kW4Waves);
#define DAPF8_W4(T)                                                                                                 \
  case T:                                                                                                          \
    if (out_dt == DAPF8_ACT_BF16)                                                                                  \
      hipLaunchKernelGGL((w4_gemv_kernel<true, T, kW4Depth>), grid, block, 0, st, (const uint16_t*)x, wp, sp, y, M,  \
                         N, K);                                                                                    \
    else                                                                                                           \
      hipLaunchKernelGGL((w4_gemv_kernel<false, T, kW4Depth>), grid, block, 0, st, (const uint16_t*)x, wp, sp, y,    \
                         M, N, K);                                                                                 \
    break;
  switch (tpw) {
    DAPF8_W4(1)
    DAPF8_W4(2)
    DAPF8_W4(3)
    DAPF8_W4(4)
    DAPF8_W4(5)
    DAPF8_W4(6)
    DAPF8_W4(7)
    DAPF8_W4(8)
  }
#undef DAPF8_W4
  return check_launch("w4a16_gemv");
}

}  // namespace dapf8
