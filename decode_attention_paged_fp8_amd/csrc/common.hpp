// common.hpp -- internal helpers shared by the gfx950 kernels of the paged decode-attention library.
//
// Page references (used throughout the sources):
//   [CF §Quantize]  Cloudflare, "Smaller, faster, safer: running Kimi and GLM at scale", Chinese
//                   translation on feinterview.poetries.top, section "量化 KV cache": K/V cache kept as
//                   FP8 (e4m3) instead of BF16; the FP8 attention kernel converts values on read.
//   [CF §Protect]   same page, section "保护共享 KV cache": per-page tags that change on
//                   reallocation, per-request expected (page, tag) lists, a separate batched check
//                   before decode reads the cache, abort on mismatch, no-op tracker when disabled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/dapf8.h"

namespace dapf8 {

// ------------------------------------------------------------------------------------------------
// Host-side error reporting (thread-local message, negative return code).
int set_error(int code, const char* fmt, ...);
void clear_error();

#define DAPF8_CHECK_ARG(cond, ...)                               \
  do {                                                           \
    if (!(cond)) return ::dapf8::set_error(DAPF8_EINVAL, __VA_ARGS__); \
  } while (0)

int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------------------------------------------
// Device helpers.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bit pattern, round to nearest with ties to even; NaN -> quiet NaN with its sign.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
  u += 0x7fffu + ((u >> 16) & 1u);  // carry into the exponent handles overflow to infinity
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Quantise four values with a per-head scale: the e4m3 code of the correctly rounded fp32 quotient
// x / s (nearest, ties to even; NaN -> 0x7F with x's sign; |x / s| >= 448, infinities included ->
// 0x7E with the sign).  The quotient, clamped to +-448, is encoded by the hardware OCP conversion
// (round to nearest even, exact up to 448 in magnitude); a NaN x gets the NaN code patched in,
// which the conversion of a clamped NaN would not give.
__device__ __forceinline__ uint32_t quantize_e4m3x4(const float* x, float s) {
  float d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = __builtin_amdgcn_fmed3f(__fdiv_rn(x[i], s), -448.0f, 448.0f);
  const int c01 = __builtin_amdgcn_cvt_pk_fp8_f32(d[0], d[1], 0, false);
  uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(d[2], d[3], c01, true);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (x[i] != x[i]) c = (c & ~(0xffu << (8 * i))) | (((__float_as_uint(x[i]) >> 24 & 0x80u) | 0x7fu) << (8 * i));
  return c;
}

// Bulk quantisation of four values with one scale s in [2^-126, 2^126) and r, the hardware
// reciprocal of s (within one ulp, a relative 2^-23, of 1/s; other scales take the division).
// q = RN(x * r) is then within a relative 2^-23 + 2^-24 of x / s, and the correctly rounded
// quotient within |q| * 2^-22 of q.  The pair q * (1 -+ 2^-20), each one fused multiply-add,
// brackets every value that close with room to spare.  Rounding to e4m3 is monotonic, so when the
// hardware conversion gives q and both brackets one code, that code is the quotient's.  q is
// clamped to +-kQClamp = +-(448 - 7 * 2^-14) first, which keeps the upper bracket <= 448; every
// quotient that large has the saturated code.  Below the normal fp32 range the relative bound
// fails, but there every candidate's code is a zero of x's sign (and -0, whose lower bracket turns
// +0, is sent to the division).  `ok` is cleared when a code is not certain: a NaN x, or brackets
// that straddle a rounding boundary -- mostly quotients that sit on an e4m3 rounding midpoint,
// which bf16 values and scales produce at rates up to a few in 10^3 for some scales, otherwise
// about 5 values in 10^6.  The caller then takes quantize_e4m3x4.
constexpr float kQClamp = 448.0f - 7.0f / 16384.0f;
__device__ __forceinline__ bool rcp_scale_ok(float s) { return s >= 0x1p-126f && s < 0x1p126f; }
__device__ __forceinline__ uint32_t quantize_e4m3x4_rcp(const float* x, float r, bool& ok) {
  float q[4], lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = x[i] * r;
    ok = ok && (q0 == q0);
    q[i] = __builtin_amdgcn_fmed3f(q0, -kQClamp, kQClamp);
    lo[i] = fmaf(q[i], -0x1p-20f, q[i]);  // toward zero
    hi[i] = fmaf(q[i], 0x1p-20f, q[i]);   // away from zero
  }
  const int c01 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c01, true);
  const int l01 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false);
  const uint32_t l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo[2], lo[3], l01, true);
  const int h01 = __builtin_amdgcn_cvt_pk_fp8_f32(hi[0], hi[1], 0, false);
  const uint32_t h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hi[2], hi[3], h01, true);
  ok = ok && l == c && h == c;
  return c;
}

// Four e4m3 codes packed in a dword -> four floats (hardware conversion, OCP e4m3 on gfx950).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo.x;
  o[1] = lo.y;
  o[2] = hi.x;
  o[3] = hi.y;
}

// Four e4m3 codes -> four bf16 values (exact: every e4m3 value is a bf16 value), packed 2 per dword.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

__device__ __forceinline__ float load_act(const void* p, int dt, size_t i) {
  return dt == DAPF8_ACT_BF16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

constexpr float kLog2e = 1.4426950408889634f;

// K pool element offset.  Inside a (page, head) block a token's Dk values are cut into chunks of
// C = 64 bytes (C = 64 FP8 codes or 32 bf16 values) stored chunk by chunk:
//   block [Dk / C][P][C]  ->  offset(page, h, slot, d) = ((page*Hkv + h)*P*Dk) + (d/C)*P*C + slot*C + d%C
// so one load instruction that reads 16 consecutive tokens' chunk covers whole 128-byte lines.
__host__ __device__ __forceinline__ size_t k_elem_offset(int page, int h, int slot, int d, int Hkv, int P, int Dk,
                                                         int C) {
  return ((size_t)page * Hkv + h) * (size_t)P * Dk + (size_t)(d / C) * P * C + (size_t)slot * C + (d % C);
}

// ------------------------------------------------------------------------------------------------
// Launchers (defined next to their kernels).
int launch_absmax(const void* x, int x_dt, int64_t T, int32_t H, int32_t D, float* amax, hipStream_t s);
int launch_scale_from_absmax(const float* amax, int32_t H, float* scale, hipStream_t s);
int launch_append(const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool, int kv_dt,
                  const int32_t* page_table, int32_t pt_stride, const int32_t* seq_ids, const int32_t* positions,
                  int32_t T, const float* k_scale, const float* v_scale, const uint8_t* abort_mask, int32_t B,
                  int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_pages, hipStream_t s);
int launch_transcode(const void* k_src, const void* v_src, void* k_dst, void* v_dst, const int32_t* src_pages,
                     const int32_t* dst_pages, int32_t n, const float* k_scale, const float* v_scale, int32_t Hkv,
                     int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_src, int32_t num_dst, hipStream_t s);
// Device page allocator (single-workgroup kernels; at most kMaxAllocRequests requests per call).
constexpr int kMaxAllocRequests = 8192;
int launch_pages_init(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages, hipStream_t s);
int launch_pages_alloc(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages,
                       const int32_t* counts, const int32_t* first_slot, int32_t B, int32_t* page_table,
                       uint32_t* expected_tags, int32_t pt_stride, uint8_t* granted, hipStream_t s);
int launch_pages_free(int32_t* free_list, int32_t* free_count, const int32_t* pages, int32_t n, int32_t num_pages,
                      int32_t* status, hipStream_t s);
// INT4 weight-only GEMV (M <= 16 rows, N a multiple of 64, K a multiple of 128, groups of 128 k).
int launch_w4_pack(const int8_t* q, const float* s, int32_t N, int32_t K, uint8_t* wp, float* sp, hipStream_t st);
int launch_w4_gemv(const void* x, const uint8_t* wp, const float* sp, void* y, int out_dt, int32_t M, int32_t N,
                   int32_t K, hipStream_t st);
// Read-only streaming probe (the attainable HBM read rate).
int launch_copy_probe(const void* src, void* dst, int64_t dst_bytes, int32_t workgroups, hipStream_t s);
int launch_read_probe(const void* buf, const int32_t* block_ids, int64_t n_blocks, int32_t block_bytes,
                      uint32_t* sink, int32_t workgroups, hipStream_t s);
int launch_verify(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                  const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                  int32_t B, int32_t page_size, hipStream_t s);
int launch_verify_append(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                         const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                         int32_t B, int32_t page_size, const void* k_new, const void* v_new, int in_dt, void* k_pool,
                         void* v_pool, int kv_dt, const int32_t* seq_ids, const int32_t* positions, int32_t T,
                         const float* k_scale, const float* v_scale, int32_t Hkv, int32_t Dk, int32_t Dv,
                         hipStream_t s);

// Arguments of one attention launch, resolved on the host.
struct AttnArgs {
  const void* q;
  int q_dt;
  const void* k_pool;
  const void* v_pool;  // NULL = shared-KV
  int kv_dt;
  const int32_t* page_table;
  int32_t pt_stride;
  const int32_t* seq_lens;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* abort_mask;
  void* out;
  int out_dt;
  float sm_scale;
  int32_t B, Hq, Hkv, G, Dk, Dv, page_size, num_pages;
  int32_t split;      // tokens per partition
  int32_t nsplit;     // partitions of the longest possible sequence (pt_stride * page_size)
  float* ws_o;        // [B][Hq][nsplit][Dv] partial outputs (nsplit > 1)
  float* ws_ml;       // [B][Hq][nsplit][2]  partial (max, sum) in the log2 domain
  int32_t gb = 1;     // generic kernel: query heads per workgroup (of the G sharing a KV head)
  // Page-tag check inside the page walk (paged_decode_attn_checked); all NULL otherwise.
  const uint32_t* live_tags = nullptr;      // [num_pages]
  const uint32_t* expected_tags = nullptr;  // [B][pt_stride]
  uint8_t* abort_out = nullptr;             // [B] written: 1 = request aborted
};

enum class Variant { kGeneric, kMfmaD128P16, kMfmaStreamK, kMfmaLatent };

// Stream-K limits: batches up to kSkMaxBatch sequences; the workspace is sized for at most
// kSkMaxWorkers workers (a launch uses min(resident waves, kSkMaxWorkers) of them), so sizing
// needs no device query.
constexpr int kSkMaxBatch = 1024;
constexpr int kSkMaxWorkers = 4096;

// Generic (VALU) kernel: a workgroup serves up to kGenMaxGB query heads of one KV head; its LDS
// holds gb x split scores and gb x Dk query values.
constexpr int kGenMaxGB = 8;
constexpr int kGenScoreFloats = 8192;
constexpr int kGenQFloats = 8192;
constexpr int kGenericMaxSplit = 4096;
int launch_attn_generic(const AttnArgs& a, hipStream_t s);
int launch_attn_mfma(const AttnArgs& a, hipStream_t s);
int launch_attn_sk(const AttnArgs& a, int max_workers, hipStream_t s);
// Shared-KV latent kernel (Dk 576, Dv 512, page 64, FP8, bf16 queries, G in {16, 32, 64, 128}):
// persistent workgroups, at most kLatMaxWorkgroups of them (the workspace is sized for that many).
constexpr int kLatMaxWorkgroups = 512;
int launch_attn_latent(const AttnArgs& a, int max_workgroups, hipStream_t s);
// merge of the pieces a persistent kernel wrote (any Dv multiple of 4, G rows per piece)
int launch_merge_sk(const AttnArgs& a, int nworkers, hipStream_t s);
int launch_merge(const AttnArgs& a, hipStream_t s);

}  // namespace dapf8
