// kv_ops.hip -- scale setup, quantize-on-append and the batched page-tag check (gfx950).
//
// [CF §Quantize] the cache stores each token's K/V as FP8 e4m3 (BF16 in the twin); the per-head
// scale, the fp32 division and round-to-nearest-even with saturation are the readings adopted.
// [CF §Protect] the tag check is its own batched pass: it compares each request's expected
// (page, tag) pairs with the live tags and produces one abort bit per request.
#include "common.hpp"

namespace dapf8 {

// ------------------------------------------------------------------------------------------------
// absmax: one workgroup per (head, token chunk); each thread folds |x| with fmaxf (NaN-dropping),
// a workgroup reduction follows, then one atomic max per workgroup on the float's bit pattern
// (non-negative floats order like their unsigned bit patterns).
__global__ __launch_bounds__(256) void absmax_kernel(const void* __restrict__ x, int x_dt, int64_t T, int32_t H,
                                                     int32_t D, int64_t tokens_per_block, float* __restrict__ amax) {
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * tokens_per_block;
  const int64_t t1 = min(T, t0 + tokens_per_block);
  float m = 0.0f;
  const int n = (int)(t1 - t0) * D;  // at most ~4096 + D elements per workgroup
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t t = t0 + i / D;
    const int d = i % D;
    m = fmaxf(m, fabsf(load_act(x, x_dt, ((size_t)t * H + h) * D + d)));
  }
  __shared__ float red[256];
  red[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(amax) + h, __float_as_uint(red[0]));
}

int launch_absmax(const void* x, int x_dt, int64_t T, int32_t H, int32_t D, float* amax, hipStream_t s) {
  if (T == 0) return DAPF8_OK;
  const int64_t tpb = (4096 + D - 1) / D;  // ~4096 elements per workgroup
  const int64_t nb = (T + tpb - 1) / tpb;
  if (nb > 0x7fffffff) return set_error(DAPF8_EUNSUPPORTED, "kv_absmax_update: T too large");
  hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)nb, (unsigned)H), dim3(256), 0, s, x, x_dt, T, H, D, tpb, amax);
  return check_launch("kv_absmax_update");
}

__global__ void scale_kernel(const float* __restrict__ amax, int32_t H, float* __restrict__ scale) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  const float a = amax[h];
  scale[h] = (a == 0.0f) ? 1.0f : __fdiv_rn(a, 448.0f);
}

int launch_scale_from_absmax(const float* amax, int32_t H, float* scale, hipStream_t s) {
  hipLaunchKernelGGL(scale_kernel, dim3((H + 63) / 64), dim3(64), 0, s, amax, H, scale);
  return check_launch("kv_scale_from_absmax");
}

// ------------------------------------------------------------------------------------------------
// append: one thread per (token, head, 16-value chunk); chunks [0, Dk/16) are K, the rest V.
// K chunks are stored with one 16-byte (FP8) or two 16-byte (BF16) stores into the token's row
// inside its 64-byte dimension chunk; V chunks scatter one element per dimension into the
// dimension-major (page, head) block.
// Unit r of token i: head r / (Dk/16 + Dv/16), 16-value chunk r % (Dk/16 + Dv/16) (K chunks
// first, then V), its 16 new values and the head's scale.
struct UnitVals {
  float x[16];
  float s;
  int h, d0;
  bool is_k;
};

template <bool KV_FP8, bool IN_BF16>
__device__ __forceinline__ UnitVals load_unit(int i, int r, const void* __restrict__ k_new,
                                              const void* __restrict__ v_new, const float* __restrict__ k_scale,
                                              const float* __restrict__ v_scale, bool has_v, int32_t Hkv, int32_t Dk,
                                              int32_t Dv) {
  UnitVals u;
  const int ck = Dk >> 4;
  const int cv = has_v ? (Dv >> 4) : 0;
  u.h = r / (ck + cv);
  const int c = r % (ck + cv);
  u.is_k = c < ck;
  const int D = u.is_k ? Dk : Dv;
  u.d0 = (u.is_k ? c : c - ck) * 16;
  const void* src = u.is_k ? k_new : v_new;
  const size_t src_off = ((size_t)i * Hkv + u.h) * D + u.d0;
  if (IN_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)src + src_off);
    uint4 w0 = p[0], w1 = p[1];
    uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u.x[2 * j] = __uint_as_float(w[j] << 16);
      u.x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>((const float*)src + src_off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 f = p[j];
      u.x[4 * j] = f.x;
      u.x[4 * j + 1] = f.y;
      u.x[4 * j + 2] = f.z;
      u.x[4 * j + 3] = f.w;
    }
  }
  u.s = KV_FP8 ? (u.is_k ? k_scale[u.h] : v_scale[u.h]) : 1.0f;
  return u;
}

// Quantise (FP8) or round (BF16) a unit and store it at (page, slot).
template <bool KV_FP8>
__device__ __forceinline__ void store_unit(const UnitVals& u, int page, int slot, void* __restrict__ k_pool,
                                           void* __restrict__ v_pool, int32_t Hkv, int32_t Dk, int32_t Dv,
                                           int32_t P) {
  const float* x = u.x;
  const float s = u.s;
  const int h = u.h, d0 = u.d0;
  const bool is_k = u.is_k;
  if (KV_FP8) {
    // the codes of quantize_e4m3x4, four at a time: the reciprocal's bracket test, and the
    // correctly rounded division for the quads it cannot decide (see quantize_e4m3x4_rcp)
    const bool scale_ok = rcp_scale_ok(s);
    const float r = __builtin_amdgcn_rcpf(s);
    uint32_t cw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bool ok = scale_ok;
      cw[q] = quantize_e4m3x4_rcp(x + 4 * q, r, ok);
      if (__builtin_expect(!ok, 0)) cw[q] = quantize_e4m3x4(x + 4 * q, s);
    }
    if (is_k) {
      uint8_t* dst = (uint8_t*)k_pool + k_elem_offset(page, h, slot, d0, Hkv, P, Dk, 64);
      *reinterpret_cast<uint4*>(dst) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    } else {
      uint8_t* dst = (uint8_t*)v_pool + (((size_t)page * Hkv + h) * Dv + d0) * P + slot;
#pragma unroll
      for (int j = 0; j < 16; ++j) dst[(size_t)j * P] = (uint8_t)(cw[j >> 2] >> (8 * (j & 3)));
    }
  } else {
    uint32_t hb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) hb[j] = f32_to_bf16_rne(x[j]);
    if (is_k) {
      uint16_t* dst = (uint16_t*)k_pool + k_elem_offset(page, h, slot, d0, Hkv, P, Dk, 32);
      uint4 o0, o1;
      o0.x = hb[0] | (hb[1] << 16);
      o0.y = hb[2] | (hb[3] << 16);
      o0.z = hb[4] | (hb[5] << 16);
      o0.w = hb[6] | (hb[7] << 16);
      o1.x = hb[8] | (hb[9] << 16);
      o1.y = hb[10] | (hb[11] << 16);
      o1.z = hb[12] | (hb[13] << 16);
      o1.w = hb[14] | (hb[15] << 16);
      reinterpret_cast<uint4*>(dst)[0] = o0;
      reinterpret_cast<uint4*>(dst)[1] = o1;
    } else {
      uint16_t* dst = (uint16_t*)v_pool + (((size_t)page * Hkv + h) * Dv + d0) * P + slot;
#pragma unroll
      for (int j = 0; j < 16; ++j) dst[(size_t)j * P] = (uint16_t)hb[j];
    }
  }
}

// Unit r of token i, its slot resolved from the token's sequence id and position (abort_mask may
// be NULL).  The new values are loaded first: their address needs no other load, so they are in
// flight while the slot is resolved (sequence id and position, then the page table).
template <bool KV_FP8, bool IN_BF16>
__device__ __forceinline__ void append_unit(
    int i, int r, const void* __restrict__ k_new, const void* __restrict__ v_new, void* __restrict__ k_pool,
    void* __restrict__ v_pool, const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const uint8_t* __restrict__ abort_mask, int32_t B, int32_t Hkv, int32_t Dk,
    int32_t Dv, int32_t P, int32_t num_pages) {
  const UnitVals u = load_unit<KV_FP8, IN_BF16>(i, r, k_new, v_new, k_scale, v_scale, v_pool != nullptr, Hkv, Dk, Dv);
  const int b = seq_ids[i];
  const int pos = positions[i];
  // the abort bit and the page-table entry are read together, at clamped (always valid) indices,
  // and only then is the request checked
  const int bc = min(max(b, 0), B - 1), pc = min(max(pos, 0), pt_stride * P - 1);
  const bool aborted = abort_mask && abort_mask[bc];
  const int page = page_table[(size_t)bc * pt_stride + pc / P];
  if (b < 0 || b >= B || aborted) return;
  if (pos < 0 || pos >= pt_stride * P) return;
  if (page < 0 || page >= num_pages) return;
  store_unit<KV_FP8>(u, page, pos % P, k_pool, v_pool, Hkv, Dk, Dv, P);
}

// Unit r of token i into a slot already resolved and checked.
template <bool KV_FP8, bool IN_BF16>
__device__ __forceinline__ void append_unit_at(int i, int r, int page, int slot, const void* __restrict__ k_new,
                                               const void* __restrict__ v_new, void* __restrict__ k_pool,
                                               void* __restrict__ v_pool, const float* __restrict__ k_scale,
                                               const float* __restrict__ v_scale, int32_t Hkv, int32_t Dk,
                                               int32_t Dv, int32_t P) {
  const UnitVals u = load_unit<KV_FP8, IN_BF16>(i, r, k_new, v_new, k_scale, v_scale, v_pool != nullptr, Hkv, Dk, Dv);
  store_unit<KV_FP8>(u, page, slot, k_pool, v_pool, Hkv, Dk, Dv, P);
}

template <bool KV_FP8, bool IN_BF16>
__global__ __launch_bounds__(256) void append_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, void* __restrict__ k_pool,
    void* __restrict__ v_pool, const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, int32_t T,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, const uint8_t* __restrict__ abort_mask,
    int32_t B, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t P, int32_t num_pages) {
  const int per_token = Hkv * ((Dk >> 4) + (v_pool ? (Dv >> 4) : 0));
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * per_token) return;
  append_unit<KV_FP8, IN_BF16>((int)(gid / per_token), (int)(gid % per_token), k_new, v_new, k_pool, v_pool,
                               page_table, pt_stride, seq_ids, positions, k_scale, v_scale, abort_mask, B, Hkv, Dk,
                               Dv, P, num_pages);
}


int launch_append(const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool, int kv_dt,
                  const int32_t* page_table, int32_t pt_stride, const int32_t* seq_ids, const int32_t* positions,
                  int32_t T, const float* k_scale, const float* v_scale, const uint8_t* abort_mask, int32_t B,
                  int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_pages, hipStream_t s) {
  if (T == 0) return DAPF8_OK;
  const int per_token = Hkv * (Dk / 16 + (v_pool ? Dv / 16 : 0));
  const int64_t n = (int64_t)T * per_token;
  const dim3 grid((unsigned)((n + 255) / 256));
  const bool fp8 = kv_dt == DAPF8_KV_FP8_E4M3, bf = in_dt == DAPF8_ACT_BF16;
#define DAPF8_APPEND(F, BF)                                                                                     \
  hipLaunchKernelGGL((append_kernel<F, BF>), grid, dim3(256), 0, s, k_new, v_new, k_pool, v_pool, page_table,  \
                     pt_stride, seq_ids, positions, T, k_scale, v_scale, abort_mask, B, Hkv, Dk, Dv, page_size, \
                     num_pages)
  if (fp8 && bf)
    DAPF8_APPEND(true, true);
  else if (fp8)
    DAPF8_APPEND(true, false);
  else if (bf)
    DAPF8_APPEND(false, true);
  else
    DAPF8_APPEND(false, false);
#undef DAPF8_APPEND
  return check_launch("kv_append");
}

// ------------------------------------------------------------------------------------------------
// transcode: BF16 pool pages -> FP8 pool pages, the prefill (BF16 cache) -> decode (FP8 cache)
// handoff.  One workgroup per page pair.  The destination page is walked in its own storage order
// in units of 16 bytes (16 codes), so every store is a contiguous 16-byte write; the matching
// source is 16 bf16 values (32 bytes) inside one token's 32-dimension chunk (K) or the same
// position of the dimension-major block (V).  Each thread loads a batch of kTcBatch units before
// converting any of them, so several loads are in flight per thread.
constexpr int kTcBatch = 4;
typedef uint32_t tc_u32x4 __attribute__((ext_vector_type(4)));

// A quotient by a block size: a shift when the size is a power of two (log2 given), else the
// division.
template <bool POW2>
__device__ __forceinline__ int tc_div(int a, int d, int lg) { return POW2 ? a >> lg : a / d; }

// Where unit u (16 destination codes) of a page pair comes from and goes to, and its scale.
struct TcUnit {
  const uint16_t* src;
  uint8_t* dst;
  float s;
};

template <bool POW2>
__device__ __forceinline__ TcUnit tc_unit(int u, int sp, int dp, const uint16_t* k_src, const uint16_t* v_src,
                                          uint8_t* k_dst, uint8_t* v_dst, const float* k_scale,
                                          const float* v_scale, int Hkv, int P, int kblk, int vblk, int kunits,
                                          int lg_kblk, int lg_vblk, int lg_pc) {
  const int pc = P * 64;  // bytes of one 64-dimension chunk of an FP8 block
  TcUnit t;
  if (u < kunits) {
    const int e = u * 16;  // destination byte inside the page's K region
    const int h = tc_div<POW2>(e, kblk, lg_kblk), r = e - h * kblk;
    const int c = tc_div<POW2>(r, pc, lg_pc), tok = (r - c * pc) >> 6, d = c * 64 + (r & 63);
    t.src = k_src + (size_t)sp * Hkv * kblk + (size_t)h * kblk + (size_t)(d >> 5) * P * 32 + (size_t)tok * 32 +
            (d & 31);
    t.dst = k_dst + (size_t)dp * Hkv * kblk + e;
    t.s = k_scale[h];
  } else {
    const int e = (u - kunits) * 16;  // same position in both V layouts
    t.src = v_src + (size_t)sp * Hkv * vblk + e;
    t.dst = v_dst + (size_t)dp * Hkv * vblk + e;
    t.s = v_scale[tc_div<POW2>(e, vblk, lg_vblk)];
  }
  return t;
}

template <bool POW2>
__global__ __launch_bounds__(256) void transcode_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, uint8_t* __restrict__ k_dst,
    uint8_t* __restrict__ v_dst, const int32_t* __restrict__ src_pages, const int32_t* __restrict__ dst_pages,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int32_t Hkv, int32_t Dk, int32_t Dv,
    int32_t P, int32_t num_src, int32_t num_dst, int32_t lg_kblk, int32_t lg_vblk, int32_t lg_pc) {
  const int sp = src_pages[blockIdx.x], dp = dst_pages[blockIdx.x];
  if (sp < 0 || sp >= num_src || dp < 0 || dp >= num_dst) return;
  const int kblk = P * Dk;                // elements of one (page, head) K block (< 2^31 / Hkv)
  const int vblk = P * Dv;
  const int kunits = Hkv * kblk / 16;     // 16-element units of the page's K region
  const int units = kunits + (v_dst ? Hkv * vblk / 16 : 0);
  for (int base = 0; base < units; base += 256 * kTcBatch) {
    tc_u32x4 w[kTcBatch][2];
    float s[kTcBatch];
    uint8_t* dst[kTcBatch];
#pragma unroll
    for (int j = 0; j < kTcBatch; ++j) {
      const int u = min(base + j * 256 + (int)threadIdx.x, units - 1);  // tail lanes redo a valid unit
      const TcUnit t = tc_unit<POW2>(u, sp, dp, k_src, v_src, k_dst, v_dst, k_scale, v_scale, Hkv, P, kblk, vblk,
                                     kunits, lg_kblk, lg_vblk, lg_pc);
      s[j] = t.s;
      dst[j] = t.dst;
      // streamed once: non-temporal loads and stores keep the pages out of the caches
      w[j][0] = __builtin_nontemporal_load(reinterpret_cast<const tc_u32x4*>(t.src));
      w[j][1] = __builtin_nontemporal_load(reinterpret_cast<const tc_u32x4*>(t.src) + 1);
    }
#pragma unroll
    for (int j = 0; j < kTcBatch; ++j) {
      const int u = base + j * 256 + (int)threadIdx.x;
      if (u >= units) break;
      const uint32_t in[8] = {w[j][0].x, w[j][0].y, w[j][0].z, w[j][0].w, w[j][1].x, w[j][1].y, w[j][1].z, w[j][1].w};
      const bool scale_ok = rcp_scale_ok(s[j]);
      const float r = __builtin_amdgcn_rcpf(s[j]);
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x[4] = {__uint_as_float(in[2 * q] << 16), __uint_as_float(in[2 * q] & 0xffff0000u),
                            __uint_as_float(in[2 * q + 1] << 16), __uint_as_float(in[2 * q + 1] & 0xffff0000u)};
        bool ok = scale_ok;
        o[q] = quantize_e4m3x4_rcp(x, r, ok);
        // rare (a code not certain, or a scale outside the reciprocal's range): the correctly
        // rounded division decides
        if (__builtin_expect(!ok, 0)) o[q] = quantize_e4m3x4(x, s[j]);
      }
      const tc_u32x4 ov = {o[0], o[1], o[2], o[3]};
      __builtin_nontemporal_store(ov, reinterpret_cast<tc_u32x4*>(dst[j]));
    }
  }
}

int launch_transcode(const void* k_src, const void* v_src, void* k_dst, void* v_dst, const int32_t* src_pages,
                     const int32_t* dst_pages, int32_t n, const float* k_scale, const float* v_scale, int32_t Hkv,
                     int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_src, int32_t num_dst, hipStream_t s) {
  if (n == 0) return DAPF8_OK;
  // the unit -> (head, chunk, token) split uses shifts when every block size is a power of two
  auto lg = [](int v) { return (v > 0 && (v & (v - 1)) == 0) ? __builtin_ctz((unsigned)v) : -1; };
  const int lk = lg(page_size * Dk), lv = lg(page_size * Dv), lp = lg(page_size * 64);
  const bool pow2 = lk >= 0 && (lv >= 0 || !v_dst) && lp >= 0;
  hipLaunchKernelGGL(pow2 ? transcode_kernel<true> : transcode_kernel<false>, dim3((unsigned)n), dim3(256), 0, s,
                     (const uint16_t*)k_src, (const uint16_t*)v_src, (uint8_t*)k_dst, (uint8_t*)v_dst, src_pages,
                     dst_pages, k_scale, v_scale, Hkv, Dk, Dv, page_size, num_src, num_dst, lk, lv, lp);
  return check_launch("kv_transcode_pages");
}

// ------------------------------------------------------------------------------------------------
// verify: one workgroup per request.  Each of its NT threads owns up to PER references per pass and
// issues all their page-id / expected-tag loads before any live-tag gather, so a pass of NT * PER
// references costs two memory round trips; a workgroup-wide OR (__syncthreads_or) combines the
// mismatches and thread 0 writes the request's bit.  Requests that may hold more references than
// one 256 x 4 pass covers (pt_stride above 1024) get 1024 x 8 passes: there are few of them and they
// cannot fill the GPU, so fewer, wider passes finish sooner (262k tokens: 2 passes instead of 16);
// short requests keep the narrower workgroups, which start sooner.
template <int NT, int PER>
__global__ __launch_bounds__(NT) void verify_kernel(
    const int32_t* __restrict__ page_table, int32_t pt_stride, const uint32_t* __restrict__ expected_tags,
    const int32_t* __restrict__ seq_lens, const uint32_t* __restrict__ live_tags, int32_t num_pages,
    uint8_t* __restrict__ abort_mask, int32_t B, int32_t P) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  int bad = 0;
  if (L < 0 || (int64_t)L > (int64_t)pt_stride * P) {
    bad = 1;
  } else {
    const int n = (int)(((int64_t)L + P - 1) / P);
    const int32_t* pt = page_table + (size_t)b * pt_stride;
    const uint32_t* et = expected_tags + (size_t)b * pt_stride;
    for (int base = 0; base < n; base += NT * PER) {
      int p[PER];
      uint32_t e[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = base + k * NT + (int)threadIdx.x;
        p[k] = j < n ? pt[j] : 0;
        e[k] = j < n ? et[j] : 0u;
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = base + k * NT + (int)threadIdx.x;
        const bool in_range = p[k] >= 0 && p[k] < num_pages;
        const uint32_t live = live_tags[in_range ? p[k] : 0];
        if (j < n) bad |= (!in_range || live != e[k]) ? 1 : 0;
      }
    }
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) abort_mask[b] = bad ? 1 : 0;
}

int launch_verify(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                  const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                  int32_t B, int32_t page_size, hipStream_t s) {
  if (pt_stride > 256 * 4)
    hipLaunchKernelGGL((verify_kernel<1024, 8>), dim3(B), dim3(1024), 0, s, page_table, pt_stride, expected_tags,
                       seq_lens, live_tags, num_pages, abort_mask, B, page_size);
  else
    hipLaunchKernelGGL((verify_kernel<256, 4>), dim3(B), dim3(256), 0, s, page_table, pt_stride, expected_tags,
                       seq_lens, live_tags, num_pages, abort_mask, B, page_size);
  return check_launch("kv_tag_verify");
}

// ------------------------------------------------------------------------------------------------
// verify + append in one launch, for a decode step's few new tokens.  Workgroup b checks request
// b's page tags exactly as verify_kernel does and appends request b's new tokens unless it
// aborted: the abort bit is known inside the workgroup after its OR, so no other workgroup's
// result is needed, and the append's work overlaps the tag check instead of following it in a
// second launch.  Memory round trips:
//   1. all independent loads at once: the sequence length, the first pass of page ids and expected
//      tags (read for the whole row prefix, masked by the length afterwards), and the token list's
//      sequence ids and positions;
//   2. the live-tag gathers and, for every token of b found (seq_ids[i] == b), its page-table
//      entry; the token's (index, page, slot) goes to LDS;
//   3. after the workgroup OR (which also publishes the LDS list) thread 0 writes the abort bit
//      and the threads share the listed tokens' units: load the new values, quantise, store.
// (Loading token b's values speculatively in step 1, for the usual decode step whose token i
// belongs to request i, measured no faster.)
// Requests with more than kVaMaxTok new tokens in one call, or token lists longer than NT * 4,
// take a slower path inside the same workgroup (a second scan of the ids) with the same results.
constexpr int kVaMaxTok = 64;

template <int NT, int PER, bool KV_FP8, bool IN_BF16>
__global__ __launch_bounds__(NT) void verify_append_kernel(
    const int32_t* __restrict__ page_table, int32_t pt_stride, const uint32_t* __restrict__ expected_tags,
    const int32_t* __restrict__ seq_lens, const uint32_t* __restrict__ live_tags, int32_t num_pages,
    uint8_t* __restrict__ abort_mask, int32_t B, int32_t P, const void* __restrict__ k_new,
    const void* __restrict__ v_new, void* __restrict__ k_pool, void* __restrict__ v_pool,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, int32_t T,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int32_t Hkv, int32_t Dk, int32_t Dv) {
  __shared__ int tok_i[kVaMaxTok], tok_page[kVaMaxTok], tok_slot[kVaMaxTok];
  __shared__ int ntok;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int per_token = Hkv * ((Dk >> 4) + (v_pool ? (Dv >> 4) : 0));
  if (tid == 0) ntok = 0;
  // 1. independent loads
  const int L = seq_lens[b];
  const int32_t* pt = page_table + (size_t)b * pt_stride;
  const uint32_t* et = expected_tags + (size_t)b * pt_stride;
  int p0[PER];
  uint32_t e0[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = k * NT + tid;
    p0[k] = j < pt_stride ? pt[j] : 0;
    e0[k] = j < pt_stride ? et[j] : 0u;
  }
  constexpr int kScan = 4;  // token ids read per thread in the fast path
  int sid[kScan], spos[kScan];
#pragma unroll
  for (int k = 0; k < kScan; ++k) {
    const int j = k * NT + tid;
    sid[k] = j < T ? seq_ids[j] : -1;
    spos[k] = j < T ? positions[j] : -1;
  }
  __syncthreads();  // ntok = 0 is visible
  // 2. the first pass's live-tag gathers, then the page-table entries of b's tokens
  const int n = (L < 0 || (int64_t)L > (int64_t)pt_stride * P) ? -1 : (int)(((int64_t)L + P - 1) / P);
  int bad = n < 0 ? 1 : 0;
  uint32_t live0[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const bool in_range = p0[k] >= 0 && p0[k] < num_pages;
    live0[k] = live_tags[in_range ? p0[k] : 0];
  }
  const int nslots = pt_stride * P;
#pragma unroll
  for (int k = 0; k < kScan; ++k) {
    if (sid[k] == b) {
      const int pos = spos[k];
      const int pc = min(max(pos, 0), nslots - 1);
      const int pg = pt[pc / P];
      const bool ok = pos >= 0 && pos < nslots && pg >= 0 && pg < num_pages;
      const int slot_k = atomicAdd(&ntok, 1);
      if (slot_k < kVaMaxTok) {
        tok_i[slot_k] = k * NT + tid;
        tok_page[slot_k] = ok ? pg : -1;
        tok_slot[slot_k] = pos % P;
      }
    }
  }
  // the tag check (verify_kernel's, with the first pass already loaded)
  if (n > 0) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = k * NT + tid;
      const bool in_range = p0[k] >= 0 && p0[k] < num_pages;
      if (j < n) bad |= (!in_range || live0[k] != e0[k]) ? 1 : 0;
    }
    for (int base = NT * PER; base < n; base += NT * PER) {
      int p[PER];
      uint32_t e[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = base + k * NT + tid;
        p[k] = j < n ? pt[j] : 0;
        e[k] = j < n ? et[j] : 0u;
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int j = base + k * NT + tid;
        const bool in_range = p[k] >= 0 && p[k] < num_pages;
        const uint32_t live = live_tags[in_range ? p[k] : 0];
        if (j < n) bad |= (!in_range || live != e[k]) ? 1 : 0;
      }
    }
  }
  // 3. the OR also makes the token list visible
  bad = __syncthreads_or(bad);
  if (tid == 0) abort_mask[b] = bad ? 1 : 0;
  if (bad) return;
  const int nt = ntok;
  if (nt <= kVaMaxTok && T <= kScan * NT) {
    for (int idx = tid; idx < nt * per_token; idx += NT) {
      const int t = idx / per_token;
      if (tok_page[t] >= 0)
        append_unit_at<KV_FP8, IN_BF16>(tok_i[t], idx - t * per_token, tok_page[t], tok_slot[t], k_new, v_new, k_pool,
                                        v_pool, k_scale, v_scale, Hkv, Dk, Dv, P);
    }
  } else {
    // many tokens: every (token, unit) of the call, filtered by sequence id
    for (int64_t idx = tid; idx < (int64_t)T * per_token; idx += NT) {
      const int i = (int)(idx / per_token);
      if (seq_ids[i] == b)
        append_unit<KV_FP8, IN_BF16>(i, (int)(idx - (int64_t)i * per_token), k_new, v_new, k_pool, v_pool, page_table,
                                     pt_stride, seq_ids, positions, k_scale, v_scale, nullptr, B, Hkv, Dk, Dv, P,
                                     num_pages);
    }
  }
}

int launch_verify_append(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                         const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                         int32_t B, int32_t page_size, const void* k_new, const void* v_new, int in_dt, void* k_pool,
                         void* v_pool, int kv_dt, const int32_t* seq_ids, const int32_t* positions, int32_t T,
                         const float* k_scale, const float* v_scale, int32_t Hkv, int32_t Dk, int32_t Dv,
                         hipStream_t s) {
  const bool fp8 = kv_dt == DAPF8_KV_FP8_E4M3, bf = in_dt == DAPF8_ACT_BF16;
#define DAPF8_VA(NT, PER, F, BF)                                                                                  \
  hipLaunchKernelGGL((verify_append_kernel<NT, PER, F, BF>), dim3(B), dim3(NT), 0, s, page_table, pt_stride,    \
                     expected_tags, seq_lens, live_tags, num_pages, abort_mask, B, page_size, k_new, v_new,       \
                     k_pool, v_pool, seq_ids, positions, T, k_scale, v_scale, Hkv, Dk, Dv)
#define DAPF8_VA_DT(NT, PER)          \
  if (fp8 && bf)                      \
    DAPF8_VA(NT, PER, true, true);    \
  else if (fp8)                       \
    DAPF8_VA(NT, PER, true, false);   \
  else if (bf)                        \
    DAPF8_VA(NT, PER, false, true);   \
  else                                \
    DAPF8_VA(NT, PER, false, false);
  if (pt_stride > 256 * 4) {
    DAPF8_VA_DT(1024, 8)
  } else {
    DAPF8_VA_DT(256, 4)
  }
#undef DAPF8_VA_DT
#undef DAPF8_VA
  return check_launch("kv_tag_verify_append");
}

}  // namespace dapf8
