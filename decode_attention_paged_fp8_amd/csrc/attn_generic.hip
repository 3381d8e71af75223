// attn_generic.hip -- shape-general decode attention on the vector ALUs, plus the split merge.
//
// [CF §Quantize] decode attention over the paged cache; stored FP8 values are converted on read
// (hardware e4m3 -> fp32 conversion) and the per-head scales are folded into the score and the
// output.  Used for shapes the matrix-core kernel does not cover (Dk a multiple of 64, Dv a multiple
// of 16, both up to 1024, any page size, shared-KV).  One workgroup handles one (sequence, query head,
// partition): scores of the partition go to LDS, a workgroup max/sum gives the softmax, and each
// thread accumulates some output dimensions.  Partition results are (max, sum, unnormalised
// output) in the log2 domain and are merged by merge_kernel with the log-sum-exp rule.
#include "common.hpp"

namespace dapf8 {

constexpr int kGenThreads = 256;
constexpr int kGenMaxSplit = 4096;  // tokens per partition (LDS score buffer)

__device__ __forceinline__ float wg_reduce(float v, float* red, bool is_max) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = kGenThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s)
      red[threadIdx.x] = is_max ? fmaxf(red[threadIdx.x], red[threadIdx.x + s]) : red[threadIdx.x] + red[threadIdx.x + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// q . K_t over the token's dimension chunks (chunk c holds dims c*C .. c*C+C-1, C = 64 bytes).
template <bool KV_FP8>
__device__ __forceinline__ float dot_row(const void* k_pool, size_t block, int slot, int P, const float* qs, int Dk) {
  constexpr int C = KV_FP8 ? 64 : 32;
  float acc = 0.0f;
  for (int c0 = 0; c0 < Dk; c0 += C) {
    const size_t row = block + (size_t)c0 * P + (size_t)slot * C;  // element offset of this chunk row
    if (KV_FP8) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>((const uint8_t*)k_pool + row);
#pragma unroll 4
      for (int d = 0; d < C; d += 4) {
        float f[4];
        fp8x4_to_f32(p[d >> 2], f);
        acc = fmaf(qs[c0 + d], f[0], acc);
        acc = fmaf(qs[c0 + d + 1], f[1], acc);
        acc = fmaf(qs[c0 + d + 2], f[2], acc);
        acc = fmaf(qs[c0 + d + 3], f[3], acc);
      }
    } else {
      const uint2* p = reinterpret_cast<const uint2*>((const uint16_t*)k_pool + row);
#pragma unroll 4
      for (int d = 0; d < C; d += 4) {
        const uint2 w = p[d >> 2];
        acc = fmaf(qs[c0 + d], __uint_as_float(w.x << 16), acc);
        acc = fmaf(qs[c0 + d + 1], __uint_as_float(w.x & 0xffff0000u), acc);
        acc = fmaf(qs[c0 + d + 2], __uint_as_float(w.y << 16), acc);
        acc = fmaf(qs[c0 + d + 3], __uint_as_float(w.y & 0xffff0000u), acc);
      }
    }
  }
  return acc;
}

template <bool KV_FP8>
__device__ __forceinline__ float kv_elem(const void* pool, size_t i) {
  if (KV_FP8) {
    const uint32_t c = ((const uint8_t*)pool)[i];
    return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
  }
  return bf16_to_f32(((const uint16_t*)pool)[i]);
}

template <bool KV_FP8>
__global__ __launch_bounds__(kGenThreads) void attn_generic_kernel(AttnArgs a) {
  __shared__ float scores[kGenMaxSplit];
  __shared__ int pages[kGenMaxSplit];
  __shared__ float qs[1024];
  __shared__ float red[kGenThreads];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / a.G;
  const int P = a.page_size;
  const int Lmax = a.pt_stride * P;
  const int L = min(max(a.seq_lens[b], 0), Lmax);
  const bool direct = a.nsplit == 1;
  const bool aborted = a.abort_mask && a.abort_mask[b];
  const int t0 = split * a.split;
  if (aborted || t0 >= L) {
    // Empty partition.  With a single partition this block owns the output row: write zeros.
    if (direct) {
      for (int d = threadIdx.x; d < a.Dv; d += kGenThreads) {
        const size_t o = ((size_t)b * a.Hq + h) * a.Dv + d;
        if (a.out_dt == DAPF8_ACT_BF16)
          ((uint16_t*)a.out)[o] = 0;
        else
          ((float*)a.out)[o] = 0.0f;
      }
    }
    return;
  }
  const int t1 = min(L, t0 + a.split);
  const int n = t1 - t0;

  const float ks = KV_FP8 ? a.k_scale[g] : 1.0f;
  const float vs = KV_FP8 ? (a.v_pool ? a.v_scale[g] : a.k_scale[g]) : 1.0f;
  const float c = a.sm_scale * ks * kLog2e;  // scores kept in the log2 domain

  for (int d = threadIdx.x; d < a.Dk; d += kGenThreads)
    qs[d] = load_act(a.q, a.q_dt, ((size_t)b * a.Hq + h) * a.Dk + d);
  const int p0 = t0 / P, p1 = (t1 - 1) / P;
  for (int j = p0 + (int)threadIdx.x; j <= p1; j += kGenThreads) {
    const int pg = a.page_table[(size_t)b * a.pt_stride + j];
    pages[j - p0] = (int)min((unsigned)pg, (unsigned)(a.num_pages - 1));  // stay inside the pool
  }
  __syncthreads();

  float mx = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kGenThreads) {
    const int t = t0 + i;
    const int pg = pages[t / P - p0];
    const size_t block = ((size_t)pg * a.Hkv + g) * (size_t)P * a.Dk;
    const float s = dot_row<KV_FP8>(a.k_pool, block, t % P, P, qs, a.Dk) * c;
    scores[i] = s;
    mx = fmaxf(mx, s);
  }
  const float m = wg_reduce(mx, red, true);
  float sum = 0.0f;
  for (int i = threadIdx.x; i < n; i += kGenThreads) {
    const float p = exp2f(scores[i] - m);
    scores[i] = p;
    sum += p;
  }
  const float l = wg_reduce(sum, red, false);  // also orders the score writes before the reads below

  for (int d = threadIdx.x; d < a.Dv; d += kGenThreads) {
    float acc = 0.0f;
    for (int i = 0; i < n; ++i) {
      const int t = t0 + i;
      const int pg = pages[t / P - p0];
      const int slot = t % P;
      size_t idx;
      if (a.v_pool)
        idx = (((size_t)pg * a.Hkv + g) * a.Dv + d) * P + slot;
      else
        idx = k_elem_offset(pg, g, slot, d, a.Hkv, P, a.Dk, KV_FP8 ? 64 : 32);
      acc = fmaf(scores[i], kv_elem<KV_FP8>(a.v_pool ? a.v_pool : a.k_pool, idx), acc);
    }
    acc *= vs;
    if (direct) {
      const float o = acc / l;
      const size_t oi = ((size_t)b * a.Hq + h) * a.Dv + d;
      if (a.out_dt == DAPF8_ACT_BF16)
        ((uint16_t*)a.out)[oi] = f32_to_bf16_rne(o);
      else
        ((float*)a.out)[oi] = o;
    } else {
      a.ws_o[(((size_t)b * a.Hq + h) * a.nsplit + split) * a.Dv + d] = acc;
    }
  }
  if (!direct && threadIdx.x == 0) {
    float* ml = a.ws_ml + (((size_t)b * a.Hq + h) * a.nsplit + split) * 2;
    ml[0] = m;
    ml[1] = l;
  }
}

int launch_attn_generic(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hq, (unsigned)a.B);
  if (a.kv_dt == DAPF8_KV_FP8_E4M3)
    hipLaunchKernelGGL(attn_generic_kernel<true>, grid, dim3(kGenThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<false>, grid, dim3(kGenThreads), 0, s, a);
  return check_launch("paged_decode_attn (generic)");
}

// ------------------------------------------------------------------------------------------------
// merge: one workgroup per (sequence, query head).  Partition i of a length-L sequence covers
// tokens [i*split, (i+1)*split); its (m_i, l_i, o_i) are combined as
//   M = max m_i,  out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i   (log2-domain scores).
__global__ __launch_bounds__(128) void merge_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(max(a.seq_lens[b], 0), a.pt_stride * a.page_size);
  const bool aborted = a.abort_mask && a.abort_mask[b];
  const int np = (aborted || L == 0) ? 0 : (L + a.split - 1) / a.split;
  const size_t row = (size_t)b * a.Hq + h;
  const float* ml = a.ws_ml + row * a.nsplit * 2;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, ml[2 * i]);
  float den = 0.0f;
  for (int i = 0; i < np; ++i) den += exp2f(ml[2 * i] - M) * ml[2 * i + 1];
  const float* o = a.ws_o + row * a.nsplit * a.Dv;
  for (int d = threadIdx.x; d < a.Dv; d += blockDim.x) {
    float num = 0.0f;
    for (int i = 0; i < np; ++i) num += exp2f(ml[2 * i] - M) * o[(size_t)i * a.Dv + d];
    const float r = np ? num / den : 0.0f;
    if (a.out_dt == DAPF8_ACT_BF16)
      ((uint16_t*)a.out)[row * a.Dv + d] = f32_to_bf16_rne(r);
    else
      ((float*)a.out)[row * a.Dv + d] = r;
  }
}

int launch_merge(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.Hq, (unsigned)a.B), dim3(128), 0, s, a);
  return check_launch("paged_decode_attn (merge)");
}

}  // namespace dapf8
