// attn_generic.hip -- shape-general decode attention on the vector ALUs, plus the split merge.
//
// [CF §Quantize] decode attention over the paged cache; stored FP8 values are converted on read
// (hardware e4m3 -> fp32 conversion) and the per-head scales are folded into the score and the
// output.  Used for shapes the matrix-core kernels do not cover (Dk a multiple of 64, Dv a multiple
// of 16, both up to 1024, any page size, shared-KV, fp32 queries on the latent shape).
//
// One workgroup (4 waves) handles one (sequence, KV head, partition) and a group of up to GB of the
// G query heads that share the KV head, so K and V are read once for all of them:
//   scores   4-lane groups take one token row each: lane j of a group holds 16 bytes of every 64-byte
//            dimension chunk of the row (coalesced: a group reads whole chunks), multiplies them by
//            the query values of its dims for each head (queries in LDS) and the group's partial
//            sums meet through two DPP quad permutations -- no LDS round trip and no barrier.
//            Scores go to LDS.
//   softmax  each wave takes heads; its lanes stride over the partition's scores, and max / sum
//            are wave reductions (DPP within 16-lane rows, then lane shuffles across rows).
//   P.V      threads take (output dimension, token slice); the V pool is dimension-major inside a
//            page, so a thread reads 4 consecutive tokens of its dimension per load where the page
//            size allows; the probabilities come from LDS as broadcast reads, and the slices' partial
//            sums meet in LDS.
// Partition results are (max, sum, unnormalised output) in the log2 domain, merged by merge_kernel.
#include <mutex>

#include "common.hpp"

namespace dapf8 {

constexpr int kGenThreads = 256;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum / max over each 16-lane row (every lane of the row gets the result)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: the other quad of each 8
  return v + dpp<0x140>(v);  // row_mirror: the other 8 of the row
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return fmaxf(v, dpp<0x140>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

template <bool KV_FP8>
__device__ __forceinline__ void kv4(const void* pool, size_t i, float* f) {  // 4 consecutive values
  if (KV_FP8) {
    fp8x4_to_f32(*reinterpret_cast<const uint32_t*>((const uint8_t*)pool + i), f);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>((const uint16_t*)pool + i);
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
  }
}

template <bool KV_FP8>
__device__ __forceinline__ float kv_elem(const void* pool, size_t i) {
  if (KV_FP8) {
    const uint32_t c = ((const uint8_t*)pool)[i];
    return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
  }
  return bf16_to_f32(((const uint16_t*)pool)[i]);
}

// LDS of one workgroup, sized per launch (dynamic shared memory): scores [gb][split], query values
// [gb][Dk] (reused for the P.V slices' partial sums, kGenThreads * kGenMaxGB floats), page ids of the
// partition.
struct GenLds {
  int sc, qs, pages, bytes;  // offsets (floats / ints) and total size
};
__host__ __device__ inline GenLds gen_lds(int gb, int split, int Dk, int P) {
  GenLds L;
  L.sc = 0;
  L.qs = gb * split;
  const int q = max(gb * Dk, kGenThreads * kGenMaxGB);
  L.pages = L.qs + q;
  L.bytes = (L.pages + (split + P - 1) / P + 2) * 4;
  return L;
}

template <bool KV_FP8>
__global__ __launch_bounds__(kGenThreads) void attn_generic_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds_gen[];
  __shared__ float mls[2][kGenMaxGB];
  const GenLds lay = gen_lds(a.gb, a.split, a.Dk, a.page_size);
  float* const sc = lds_gen + lay.sc;
  float* const qs = lds_gen + lay.qs;
  int* const pages = reinterpret_cast<int*>(lds_gen + lay.pages);

  const int GB = a.gb, ngb = (a.G + GB - 1) / GB;
  const int split = blockIdx.x, g = blockIdx.y / ngb, h0 = g * a.G + (blockIdx.y % ngb) * GB;
  const int nh = min(GB, g * a.G + a.G - h0);  // heads of this workgroup: h0 .. h0 + nh - 1
  const int b = blockIdx.z;
  const int P = a.page_size, Dk = a.Dk, Dv = a.Dv;
  const int Lmax = a.pt_stride * P;
  const int L = min(max(a.seq_lens[b], 0), Lmax);
  const bool direct = a.nsplit == 1;
  const bool aborted = a.abort_mask && a.abort_mask[b];
  const int t0 = split * a.split;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (aborted || t0 >= L) {
    // Empty partition.  With a single partition this block owns the output rows: write zeros.
    if (direct) {
      for (int i = tid; i < nh * Dv; i += kGenThreads) {
        const size_t o = ((size_t)b * a.Hq + h0) * Dv + i;
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

  for (int i = tid; i < nh * Dk; i += kGenThreads) qs[i] = load_act(a.q, a.q_dt, ((size_t)b * a.Hq + h0) * Dk + i);
  const int p0 = t0 / P, p1 = (t1 - 1) / P;
  for (int j = p0 + tid; j <= p1; j += kGenThreads) {
    const int pg = a.page_table[(size_t)b * a.pt_stride + j];
    pages[j - p0] = (int)min((unsigned)pg, (unsigned)(a.num_pages - 1));  // stay inside the pool
  }
  __syncthreads();

  // ---- scores: 4-lane group q takes tokens q, q + 64, ...; lane j of the group holds bytes 16j ..
  // 16j+15 of each 64-byte chunk of the row (FP8: dims 64 c + 16 j .. +15; BF16: dims 32 c + 8 j .. +7)
  {
    constexpr int C = KV_FP8 ? 64 : 32;   // dims per 64-byte chunk
    constexpr int DPL = KV_FP8 ? 16 : 8;  // dims per lane per chunk
    const int grp = tid >> 2, j = tid & 3;
#pragma unroll 2
    for (int i = grp; i < n; i += kGenThreads / 4) {  // group-uniform trip count
      const int t = t0 + i;
      const int slot = t % P;
      const size_t block = ((size_t)pages[t / P - p0] * a.Hkv + g) * (size_t)P * Dk;
      float acc[kGenMaxGB];
#pragma unroll
      for (int hh = 0; hh < kGenMaxGB; ++hh) acc[hh] = 0.0f;
      for (int c0 = 0; c0 < Dk; c0 += C) {
        float f[16];
        const size_t e = block + (size_t)c0 * P + (size_t)slot * C + DPL * j;  // element offset
        const uint4 w = *reinterpret_cast<const uint4*>(KV_FP8 ? (const void*)((const uint8_t*)a.k_pool + e)
                                                                : (const void*)((const uint16_t*)a.k_pool + e));
        if (KV_FP8) {
          fp8x4_to_f32(w.x, f);
          fp8x4_to_f32(w.y, f + 4);
          fp8x4_to_f32(w.z, f + 8);
          fp8x4_to_f32(w.w, f + 12);
        } else {
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(u[k] << 16);
            f[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
          }
        }
        const int d0 = c0 + DPL * j;
#pragma unroll
        for (int hh = 0; hh < kGenMaxGB; ++hh) {
          if (hh < nh) {
            const float4* qq = reinterpret_cast<const float4*>(qs + hh * Dk + d0);
            float s0 = acc[hh];
#pragma unroll
            for (int u = 0; u < DPL / 4; ++u) {
              const float4 qv = qq[u];
              s0 = fmaf(qv.x, f[4 * u], s0);
              s0 = fmaf(qv.y, f[4 * u + 1], s0);
              s0 = fmaf(qv.z, f[4 * u + 2], s0);
              s0 = fmaf(qv.w, f[4 * u + 3], s0);
            }
            acc[hh] = s0;
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < kGenMaxGB; ++hh) {
        if (hh < nh) {
          float s0 = acc[hh];
          s0 += dpp<0xB1>(s0);  // quad_perm [1,0,3,2]
          s0 += dpp<0x4E>(s0);  // quad_perm [2,3,0,1]: the group's sum in all four lanes
          if (j == 0) sc[hh * a.split + i] = s0 * c;
        }
      }
    }
  }
  __syncthreads();

  // ---- softmax of each head over the partition: wave w takes heads w, w + 4, ...
  for (int hh = wave; hh < nh; hh += kGenThreads / 64) {
    float* row = sc + hh * a.split;
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) mx = fmaxf(mx, row[i]);
    const float m = wave_max(mx);
    float sum = 0.0f;
    for (int i = lane; i < n; i += 64) {
      const float p = exp2f(row[i] - m);
      row[i] = p;
      sum += p;
    }
    const float l = wave_sum(sum);
    if (lane == 0) {
      mls[0][hh] = m;
      mls[1][hh] = l;
    }
  }
  __syncthreads();

  // ---- P.V: threads take (dimension, token slice): Dv' = min(Dv, 256) dims per pass and NS =
  // 256 / Dv' contiguous slices of the partition's tokens, 4 consecutive tokens of a dimension per
  // load where they share a page (separate V pool, page size a multiple of 4); the slices' partial
  // sums meet in LDS (the query buffer, free by now).
  const int Dvp = min(Dv, kGenThreads), NS = kGenThreads / Dvp;
  const int slice = tid / Dvp;
  const int per = (((n + NS - 1) / NS) + 3) & ~3;  // tokens per slice, a multiple of 4
  const int i0 = min(n, slice * per), i1 = min(n, i0 + per);
  for (int dbase = 0; dbase < Dv; dbase += Dvp) {
    const int d = dbase + tid % Dvp;
    const bool active = slice < NS && d < Dv;
    float acc[kGenMaxGB];
#pragma unroll
    for (int hh = 0; hh < kGenMaxGB; ++hh) acc[hh] = 0.0f;
    if (active) {
      auto add = [&](int i, float v) __attribute__((always_inline)) {
#pragma unroll
        for (int hh = 0; hh < kGenMaxGB; ++hh)
          if (hh < nh) acc[hh] = fmaf(sc[hh * a.split + i], v, acc[hh]);
      };
      auto velem = [&](int i) __attribute__((always_inline)) {
        const int t = t0 + i, pg = pages[t / P - p0], slot = t % P;
        const size_t idx = a.v_pool ? (((size_t)pg * a.Hkv + g) * Dv + d) * P + slot
                                    : k_elem_offset(pg, g, slot, d, a.Hkv, P, Dk, KV_FP8 ? 64 : 32);
        return kv_elem<KV_FP8>(a.v_pool ? a.v_pool : a.k_pool, idx);
      };
      int i = i0;
      if (a.v_pool && P % 4 == 0) {
        for (; i < i1 && (t0 + i) % 4 != 0; ++i) add(i, velem(i));  // up to the first 4-aligned token
        auto v4 = [&](int ii, float* f) __attribute__((always_inline)) {
          const int t = t0 + ii;
          kv4<KV_FP8>(a.v_pool, (((size_t)pages[t / P - p0] * a.Hkv + g) * Dv + d) * P + t % P, f);
        };
        auto fma4 = [&](int ii, const float* f) __attribute__((always_inline)) {
#pragma unroll
          for (int hh = 0; hh < kGenMaxGB; ++hh) {
            if (hh < nh) {
              const float4 pr = *reinterpret_cast<const float4*>(sc + hh * a.split + ii);
              acc[hh] = fmaf(pr.x, f[0], fmaf(pr.y, f[1], fmaf(pr.z, f[2], fmaf(pr.w, f[3], acc[hh]))));
            }
          }
        };
        for (; i + 16 <= i1; i += 16) {  // four loads in flight
          float f[4][4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v4(i + 4 * u, f[u]);
#pragma unroll
          for (int u = 0; u < 4; ++u) fma4(i + 4 * u, f[u]);
        }
        for (; i + 4 <= i1; i += 4) {
          float f[4];
          v4(i, f);
          fma4(i, f);
        }
      }
      for (; i < i1; ++i) add(i, velem(i));
    }
    __syncthreads();  // every slice done with the previous pass's sums in qs
    if (active)
#pragma unroll
      for (int hh = 0; hh < kGenMaxGB; ++hh)
        if (hh < nh) qs[(slice * kGenMaxGB + hh) * Dvp + tid % Dvp] = acc[hh];
    __syncthreads();
    for (int x = tid; x < nh * Dvp; x += kGenThreads) {
      const int hh = x / Dvp, dd = x - hh * Dvp, dv = dbase + dd;
      if (dv >= Dv) continue;
      float o = 0.0f;
      for (int sl = 0; sl < NS; ++sl) o += qs[(sl * kGenMaxGB + hh) * Dvp + dd];
      o *= vs;
      const int h = h0 + hh;
      if (direct) {
        const size_t oi = ((size_t)b * a.Hq + h) * Dv + dv;
        if (a.out_dt == DAPF8_ACT_BF16)
          ((uint16_t*)a.out)[oi] = f32_to_bf16_rne(o / mls[1][hh]);
        else
          ((float*)a.out)[oi] = o / mls[1][hh];
      } else {
        a.ws_o[(((size_t)b * a.Hq + h) * a.nsplit + split) * Dv + dv] = o;
      }
    }
  }
  if (!direct && tid < nh) {
    float* ml = a.ws_ml + (((size_t)b * a.Hq + h0 + tid) * a.nsplit + split) * 2;
    ml[0] = mls[0][tid];
    ml[1] = mls[1][tid];
  }
}

int launch_attn_generic(const AttnArgs& a, hipStream_t s) {
  if (a.gb < 1 || a.gb > kGenMaxGB || a.gb * a.split > kGenScoreFloats || a.gb * a.Dk > kGenQFloats ||
      a.split > kGenericMaxSplit)
    return set_error(DAPF8_EUNSUPPORTED, "paged_decode_attn (generic): unsupported partition of %d tokens for %d heads",
                     a.split, a.gb);
  const int ngb = (a.G + a.gb - 1) / a.gb;
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.Hkv * ngb), (unsigned)a.B);
  if (grid.y > 65535) return set_error(DAPF8_EUNSUPPORTED, "paged_decode_attn (generic): too many head groups");
  const size_t lds = (size_t)gen_lds(a.gb, a.split, a.Dk, a.page_size).bytes;  // < 96 KB for the limits above
  // allow more than the default 64 KB of dynamic LDS (once per process; the limit is per function)
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute((const void*)attn_generic_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              96 * 1024);
    (void)hipFuncSetAttribute((const void*)attn_generic_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              96 * 1024);
  });
  if (a.kv_dt == DAPF8_KV_FP8_E4M3)
    hipLaunchKernelGGL(attn_generic_kernel<true>, grid, dim3(kGenThreads), lds, s, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<false>, grid, dim3(kGenThreads), lds, s, a);
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
