// attn_mfma.hip -- decode attention on the gfx950 matrix cores for G <= 16 query heads per KV head,
// head dim 128, page size 16, separate K and V pools, FP8 (e4m3) or BF16 storage.
//
// [CF §Quantize] the FP8 kernel converts stored values on read: each lane converts its e4m3 bytes
// to bf16 with the hardware conversion (exact), the per-head scales are applied to the fp32 score
// and output, and both products run as v_mfma_f32_16x16x32_bf16.
//
// Work decomposition.  One workgroup (4 waves) owns one (sequence b, KV head g, partition of
// `split` tokens).  The partition is walked in segments of <= 4096 tokens; each wave takes a
// contiguous quarter of a segment and walks it in windows of 32 tokens (two 16-token pages),
// keeping its own running max / sum / output; the four waves are merged through LDS at the end.
// The K/V data of a window is consumed by exactly one wave, so it goes from HBM straight to
// registers (no LDS staging); the next window's loads are issued before the current one is used.
//
// Register layouts (16x16x32 bf16 MFMA: A row = lane%16, B column = lane%16, the 8 k-values a
// lane holds belong to k-group lane/16, D[row][col] sits in lane col+16*(row/4), element row%4):
//   S^T = K Q^T   A = K tile (16 tokens x 32 dims), B = Q^T (32 dims x 16 heads).  Lane l loads
//                 32 contiguous dims [32*(l/16), +32) of one token row; chunk c of the contraction
//                 uses its dims 8c..8c+7.  Q is loaded with the same dimension permutation.
//                 Tile a (0/1) row r holds window token 8*(r/4) + 4a + r%4, so lane l ends up with
//                 the scores of tokens 8*(l/16) .. +7 for head l%16.
//   O^T = V^T P^T A = V^T block (16 dims x 32 tokens), B = P^T (32 tokens x 16 heads).  The V pool
//                 is dimension-major inside a page, so lane l loads the 8 contiguous values of
//                 dimension 16*blk + l%16 for window tokens 8*(l/16) .. +7 -- exactly the tokens
//                 whose probabilities the lane already holds from S^T.  No shuffles are needed
//                 between the two products.  O^T block blk: lane l holds head l%16, dims
//                 16*blk + 4*(l/16) .. +3.
// P is split into 1-3 bf16 terms (p = p1 + p2 + p3) so that P*V keeps ~8, ~16 or ~24 bits.
#include "common.hpp"

namespace dapf8 {

namespace {

constexpr int kD = 128;
constexpr int kP = 16;
constexpr int kSeg = 4096;  // tokens per segment: a wave's quarter spans <= 64 pages (one VGPR of ids)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct KvRegs {
  u32x4 k[2][4];  // [tile][16-byte piece]: FP8 uses pieces 0..1 (32 dims), BF16 pieces 0..3
  u32x4 v[8];     // [dim block]: FP8 uses .x/.y (8 tokens), BF16 all four dwords
};

template <bool KV_FP8>
__device__ __forceinline__ void load_window(KvRegs& r, const uint8_t* __restrict__ kbase,
                                            const uint8_t* __restrict__ vbase, int pA, int pB, int lane, int Hkv) {
  const int row = lane & 15, grp = lane >> 4;
  constexpr int el = KV_FP8 ? 1 : 2;
  // K: this lane's token rows in tiles 0 and 1 share the page (rows 0-7 -> first page)
  const int kpage = row < 8 ? pA : pB;
  const size_t kblock = (size_t)kpage * Hkv * (kP * kD * el);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tok = 8 * (row >> 2) + 4 * a + (row & 3);
    const u32x4* src = reinterpret_cast<const u32x4*>(kbase + kblock + (size_t)((tok & 15) * kD + 32 * grp) * el);
    r.k[a][0] = src[0];
    r.k[a][1] = src[1];
    if (!KV_FP8) {
      r.k[a][2] = src[2];
      r.k[a][3] = src[3];
    }
  }
  // V: tokens 8*grp .. 8*grp+7 of the window, dimension 16*blk + row
  const int vpage = grp < 2 ? pA : pB;
  const size_t vblock = (size_t)vpage * Hkv * (kD * kP * el);
  const int slot0 = 8 * (grp & 1);
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const uint8_t* src = vbase + vblock + (size_t)((16 * blk + row) * kP + slot0) * el;
    if (KV_FP8) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(src);
      r.v[blk].x = w.x;
      r.v[blk].y = w.y;
    } else {
      r.v[blk] = *reinterpret_cast<const u32x4*>(src);
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, u);
}

// 8 e4m3 codes (two dwords) -> bf16x8
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const uint2 lo = fp8x4_to_bf16x4(w0);
  const uint2 hi = fp8x4_to_bf16x4(w1);
  return as_bf16x8(lo.x, lo.y, hi.x, hi.y);
}

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Split fp32 values into NT bf16 terms (round to nearest even each time).
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

}  // namespace

template <bool KV_FP8, int QSPLIT, int PSPLIT, bool DIRECT, bool OUT_BF16>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a) {
  __shared__ float sm_o[4][16][kD + 4];
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.G;
  const int L = min(max(a.seq_lens[b], 0), a.pt_stride * kP);
  const bool aborted = a.abort_mask && a.abort_mask[b];
  const int t0 = split * a.split;
  if (aborted || t0 >= L) {
    if (DIRECT) {  // this block owns the output rows of (b, kvh): write zeros
      for (int i = threadIdx.x; i < G * kD; i += 256) {
        const size_t o = ((size_t)b * a.Hq + kvh * G) * kD + i;
        if (OUT_BF16)
          ((uint16_t*)a.out)[o] = 0;
        else
          ((float*)a.out)[o] = 0.0f;
      }
    }
    return;
  }
  const int t1 = min(L, t0 + a.split);
  const int row = lane & 15, grp = lane >> 4;
  const int gq = row;  // query head handled by this lane's column

  const float ks = KV_FP8 ? a.k_scale[kvh] : 1.0f;
  const float vs = KV_FP8 ? a.v_scale[kvh] : 1.0f;
  const float c = a.sm_scale * ks * kLog2e;

  // Q^T operand: chunk cc holds dims 32*grp + 8*cc .. +7 of head gq (zeros for gq >= G)
  bf16x8 qop[QSPLIT][4];
  {
    const size_t qrow = ((size_t)b * a.Hq + kvh * G + gq) * kD + 32 * grp;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      float f[8];
      if (gq < G) {
        if (QSPLIT == 1) {
          const u32x4 w = *reinterpret_cast<const u32x4*>((const uint16_t*)a.q + qrow + 8 * cc);
          qop[0][cc] = __builtin_bit_cast(bf16x8, w);
          continue;
        }
        const float4* src = reinterpret_cast<const float4*>((const float*)a.q + qrow + 8 * cc);
        const float4 x0 = src[0], x1 = src[1];
        f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
        f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = 0.0f;
      }
      bf16x8 parts[QSPLIT];
      split_bf16<QSPLIT>(f, parts);
#pragma unroll
      for (int t = 0; t < QSPLIT; ++t) qop[t][cc] = parts[t];
    }
  }

  const uint8_t* kbase = (const uint8_t*)a.k_pool + (size_t)kvh * (kP * kD * (KV_FP8 ? 1 : 2));
  const uint8_t* vbase = (const uint8_t*)a.v_pool + (size_t)kvh * (kD * kP * (KV_FP8 ? 1 : 2));
  const int32_t* ptrow = a.page_table + (size_t)b * a.pt_stride;
  const unsigned last_page = (unsigned)(a.num_pages - 1);

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc_o[8];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) acc_o[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int seg0 = t0; seg0 < t1; seg0 += kSeg) {
    const int seg1 = min(t1, seg0 + kSeg);
    const int nw = (seg1 - seg0 + 31) >> 5;
    const int qw = (nw + 3) >> 2;
    const int w_begin = wave * qw;
    const int my_nwin = max(0, min(nw, w_begin + qw) - w_begin);
    if (my_nwin == 0) continue;  // wave-uniform
    const int ws = seg0 + 32 * w_begin;  // first token of this wave's range (multiple of 32)
    // page ids of this wave's range: lane i <- entry ws/16 + i (clamped into the pool)
    int ptv = 0;
    {
      const int e = (ws >> 4) + lane;
      if (lane < 2 * my_nwin && e < a.pt_stride) ptv = (int)min((unsigned)ptrow[e], last_page);
    }
    KvRegs cur, nxt;
    load_window<KV_FP8>(cur, kbase, vbase, __builtin_amdgcn_readlane(ptv, 0), __builtin_amdgcn_readlane(ptv, 1),
                        lane, a.Hkv);
    for (int w = 0; w < my_nwin; ++w) {
      if (w + 1 < my_nwin)
        load_window<KV_FP8>(nxt, kbase, vbase, __builtin_amdgcn_readlane(ptv, 2 * w + 2),
                            __builtin_amdgcn_readlane(ptv, 2 * w + 3), lane, a.Hkv);
      const int nvalid = min(32, t1 - (ws + 32 * w));

      // ---- S^T = K Q^T for the 32 tokens of the window (two 16-token tiles)
      f32x4 acc_s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 kop;
          if (KV_FP8) {
            const u32x4 w4 = cur.k[t][cc >> 1];
            kop = (cc & 1) ? fp8x8_to_bf16x8(w4.z, w4.w) : fp8x8_to_bf16x8(w4.x, w4.y);
          } else {
            kop = __builtin_bit_cast(bf16x8, cur.k[t][cc]);
          }
#pragma unroll
          for (int qs = 0; qs < QSPLIT; ++qs)
            acc_s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[qs][cc], acc_s[t], 0, 0, 0);
        }
      }

      // ---- online softmax (log2 domain); lane holds tokens 8*grp + i of head gq
      float s[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = acc_s[0][i] * c;
        s[4 + i] = acc_s[1][i] * c;
      }
      const int nv_lane = nvalid - 8 * grp;  // valid tokens among this lane's 8
      if (nvalid < 32) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i >= nv_lane) s[i] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
      mx = xor_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float p[8];
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2f(s[i] - m_new);
        psum += p[i];
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) acc_o[blk] *= alpha;
      bf16x8 pop[PSPLIT];
      split_bf16<PSPLIT>(p, pop);

      // ---- O^T += V^T P^T, one 16-dim block at a time
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        bf16x8 vop;
        if (KV_FP8) {
          vop = fp8x8_to_bf16x8(cur.v[blk].x, cur.v[blk].y);
        } else {
          vop = __builtin_bit_cast(bf16x8, cur.v[blk]);
        }
        if (nvalid < 32) {  // stale slots past the sequence end may hold anything: zero them
          u32x4 u = __builtin_bit_cast(u32x4, vop);
          u.x &= nv_lane > 1 ? 0xffffffffu : (nv_lane > 0 ? 0x0000ffffu : 0u);
          u.y &= nv_lane > 3 ? 0xffffffffu : (nv_lane > 2 ? 0x0000ffffu : 0u);
          u.z &= nv_lane > 5 ? 0xffffffffu : (nv_lane > 4 ? 0x0000ffffu : 0u);
          u.w &= nv_lane > 7 ? 0xffffffffu : (nv_lane > 6 ? 0x0000ffffu : 0u);
          vop = __builtin_bit_cast(bf16x8, u);
        }
#pragma unroll
        for (int t = 0; t < PSPLIT; ++t)
          acc_o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t], acc_o[blk], 0, 0, 0);
      }
      if (w + 1 < my_nwin) cur = nxt;
    }
  }

  // ---- merge the four waves through LDS
  const float l_tot = xor_sum(l_run);
  if (grp == 0) {
    sm_m[wave][gq] = m_run;
    sm_l[wave][gq] = l_tot;
  }
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[wave][gq][16 * blk + 4 * grp + i] = acc_o[blk][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
    const int g = idx >> 7, d = idx & (kD - 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][g]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = exp2f(sm_m[w][g] - M);  // waves without windows carry m = -inf -> weight 0
      den += e * sm_l[w][g];
      num += e * sm_o[w][g][d];
    }
    const int h = kvh * G + g;
    if (DIRECT) {
      const float o = num / den * vs;
      const size_t oi = ((size_t)b * a.Hq + h) * kD + d;
      if (OUT_BF16)
        ((uint16_t*)a.out)[oi] = f32_to_bf16_rne(o);
      else
        ((float*)a.out)[oi] = o;
    } else {
      const size_t r = ((size_t)b * a.Hq + h) * a.nsplit + split;
      a.ws_o[r * kD + d] = num * vs;
      if (d == 0) {
        a.ws_ml[2 * r] = M;
        a.ws_ml[2 * r + 1] = den;
      }
    }
  }
}

int launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B), block(256);
  const bool fp8 = a.kv_dt == DAPF8_KV_FP8_E4M3;
  const bool qf32 = a.q_dt == DAPF8_ACT_F32;
  const bool direct = a.nsplit == 1;
  const bool obf = a.out_dt == DAPF8_ACT_BF16;
  // P keeps ~16 bits for bf16 outputs and ~24 bits for fp32 outputs; fp32 queries keep ~24 bits.
#define DAPF8_MFMA(F, QS, PS, DI, OB) hipLaunchKernelGGL((attn_mfma_kernel<F, QS, PS, DI, OB>), grid, block, 0, s, a)
#define DAPF8_MFMA_OUT(F, QS)                    \
  if (direct && obf)                             \
    DAPF8_MFMA(F, QS, 2, true, true);            \
  else if (direct)                               \
    DAPF8_MFMA(F, QS, 3, true, false);           \
  else if (obf)                                  \
    DAPF8_MFMA(F, QS, 2, false, false);          \
  else                                           \
    DAPF8_MFMA(F, QS, 3, false, false);
  if (fp8) {
    if (qf32) {
      DAPF8_MFMA_OUT(true, 3)
    } else {
      DAPF8_MFMA_OUT(true, 1)
    }
  } else {
    if (qf32) {
      DAPF8_MFMA_OUT(false, 3)
    } else {
      DAPF8_MFMA_OUT(false, 1)
    }
  }
#undef DAPF8_MFMA_OUT
#undef DAPF8_MFMA
  return check_launch("paged_decode_attn (mfma)");
}

}  // namespace dapf8
