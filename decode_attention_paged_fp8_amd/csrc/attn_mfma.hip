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
//   S^T = K Q^T   A = K tile (16 tokens x 32 dims), B = Q^T (32 dims x 16 heads).  Contraction
//                 chunk c of lane l covers 8 dims starting at dim0(c, l/16) (see k_dim0): the four
//                 lanes of a token row read one contiguous 64-byte run per load instruction.  Q is
//                 loaded with the same dimension permutation.
//                 Tile a (0/1) row r holds window token 8*(r/4) + 4a + r%4, so lane l ends up with
//                 the scores of tokens 8*(l/16) .. +7 for head l%16.
//   O^T = V^T P^T A = V^T block (16 dims x 32 tokens), B = P^T (32 tokens x 16 heads).  The V pool
//                 is dimension-major inside a page, so lane l loads the 8 contiguous values of
//                 dimension 16*blk + l%16 for window tokens 8*(l/16) .. +7 -- exactly the tokens
//                 whose probabilities the lane already holds from S^T.  No shuffles are needed
//                 between the two products.  O^T block blk: lane l holds head l%16, dims
//                 16*blk + 4*(l/16) .. +3.
// P is split into 1 or 3 bf16 terms (p = p1 + p2 + p3) so that P*V keeps ~8 or ~24 bits.
#include <atomic>

#include "mfma_util.hpp"

namespace dapf8 {

namespace {

constexpr int kD = 128;
constexpr int kP = 16;
constexpr int kSeg = 4096;  // tokens per segment: a wave's quarter spans <= 64 pages (one VGPR of ids)

struct KvRegs {
  u32x4 k[2][4];  // [tile][16-byte piece]: FP8 uses pieces 0..1 (32 dims), BF16 pieces 0..3
  u32x4 v[8];     // [dim block]: FP8 uses .x/.y (8 tokens), BF16 all four dwords
};

// First of the 8 dims that contraction chunk cc (0..3) of k-group grp covers.  A lane reads one
// 16-byte piece from each 64-byte dimension chunk p of its token row: FP8 dims 64p + 16*grp .. +15
// (two chunks), BF16 dims 32p + 8*grp .. +7 (four chunks).  K and V are streamed with non-temporal
// loads, and every load instruction covers whole 128-byte lines (16 tokens x 64 B of a chunk for
// K, 16 dimensions x 16 tokens for V).
template <bool KV_FP8>
__device__ __forceinline__ int k_dim0(int cc, int grp) {
  return KV_FP8 ? 64 * (cc >> 1) + 16 * grp + 8 * (cc & 1) : 32 * cc + 8 * grp;
}

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
    // 64-byte dimension chunk p of this token row sits at p * (16 tokens * 64 B) + token * 64 B
    const uint8_t* cp = kbase + kblock + (size_t)(tok & 15) * 64 + 16 * grp;
#pragma unroll
    for (int p = 0; p < 2 * el; ++p)
      r.k[a][p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cp + p * (kP * 64)));
  }
  // V: tokens 8*grp .. 8*grp+7 of the window, dimension 16*blk + row
  const int vpage = grp < 2 ? pA : pB;
  const size_t vblock = (size_t)vpage * Hkv * (kD * kP * el);
  const int slot0 = 8 * (grp & 1);
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const uint8_t* src = vbase + vblock + (size_t)((16 * blk + row) * kP + slot0) * el;
    if (KV_FP8) {
      const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
      r.v[blk].x = w.x;
      r.v[blk].y = w.y;
    } else {
      r.v[blk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
  }
}

}  // namespace

// Running softmax state of one wave.  m is the reference max (per lane: head row%16, replicated
// over the four k-groups), l the lane's partial sum and o the unnormalised O^T blocks -- all
// relative to 2^m.
struct WaveState {
  float m, l;
  f32x4 o[8];
};


// One 32-token window: S^T = K Q^T, online-softmax update, O^T += V^T P^T.  MASKED handles the
// sequence's last window, whose slots past the end may hold anything.
template <bool KV_FP8, int QSPLIT, int PSPLIT, bool MASKED>
__device__ __forceinline__ void process_window(WaveState& st, const KvRegs& r, const bf16x8 (&qop)[QSPLIT][4],
                                               float c, int nvalid, int grp) {
  f32x4 acc_s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 kop;
      if (KV_FP8) {
        const u32x4 w4 = r.k[t][cc >> 1];
        kop = (cc & 1) ? fp8x8_to_bf16x8(w4.z, w4.w) : fp8x8_to_bf16x8(w4.x, w4.y);
      } else {
        kop = __builtin_bit_cast(bf16x8, r.k[t][cc]);
      }
#pragma unroll
      for (int qs = 0; qs < QSPLIT; ++qs)
        acc_s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[qs][cc], acc_s[t], 0, 0, 0);
    }
  }
  // scores in the log2 domain; this lane holds window tokens 8*grp + i of its head
  float s[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = acc_s[0][i] * c;
    s[4 + i] = acc_s[1][i] * c;
  }
  const int nv_lane = nvalid - 8 * grp;  // valid tokens among this lane's 8
  if (MASKED) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i >= nv_lane) s[i] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  mx = xor_max(mx);
  // raise the reference only when needed (wave-uniform decision)
  if (__builtin_expect(__any(mx > st.m + kRescaleSlack), 0)) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 on the first window (m = -inf)
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) st.o[blk] *= alpha;
  }
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - st.m);  // masked: exp2(-inf) = 0
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  bf16x8 pop[PSPLIT];
  split_bf16<PSPLIT>(p, pop);
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    bf16x8 vop;
    if (KV_FP8)
      vop = fp8x8_to_bf16x8(r.v[blk].x, r.v[blk].y);
    else
      vop = __builtin_bit_cast(bf16x8, r.v[blk]);
    if (MASKED) {  // zero the values of slots past the end (a stale NaN times 0 would be NaN)
      u32x4 u = __builtin_bit_cast(u32x4, vop);
      u.x &= nv_lane > 1 ? 0xffffffffu : (nv_lane > 0 ? 0x0000ffffu : 0u);
      u.y &= nv_lane > 3 ? 0xffffffffu : (nv_lane > 2 ? 0x0000ffffu : 0u);
      u.z &= nv_lane > 5 ? 0xffffffffu : (nv_lane > 4 ? 0x0000ffffu : 0u);
      u.w &= nv_lane > 7 ? 0xffffffffu : (nv_lane > 6 ? 0x0000ffffu : 0u);
      vop = __builtin_bit_cast(bf16x8, u);
    }
#pragma unroll
    for (int t = 0; t < PSPLIT; ++t)
      st.o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t], st.o[blk], 0, 0, 0);
  }
}

template <bool KV_FP8, int QSPLIT, int PSPLIT, bool DIRECT, bool OUT_BF16>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a) {
  __shared__ float sm_o[4][16][kD + 4];
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  // wave index made explicitly wave-uniform so everything derived from it stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
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

  const uint8_t* kbase = (const uint8_t*)a.k_pool + (size_t)kvh * (kP * kD * (KV_FP8 ? 1 : 2));
  const uint8_t* vbase = (const uint8_t*)a.v_pool + (size_t)kvh * (kD * kP * (KV_FP8 ? 1 : 2));
  const int32_t* ptrow = a.page_table + (size_t)b * a.pt_stride;
  const unsigned last_page = (unsigned)(a.num_pages - 1);

  // Q^T operand: chunk cc holds dims k_dim0(cc, grp) .. +7 of head gq (zeros for gq >= G)
  bf16x8 qop[QSPLIT][4];
  {
    const size_t qrow = ((size_t)b * a.Hq + kvh * G + gq) * kD;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int d0 = k_dim0<KV_FP8>(cc, grp);
      float f[8];
      if (gq < G) {
        if (QSPLIT == 1) {
          const u32x4 w = *reinterpret_cast<const u32x4*>((const uint16_t*)a.q + qrow + d0);
          qop[0][cc] = __builtin_bit_cast(bf16x8, w);
          continue;
        }
        const float4* src = reinterpret_cast<const float4*>((const float*)a.q + qrow + d0);
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

  const float ks = KV_FP8 ? a.k_scale[kvh] : 1.0f;
  const float vs = KV_FP8 ? a.v_scale[kvh] : 1.0f;
  const float c = a.sm_scale * ks * kLog2e;

  WaveState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) st.o[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int seg0 = t0; seg0 < t1; seg0 += kSeg) {
    const int seg1 = min(t1, seg0 + kSeg);
    const int nw = (seg1 - seg0 + 31) >> 5;
    const int qw = (nw + 3) >> 2;
    const int w_begin = wave * qw;
    const int n = max(0, min(nw, w_begin + qw) - w_begin);  // windows of this wave in the segment
    if (n == 0) continue;                                  // wave-uniform
    const int ws = seg0 + 32 * w_begin;  // first token of this wave's range (multiple of 32)
    // page ids of this wave's range: lane i <- entry ws/16 + i (clamped into the pool)
    int ptv = 0;
    {
      const int e = (ws >> 4) + lane;
      if (lane < 2 * n && e < a.pt_stride) ptv = (int)min((unsigned)ptrow[e], last_page);
    }
    // Full windows go through register buffers in rotation (three for FP8, two for the
    // twice-as-large BF16 windows): while window w is processed the next one or two are in flight.
    // The rotation is unrolled so no buffer is ever copied (a copy would have to wait for its
    // loads), and every prefetch is issued unconditionally (past the end it re-reads the last full
    // window, a cache hit) so the load-counter waits stay exact.  Only the sequence's final window
    // can be partial; it is loaded and processed on its own after the loop.
    const bool tail = t1 - (ws + 32 * (n - 1)) < 32;
    const int nf = n - (tail ? 1 : 0);  // full windows
    const int last = max(nf - 1, 0);
    KvRegs b0, b1;
#define DAPF8_LOAD(BUF, W)                                                                             \
  load_window<KV_FP8>(BUF, kbase, vbase, __builtin_amdgcn_readlane(ptv, 2 * (W)),                       \
                      __builtin_amdgcn_readlane(ptv, 2 * (W) + 1), lane, a.Hkv)
#define DAPF8_PROC(BUF) process_window<KV_FP8, QSPLIT, PSPLIT, false>(st, BUF, qop, c, 32, grp)
    if (nf > 0) {
      DAPF8_LOAD(b0, 0);
      if constexpr (KV_FP8) {
        KvRegs b2;
        DAPF8_LOAD(b1, min(1, last));
        for (int w = 0; w < nf; w += 3) {
          DAPF8_LOAD(b2, min(w + 2, last));
          DAPF8_PROC(b0);
          if (w + 1 >= nf) break;
          DAPF8_LOAD(b0, min(w + 3, last));
          DAPF8_PROC(b1);
          if (w + 2 >= nf) break;
          DAPF8_LOAD(b1, min(w + 4, last));
          DAPF8_PROC(b2);
        }
      } else {
        for (int w = 0; w < nf; w += 2) {
          DAPF8_LOAD(b1, min(w + 1, last));
          DAPF8_PROC(b0);
          if (w + 1 >= nf) break;
          DAPF8_LOAD(b0, min(w + 2, last));
          DAPF8_PROC(b1);
        }
      }
    }
    if (tail) {
      DAPF8_LOAD(b0, n - 1);
      process_window<KV_FP8, QSPLIT, PSPLIT, true>(st, b0, qop, c, t1 - (ws + 32 * (n - 1)), grp);
    }
#undef DAPF8_LOAD
#undef DAPF8_PROC
  }
  const float m_run = st.m, l_run = st.l;

  // ---- merge the four waves through LDS
  const float l_tot = xor_sum(l_run);
  if (grp == 0) {
    sm_m[wave][gq] = m_run;
    sm_l[wave][gq] = l_tot;
  }
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[wave][gq][16 * blk + 4 * grp + i] = st.o[blk][i];
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

// ================================================================================================
// Stream-K variant.  All work -- every (sequence b, KV head, 32-token window) -- is flattened in
// (b, head, window) order and cut into `nworkers` equal contiguous slices, one per wave; the grid
// holds exactly as many waves as the GPU keeps resident, so every wave streams the same number of
// bytes from start to end, prefetching across sequence boundaries.  A slice yields one partial
// result ("piece") per (b, head, partition) it touches; merge_sk_kernel combines the pieces.
// Partitions (split_tokens) only add piece boundaries, so the result is the log-sum-exp merge of
// fixed token partitions whatever the slicing.  Aborted and empty sequences own no windows.
//
// Piece numbering: the global partition index sg (in (b, head, partition) order) plus the worker
// index k.  A worker's pieces have consecutive sg; the next worker starts at the partition where
// this one ended or later, so sg + k never collides, and the pieces of partition sg are
// sg + k0 .. sg + k1 for the workers k0..k1 that cover it.  Workspace layout (floats):
//   pieces  [npieces][G][Dv + 4]  (unnormalised O scaled by s_V, then (m, l) in the log2 domain;
//                                  the row is padded to keep 16-byte alignment)
//   prefix  [2][B + 1] int        (window / partition prefix sums, written by workgroup 0)
// Page-tag check of one window's two pages, carried from its load to its compute: the live tags
// are gathered with one uniform load issued just before the window's K/V loads, so the wait for
// the window's data covers it and the check costs no extra memory round trip.
struct TagChk {
  uint32_t tA, tB;  // live tags of the two pages (uniform)
  uint32_t eA, eB;  // expected tags
  int bad_id;       // a page id outside the pool
  int vA, vB;       // page slot inside the sequence
};

template <bool KV_FP8, int QSPLIT, int PSPLIT, bool OUT_BF16, bool CHECK>
__global__ __launch_bounds__(256) void attn_sk_kernel(AttnArgs a, int nworkers) {
  __shared__ SkPrefix px;
  const int wpp = a.split >> 5;  // windows per partition
  sk_prefix<256>(px, a, 5, wpp);
  const int B = a.B, Hkv = a.Hkv, G = a.G;
  if (blockIdx.x == 0) sk_publish_prefix(px, a, 256);  // for the merge kernel
  // no workgroup barrier below this point: the four waves are independent workers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + wave;
  const long T = (long)Hkv * px.unit[B];
  const long nw_eff = min((long)nworkers, T);  // never more workers than windows: no empty slice
  if (k >= nw_eff) return;
  const long lo = (long)k * T / nw_eff, hi = (long)(k + 1) * T / nw_eff;
  const int n = (int)(hi - lo);
  const int row = lane & 15, grp = lane >> 4;
  const int gq = row;
  const unsigned last_page = (unsigned)(a.num_pages - 1);
  const long piece_stride = (long)G * (kD + 4);

  // Per-chunk window tables (32 windows; lane i describes page slot i & 1 of window i >> 1):
  //   load side:    vpage = the raw page-table entry (-1 past the sequence end), odd lanes' vhead =
  //                 the KV head;
  //   compute side: even lanes' vseg = b * Hkv + head and vw = the window index in (b, head).
  // Each side keeps its own current/next pair and rotates it when its window index crosses a
  // chunk boundary, so it only ever reads a table loaded 32 windows earlier: the page-table loads
  // are never waited for (no arithmetic on them here either) while window loads are in flight.
  auto locate = [&](int chunk, int& b, int& h, int& w) __attribute__((always_inline)) {
    const long gi = lo + 32L * chunk + (lane >> 1);
    b = -1;
    h = w = 0;
    if (gi < hi) {
      b = sk_find_seq(px, B, Hkv, gi);
      const int W = px.unit[b + 1] - px.unit[b];
      const int local = (int)(gi - (long)Hkv * px.unit[b]);
      h = local / W;
      w = local - h * W;
    }
  };
  // With CHECK, bit 16 of vhead marks a page slot inside the sequence and vexp is its expected tag.
  auto resolve_load = [&](int chunk, int& vpage, int& vhead, uint32_t& vexp) __attribute__((always_inline)) {
    int b, h, w;
    locate(chunk, b, h, w);
    vpage = -1;
    vhead = h;
    vexp = 0u;
    if (b >= 0) {
      const int e = 2 * w + (lane & 1);
      const int np = (px.len[b] + kP - 1) / kP;
      if (e < np) {
        vpage = a.page_table[(size_t)b * a.pt_stride + e];
        if (CHECK) {
          vexp = a.expected_tags[(size_t)b * a.pt_stride + e];
          vhead |= 0x10000;
        }
      }
    }
  };
  auto resolve_compute = [&](int chunk, int& vseg, int& vw) __attribute__((always_inline)) {
    int b, h, w;
    locate(chunk, b, h, w);
    vseg = b >= 0 ? b * Hkv + h : 0;
    vw = w;
  };
  int lp0, lh0, lp1, lh1;  // load tables: current, next
  uint32_t le0, le1;       // expected tags (CHECK)
  int cs0, cw0, cs1, cw1;  // compute tables: current, next
  resolve_load(0, lp0, lh0, le0);
  resolve_load(1, lp1, lh1, le1);
  resolve_compute(0, cs0, cw0);
  resolve_compute(1, cs1, cw1);

  WaveState st;
  bf16x8 qop[QSPLIT][4];
  // the open piece: (b*Hkv + head), its partition, and values fixed for the whole piece
  int cur_seg = -1, cur_part = -1, part_end = 0, last_w = 0, last_nvalid = 0;
  int seg_bad = 0;  // CHECK: a page of the open (b, head) failed the tag check
  float c = 0.0f, v_scale_cur = 1.0f;

  const uint8_t* kpool = (const uint8_t*)a.k_pool;
  const uint8_t* vpool = (const uint8_t*)a.v_pool;
  int load_base = 0, comp_base = 0;  // first window of each side's current table

  auto do_load = [&](KvRegs& r, TagChk& tc, int i) __attribute__((always_inline)) {
    // The pipeline issues one load past the slice end (so every wait count stays exact); it reads
    // block 0 of the pool, which the caches already hold after the first such load, instead of
    // fetching the last window again from HBM (non-temporal loads do not keep it cached).
    const bool past = i >= n;
    i = min(i, n - 1);
    if (i - load_base == 32) {  // windows are loaded in order: rotate the load tables
      load_base += 32;
      lp0 = lp1;
      lh0 = lh1;
      le0 = le1;
      resolve_load(load_base / 32 + 1, lp1, lh1, le1);
    }
    const int sl = 2 * (i - load_base);
    unsigned pA = (unsigned)__builtin_amdgcn_readlane(lp0, sl);
    unsigned pB = (unsigned)__builtin_amdgcn_readlane(lp0, sl + 1);
    const int hB = __builtin_amdgcn_readlane(lh0, sl + 1);
    int h = CHECK ? (hB & 0xffff) : hB;
    if (CHECK) {
      tc.vA = __builtin_amdgcn_readlane(lh0, sl) >> 16;
      tc.vB = hB >> 16;
      tc.eA = (uint32_t)__builtin_amdgcn_readlane((int)le0, sl);
      tc.eB = (uint32_t)__builtin_amdgcn_readlane((int)le0, sl + 1);
      tc.bad_id = (tc.vA && pA > last_page) || (tc.vB && pB > last_page);  // negative ids wrap past it
      tc.tA = a.live_tags[min(pA, last_page)];
      tc.tB = a.live_tags[min(pB, last_page)];
    }
    if (past) {  // never computed: its tag check result is not used either
      pA = pB = 0u;
      h = 0;
    }
    // out-of-range ids (and -1 past the sequence end) read the last page: stays inside the pool
    const int bA = (int)min(pA, last_page) * Hkv + h;  // < num_pages * Hkv <= INT32_MAX
    const int bB = (int)min(pB, last_page) * Hkv + h;
    load_window<KV_FP8>(r, kpool, vpool, bA, bB, lane, 1);
  };

  auto flush = [&]() __attribute__((always_inline)) {
    if (cur_seg < 0) return;
    const int b = cur_seg / Hkv, h = cur_seg - b * Hkv;
    const float vs = v_scale_cur;  // read when (b, head) was opened: no load (and no wait) here
    const float l_tot = xor_sum(st.l);
    const int W = px.unit[b + 1] - px.unit[b];
    const int npart = px.part[b + 1] - px.part[b];
    const long seg_first = (long)Hkv * px.unit[b] + (long)h * W;
    const bool whole = npart == 1 && seg_first >= lo && seg_first + W <= hi;
    if (whole) {  // this worker saw every window of (b, head): write the final rows
      if (CHECK && lane == 0) a.abort_out[b] = (uint8_t)seg_bad;  // it also checked every page of b
      if (gq < G) {
        const float r = vs / l_tot;
        const size_t ob = ((size_t)b * a.Hq + h * G + gq) * kD;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float o = (CHECK && seg_bad) ? 0.0f : st.o[blk][i] * r;  // aborted: exact zeros
            const size_t oi = ob + 16 * blk + 4 * grp + i;
            if (OUT_BF16)
              ((uint16_t*)a.out)[oi] = f32_to_bf16_rne(o);
            else
              ((float*)a.out)[oi] = o;
          }
      }
    } else if (gq < G) {
      const long sg = (long)Hkv * px.part[b] + (long)h * npart + cur_part;
      float* pc = a.ws_o + (sg + k) * piece_stride + (long)gq * (kD + 4);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        f32x4 v = st.o[blk] * vs;
        *reinterpret_cast<f32x4*>(pc + 16 * blk + 4 * grp) = v;
      }
      if (grp == 0) {
        pc[kD] = st.m;
        pc[kD + 1] = (CHECK && seg_bad) ? -1.0f : l_tot;  // a negative sum marks a failed tag check
      }
    }
  };

  // next partition of the same (b, head): only the piece changes (the query stays loaded)
  auto next_part = [&](int w) __attribute__((always_inline)) {
    flush();
    cur_part = w / wpp;
    part_end = (cur_part + 1) * wpp;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) st.o[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };

  auto open = [&](int seg, int w) __attribute__((always_inline)) {
    flush();
    const int b = seg / Hkv, h = seg - b * Hkv;
    cur_seg = seg;
    seg_bad = 0;
    cur_part = w / wpp;
    part_end = (cur_part + 1) * wpp;
    const int len = px.len[b];
    last_w = (len - 1) >> 5;
    last_nvalid = len - 32 * last_w;
    c = a.sm_scale * (KV_FP8 ? a.k_scale[h] : 1.0f) * kLog2e;
    v_scale_cur = KV_FP8 ? a.v_scale[h] : 1.0f;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) st.o[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // query operand of the new (b, head); lanes past G read head G-1 (finite, discarded)
    const size_t qrow = ((size_t)b * a.Hq + h * G + min(gq, G - 1)) * kD;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int d0 = k_dim0<KV_FP8>(cc, grp);
      if (QSPLIT == 1) {
        qop[0][cc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>((const uint16_t*)a.q + qrow + d0));
      } else {
        const float4* src = reinterpret_cast<const float4*>((const float*)a.q + qrow + d0);
        const float4 x0 = src[0], x1 = src[1];
        const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        bf16x8 parts[QSPLIT];
        split_bf16<QSPLIT>(f, parts);
#pragma unroll
        for (int t = 0; t < QSPLIT; ++t) qop[t][cc] = parts[t];
      }
    }
  };

  auto proc = [&](const KvRegs& r, const TagChk& tc, int i) __attribute__((always_inline)) {
    if (i - comp_base == 32) {  // entering the next 32-window chunk: rotate the compute tables
      comp_base += 32;
      cs0 = cs1;
      cw0 = cw1;
      resolve_compute(comp_base / 32 + 1, cs1, cw1);
    }
    const int sl = 2 * (i - comp_base);
    const int seg = __builtin_amdgcn_readlane(cs0, sl);
    const int w = __builtin_amdgcn_readlane(cw0, sl);
    if (seg != cur_seg)
      open(seg, w);
    else if (w >= part_end)
      next_part(w);
    if (CHECK) {
      const bool bad = tc.bad_id || (tc.vA && tc.tA != tc.eA) || (tc.vB && tc.tB != tc.eB);
      seg_bad |= __builtin_amdgcn_readfirstlane((int)bad);
    }
    // only a sequence's last window can be partial: full windows skip the masking (uniform branch)
    if (w == last_w && last_nvalid < 32)
      process_window<KV_FP8, QSPLIT, PSPLIT, true>(st, r, qop, c, last_nvalid, grp);
    else
      process_window<KV_FP8, QSPLIT, PSPLIT, false>(st, r, qop, c, 32, grp);
  };

  // Two register buffers in ping-pong; with non-temporal loads, one window in flight during each
  // window's compute keeps HBM saturated at two resident waves per SIMD.
  KvRegs b0, b1;
  TagChk t0{}, t1{};
  do_load(b0, t0, 0);
  for (int i = 0; i < n; i += 2) {
    do_load(b1, t1, i + 1);
    proc(b0, t0, i);
    if (i + 1 >= n) break;
    do_load(b0, t0, i + 2);
    proc(b1, t1, i + 1);
  }
  flush();
  // A slice that ends exactly on a partition boundary inside a (sequence, head) leaves the slot of
  // (next partition, this worker) unused: write an empty piece there (m = -inf, l = 0, zeros) so
  // that the merge can read the sequence-head's slots as one contiguous range.
  if (cur_seg >= 0 && gq < G) {
    const int b = cur_seg / Hkv, h = cur_seg - b * Hkv;
    const int W = px.unit[b + 1] - px.unit[b];
    const int npart = px.part[b + 1] - px.part[b];
    const long rel = hi - ((long)Hkv * px.unit[b] + (long)h * W);  // windows of (b, h) up to the slice end
    if (npart > 1 && rel < W && rel % wpp == 0) {
      const long slot = (long)Hkv * px.part[b] + (long)h * npart + rel / wpp + k;
      float* pc = a.ws_o + slot * piece_stride + (long)gq * (kD + 4);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk)
        *reinterpret_cast<f32x4*>(pc + 16 * blk + 4 * grp) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (grp == 0) {
        pc[kD] = -INFINITY;
        pc[kD + 1] = 0.0f;
      }
    }
  }
}

// merge for the stream-K kernel: one workgroup per (KV head, sequence).  Piece (partition p,
// worker k) of sequence-head (b, head) sits in slot C + p + k, where C numbers the sequence-head's
// first partition; over the workers K0..K1 that hold its windows these slots form the contiguous
// range C + K0 .. C + K1 + npart - 1.  A slot no (p, k) pair maps to -- a worker slice ending exactly
// on a partition boundary -- holds an empty piece written by the main kernel, so the merge reads
// the range without any per-piece index arithmetic.  The pieces cover disjoint token ranges and
// the log-sum-exp combination of all of them is the result, whatever the partitioning.
// Threads: the G x 128 outputs form G * 32 float4 slots; r adjacent threads (a power of two) share
// a slot and take every r-th piece.  Each thread loads a batch of pieces' (m, l) and values at once
// (one memory round trip), combines them, and the r partial results meet through lane shuffles.
constexpr int kMergeBatch = 8;
constexpr int kMergeSlots = 2048;  // float4 output slots per merge workgroup

__device__ __forceinline__ void lse_combine(float& M, float& den, f32x4& num, float Mo, float deno, f32x4 numo) {
  const float Mn = fmaxf(M, Mo);
  if (Mn > -INFINITY) {
    const float sa = exp2f(M - Mn), sb = exp2f(Mo - Mn);  // exp2(-inf) = 0
    den = den * sa + deno * sb;
    num = num * sa + numo * sb;
    M = Mn;
  }
}

__global__ __launch_bounds__(256) void merge_sk_kernel(AttnArgs a, int nworkers, int slots_per_block) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int B = a.B, Hkv = a.Hkv, G = a.G, Dv = a.Dv, D4 = a.Dv >> 2;
  const int* wsp = reinterpret_cast<const int*>(a.ws_ml);
  const int win0 = wsp[b], win1 = wsp[b + 1], part0 = wsp[B + 1 + b], part1 = wsp[B + 1 + b + 1];
  const int W = win1 - win0, npart = part1 - part0;
  const int S = G * D4;  // float4 output slots of this (sequence, KV head)
  // this block's share of the slots (grid.z splits them); r threads share a slot
  const int s_begin = blockIdx.z * slots_per_block, s_end = min(S, s_begin + slots_per_block);
  int r = 1;
  while (r < 8 && 2 * r * (s_end - s_begin) <= 256) r *= 2;
  const int t = threadIdx.x, sub = t & (r - 1);
  const size_t ob0 = ((size_t)b * a.Hq + (size_t)h * G) * Dv;
  const bool obf = a.out_dt == DAPF8_ACT_BF16;
  auto write_zeros = [&]() {
    for (int slot = s_begin + t / r; slot < s_end && sub == 0; slot += 256 / r) {
      const int g = slot / D4, d4 = (slot - g * D4) * 4;
      if (obf)
        *reinterpret_cast<uint2*>((uint16_t*)a.out + ob0 + (size_t)g * Dv + d4) = make_uint2(0u, 0u);
      else
        *reinterpret_cast<f32x4*>((float*)a.out + ob0 + (size_t)g * Dv + d4) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  if (W == 0) {  // aborted or empty sequence: zeros
    write_zeros();
    if (a.abort_out && blockIdx.z == 0 && t == 0) {  // in-walk tag check: only a bad length aborts here
      const int raw = a.seq_lens[b];
      a.abort_out[b] = (raw < 0 || (int64_t)raw > (int64_t)a.pt_stride * a.page_size) ? 1 : 0;
    }
    return;
  }
  const long T = (long)Hkv * wsp[B];  // > 0 here
  const long nw_eff = min((long)nworkers, T);
  const long seg_first = (long)Hkv * win0 + (long)h * W;
  const long K0 = ((seg_first + 1) * nw_eff - 1) / T;      // worker holding unit seg_first
  const long K1 = ((seg_first + W) * nw_eff - 1) / T;      // worker holding unit seg_first + W - 1
  if (npart == 1 && K0 == K1) return;  // that worker wrote the final rows itself
  const int nj = (int)(K1 - K0) + npart;
  const long piece_stride = (long)G * (Dv + 4);
  const float* first = a.ws_o + ((long)Hkv * part0 + (long)h * npart + K0) * piece_stride;
  if (a.abort_out) {  // in-walk tag check: any piece with a failed page (negative sum) aborts b
    int bad = 0;
    for (int j = t; j < nj; j += 256) bad |= first[(long)j * piece_stride + Dv + 1] < 0.0f;
    bad = __syncthreads_or(bad);
    if (blockIdx.z == 0 && t == 0) a.abort_out[b] = (uint8_t)bad;
    if (bad) {
      write_zeros();
      return;
    }
  }
  for (int base = s_begin; base < s_end; base += 256 / r) {  // wave-uniform trip count
    const int slot = base + t / r;
    const int sl = min(slot, s_end - 1);  // lanes past the last slot read a valid slot, write nothing
    const int g = sl / D4, d4 = (sl - g * D4) * 4;
    const float* row = first + (long)g * (Dv + 4);
    float M = -INFINITY, den = 0.0f;
    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = sub; j0 < nj; j0 += r * kMergeBatch) {
      float2 ml[kMergeBatch];
      f32x4 v[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {  // clamped indices: every load is in range, no branches
        const int j = min(j0 + u * r, nj - 1);
        const float* pc = row + (long)j * piece_stride;
        ml[u] = *reinterpret_cast<const float2*>(pc + Dv);
        v[u] = *reinterpret_cast<const f32x4*>(pc + d4);
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (j0 + u * r >= nj) ml[u].x = -INFINITY;  // past the end: no contribution
        lse_combine(M, den, num, ml[u].x, ml[u].y, ml[u].x > -INFINITY ? v[u] : f32x4{0.0f, 0.0f, 0.0f, 0.0f});
      }
    }
    for (int off = 1; off < r; off <<= 1) {
      const float Mo = __shfl_xor(M, off), deno = __shfl_xor(den, off);
      const f32x4 numo = {__shfl_xor(num[0], off), __shfl_xor(num[1], off), __shfl_xor(num[2], off),
                          __shfl_xor(num[3], off)};
      lse_combine(M, den, num, Mo, deno, numo);
    }
    if (sub == 0 && slot < s_end) {
      const f32x4 o = num / den;
      const size_t oi = ob0 + (size_t)g * Dv + d4;
      if (obf) {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[2]) | ((uint32_t)f32_to_bf16_rne(o[3]) << 16);
        *reinterpret_cast<uint2*>((uint16_t*)a.out + oi) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<f32x4*>((float*)a.out + oi) = o;
      }
    }
  }
}

int launch_merge_sk(const AttnArgs& a, int nworkers, hipStream_t s) {
  // Slots per block: up to kMergeSlots.  When a sequence-head's piece list is long (many workers
  // per sequence-head, as for a few very long sequences) narrow heads are spread over several
  // blocks (down to 32 slots, i.e. 8 threads per slot) so each list is combined by many threads.
  // Wide pieces (many query heads, as in the latent shape) are spread so each thread handles about
  // two slots: a thread combines its slots one after another, each a memory round trip.
  const int slots = a.G * (a.Dv / 4);
  const long pieces_per_seq = (long)nworkers / ((long)a.B * a.Hkv) + a.nsplit;
  int per_block = slots > kMergeSlots ? 512 : kMergeSlots;
  if (pieces_per_seq > 16)
    while (per_block > 32 && per_block * 16 > slots) per_block >>= 1;
  const dim3 grid((unsigned)a.Hkv, (unsigned)a.B, (unsigned)((slots + per_block - 1) / per_block));
  hipLaunchKernelGGL(merge_sk_kernel, grid, dim3(256), 0, s, a, nworkers, per_block);
  return check_launch("paged_decode_attn (stream-K merge)");
}

// Waves the GPU keeps resident for one stream-K instantiation on the current device; the grid is
// sized to exactly that many workers so all of them run in a single round.
// The count is cached per device and instantiation (a property of the device and the compiled
// kernel), so launches inside a graph capture make no runtime queries.
template <auto Kernel>
static int resident_waves() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0, cus = 0, wgs = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs, Kernel, 256, 0) != hipSuccess) return 0;
  const int n = cus * (wgs > 0 ? wgs : 1) * 4;
  if (dev >= 0 && dev < kMaxDev) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int launch_attn_sk(const AttnArgs& a, int max_workers, hipStream_t s) {
  const bool fp8 = a.kv_dt == DAPF8_KV_FP8_E4M3;
  const bool obf = a.out_dt == DAPF8_ACT_BF16;
  const bool qf32 = a.q_dt == DAPF8_ACT_F32;
  const bool check = a.abort_out != nullptr;
  if (check && qf32) return set_error(DAPF8_EUNSUPPORTED, "paged_decode_attn_checked: bf16 queries only");
  int nworkers = 0;
#define DAPF8_SK(F, QS, PS, OB, CK)                                                                  \
  do {                                                                                               \
    auto kern = attn_sk_kernel<F, QS, PS, OB, CK>;                                                   \
    nworkers = min(resident_waves<attn_sk_kernel<F, QS, PS, OB, CK>>(), max_workers);                \
    if (nworkers < 4) return set_error(DAPF8_ELAUNCH, "paged_decode_attn: no resident waves");       \
    nworkers &= ~3;                                                                                  \
    hipLaunchKernelGGL(kern, dim3((unsigned)(nworkers / 4)), dim3(256), 0, s, a, nworkers);          \
  } while (0)
#define DAPF8_SK_Q(F, PS, OB)   \
  if (check)                    \
    DAPF8_SK(F, 1, PS, OB, true); \
  else if (qf32)                \
    DAPF8_SK(F, 3, PS, OB, false); \
  else                          \
    DAPF8_SK(F, 1, PS, OB, false);
  if (fp8 && obf) {
    DAPF8_SK_Q(true, 1, true)
  } else if (fp8) {
    DAPF8_SK_Q(true, 3, false)
  } else if (obf) {
    DAPF8_SK_Q(false, 1, true)
  } else {
    DAPF8_SK_Q(false, 3, false)
  }
#undef DAPF8_SK_Q
#undef DAPF8_SK
  int rc = check_launch("paged_decode_attn (stream-K)");
  if (rc != DAPF8_OK) return rc;
  return launch_merge_sk(a, nworkers, s);
}

int launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B), block(256);
  const bool fp8 = a.kv_dt == DAPF8_KV_FP8_E4M3;
  const bool qf32 = a.q_dt == DAPF8_ACT_F32;
  const bool direct = a.nsplit == 1;
  const bool obf = a.out_dt == DAPF8_ACT_BF16;
  // P keeps 8 bits (one bf16 term) for bf16 outputs -- its rounding error, at most 2^-9 of |V|, is
  // far inside the bf16 output's own tolerance -- and ~24 bits (three terms) for fp32 outputs;
  // fp32 queries are split into three bf16 terms (~24 bits).
#define DAPF8_MFMA(F, QS, PS, DI, OB) hipLaunchKernelGGL((attn_mfma_kernel<F, QS, PS, DI, OB>), grid, block, 0, s, a)
#define DAPF8_MFMA_OUT(F, QS)                    \
  if (direct && obf)                             \
    DAPF8_MFMA(F, QS, 1, true, true);            \
  else if (direct)                               \
    DAPF8_MFMA(F, QS, 3, true, false);           \
  else if (obf)                                  \
    DAPF8_MFMA(F, QS, 1, false, false);          \
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
