// attn_latent.hip -- decode attention on the matrix cores for the shared-KV ("latent") layout:
// V is the first Dv = 512 dims of each Dk = 576-dim K row, page size 64, FP8 (e4m3) storage,
// G = Hq / Hkv query heads per KV head with G a multiple of 16 up to 128.
//
// [CF §Quantize] the cache holds FP8 codes; the kernel reads them without widening where it can and
// converts them to bf16 on read (exact) where it must, and folds the single per-head scale into the
// score and the output.
//
// Why a kernel of its own: with 128 query heads sharing one 576-dim KV row the work is a real
// dense contraction (about 480 flop per cached byte), so the matrix cores -- not HBM -- set the
// pace, and every cached byte must be reused by all query heads.  One workgroup of G / 16 waves
// owns all G heads: each 64-token page is copied once into LDS (direct global->LDS loads, no
// registers), and every wave computes its 16 heads against it:
//   S^T = K Q^T   A = K tile (16 tokens x k dims) read from LDS, B = Q^T (k dims x 16 heads) held in
//                 registers for the whole piece.  For bf16 outputs dims 0..511 run on the FP8 matrix
//                 cores (v_mfma_scale_f32_16x16x128_f8f6f4): the stored codes are the A operand as
//                 they are, and the bf16 query is carried as two e4m3 terms with a power-of-two
//                 scale per 32-dim block (q = t1 2^e1 + t2 2^e2 + r, |r| <= 2^-8 of the block's
//                 largest |q|), so no instruction widens K; dims 512..575 and every dim of the fp32-
//                 output variant take the bf16 product with K widened to bf16 (exact).  Widening
//                 each page's K for every wave was 60 % of the kernel's vector instructions.
//   O^T = V^T P^T A = V^T tile (16 dims x 32 tokens) read from the same LDS page with the
//                 byte-transposing LDS read, B = P^T taken straight from the S^T registers (the token
//                 order inside a 32-token window is permuted so each lane holds the 8 probabilities
//                 its operand needs, as in the 128-dim kernel).
// The page's LDS rows are padded to 592 bytes so both read patterns spread over all LDS banks.
//
// Work decomposition: stream-K over (sequence, KV head, 64-token page) units, one persistent
// workgroup per CU, equal contiguous slices; a slice yields one piece per (sequence, head,
// partition) it touches, combined by merge_sk_kernel (the same piece-slot scheme as the 128-dim
// stream-K kernel).  Pages stream through a ring of three LDS buffers: page i + 2 is loaded while
// page i is computed, with one workgroup barrier per page.
#include <atomic>

#include "mfma_util.hpp"

namespace dapf8 {

namespace {

constexpr int kLD = 576;                    // K row dims
constexpr int kLV = 512;                    // V dims (first kLV of the row)
constexpr int kLP = 64;                     // tokens per page
constexpr int kLRow = kLD + 16;             // LDS bytes per token row (padded)
constexpr int kLRowUnits = kLRow / 16;      // 37 16-byte units per LDS row
constexpr int kLUnits = kLP * kLRowUnits;   // 2368 units per page = 37 wave-wide loads
constexpr int kLWaveLoads = kLUnits / 64;   // 37
constexpr int kLChunk = 64;                 // K pool dimension chunk (bytes) for FP8
constexpr int kLBlock = kLP * kLD;          // bytes of one (page, head) block in the pool
static_assert(kLUnits % 64 == 0, "a page must be a whole number of wave-wide loads");
constexpr int kLRing = 3;                   // LDS page buffers in the ring
constexpr int kLQF8 = 4;                    // 128-dim chunks of the QK product on FP8 matrix cores (dims 0..511)
typedef int i32x8 __attribute__((ext_vector_type(8)));

// LDS pointers keep their address space, so the compiler can tell the two page buffers apart
// (a generic pointer would make every LDS read wait for every outstanding global->LDS load)
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 16 bytes per lane from global memory straight into LDS at base + 16 * lane.  Issued as inline
// assembly so the compiler does not treat the LDS writes as outstanding when the other page buffer is
// read (its LDS alias check cannot separate the two buffers and would drain every load); the kernel
// waits for these loads itself (vmcnt) and orders them with barriers.  The LDS address goes in m0
// through an operand constraint, so the compiler sets m0 itself and knows it is in use.
__device__ __forceinline__ void lds_dma16(const void* src, const lds_u8* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// workgroup barrier that also stops the compiler from moving memory accesses across it
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ u32x4 lds_read16(const lds_u8* p) {
  return *reinterpret_cast<const lds_u32x4*>(p);
}

__device__ __forceinline__ u32x2 lds_read8_tr(const lds_u8* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 A and B), probed on the GPU: lane
// l holds row (A) or column (B) l % 16; with g = l / 16, its bytes 0..15 are k = 16 g .. 16 g + 15 and
// bytes 16..31 are k = 64 + 16 g .. +15; the E8M0 scale of row (column) r's k-block q (k = 32 q ..
// 32 q + 31) is the scale operand of lane r + 16 q.  So the two 16-byte halves a lane holds lie in
// k-blocks g / 2 and 2 + g / 2, each block is shared by lanes g and g ^ 1, and a lane's own scale
// operand serves block g.
//
// Split one lane's 32 query values -- x[0..15] at k = 16 g + i, x[16..31] at k = 64 + 16 g + i of one
// head and one 128-dim chunk -- into NT e4m3 terms that share one E8M0 scale per 32-dim block:
// q = 2^(s - 127) sum_j dec(t_j) + r.  The scale puts the block's largest magnitude in [128, 256),
// inside e4m3's finite range; every term is rounded to nearest even, so each leaves at most 2^-4 of
// what it was given (every later term's values stay above e4m3's subnormal range for all but
// magnitudes below 2^-14 of the block's largest), and two terms leave |r| <= 2^-8 max|q| over the
// block.  Each residual is exact in fp32 (a value of at most 24 significant bits minus a 4-bit one of
// similar magnitude).  sc is this lane's scale operand, which serves block g.
template <int NT>
__device__ __forceinline__ void split_q_fp8(float (&x)[32], int g, i32x8 (&t)[NT], int& sc) {
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a0 = fmaxf(a0, fabsf(x[i]));
    a1 = fmaxf(a1, fabsf(x[16 + i]));
  }
  a0 = fmaxf(a0, __shfl_xor(a0, 16));  // lanes g and g ^ 1 hold the two halves of each block
  a1 = fmaxf(a1, __shfl_xor(a1, 16));
  // amax = m 2^E with m in [0.5, 1): amax / 2^(E - 8) lies in [128, 256)
  const int e0 = a0 > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(a0) - 8, -126), 126) : 0;
  const int e1 = a1 > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(a1) - 8, -126), 126) : 0;
  // this lane's scale operand serves block g: block 0 = own first half (g = 0), block 1 = first
  // half of group 2, block 2 = second half of group 1, block 3 = own second half (g = 3)
  const int up = __shfl_down(e0, 16), dn = __shfl_up(e1, 16);
  sc = (g == 0 ? e0 : g == 1 ? up : g == 2 ? dn : e1) + 127;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = __builtin_ldexpf(x[i], i < 16 ? -e0 : -e1);  // exact
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w], x[4 * w + 1], 0, false);
      const int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], lo, true);
      t[j][w] = word;
      if (j + 1 < NT) {  // residual for the next term
        const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false), d1 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
        x[4 * w] -= d0.x;
        x[4 * w + 1] -= d0.y;
        x[4 * w + 2] -= d1.x;
        x[4 * w + 3] -= d1.y;
      }
    }
  }
}

// The same for the last 64 dims (512..575): this lane's 16 values x[0..15] at k = 16 g + i are split
// into two e4m3 terms sharing one scale per 32-dim block, packed into ONE operand -- term 1 in bytes
// 0..15, term 2 in bytes 16..31 -- to be multiplied by a K operand that repeats its 16 bytes in both
// halves, so one product adds both terms.  Bytes 16..31 sit in k-blocks 2 + g / 2, which take the
// same scale as blocks g / 2; the lane's scale operand serves block g.
__device__ __forceinline__ void split_q_fp8_tail(float (&x)[16], int g, i32x8& t, int& sc) {
  float a0 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a0 = fmaxf(a0, fabsf(x[i]));
  a0 = fmaxf(a0, __shfl_xor(a0, 16));
  const int e0 = a0 > 0.0f ? min(max(__builtin_amdgcn_frexp_expf(a0) - 8, -126), 126) : 0;
  // block g of this lane: blocks 0 and 2 are dims 512..543 (groups 0, 1), blocks 1 and 3 dims
  // 544..575 (groups 2, 3)
  const int up = __shfl_down(e0, 16), dn = __shfl_up(e0, 32);  // every lane takes part in both
  sc = (g == 1 ? up : g == 2 ? dn : e0) + 127;
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = __builtin_ldexpf(x[i], -e0);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w], x[4 * w + 1], 0, false);
    const int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], lo, true);
    t[w] = word;
    const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false), d1 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
    const int lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w] - d0.x, x[4 * w + 1] - d0.y, 0, false);
    t[4 + w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2] - d1.x, x[4 * w + 3] - d1.y, lo2, true);
  }
}

}  // namespace

// One wave per SIMD, NHG groups of 16 query heads per wave (HPW = 16 NHG heads), NW = G / HPW
// waves per workgroup, one workgroup per CU.  Each K or V operand a wave reads from LDS (and each V
// operand it widens) feeds the products of all its head groups, and a wave may hold up to 512
// registers (the output accumulators live in the accumulation registers).
// QF8: dims 0..511 of the QK product on the FP8 matrix cores (bf16 outputs); otherwise every dim in
// bf16 (fp32 outputs, whose tighter bar the two-term query split would not meet everywhere).
template <int NW, int NHG, int PSPLIT, bool QF8>
__global__ __launch_bounds__(NW * 64) void attn_latent_kernel(AttnArgs a, int nwg) {
  constexpr int kLPW = (kLWaveLoads + NW - 1) / NW;  // wave-wide loads per wave per page
  constexpr int kBufBytes = NW * kLPW * 1024;        // >= kLUnits * 16; the rest is padding
  constexpr int kQT = 2;                             // e4m3 terms of the query (QF8)
  constexpr int HPW = 16 * NHG;                      // query heads per wave
  __shared__ __attribute__((aligned(16))) uint8_t ring_[kLRing * kBufBytes];
  lds_u8* const ring = (lds_u8*)ring_;
  __shared__ SkPrefix px;

  const int upp = a.split / kLP;  // pages per partition
  sk_prefix<NW * 64>(px, a, 6, upp);
  const int B = a.B, Hkv = a.Hkv, G = a.G;
  if (blockIdx.x == 0) sk_publish_prefix(px, a, NW * 64);  // for the merge kernel
  const long T = (long)Hkv * px.unit[B];
  const long nw_eff = min((long)nwg, T);
  const int k = blockIdx.x;
  if (k >= nw_eff) return;  // workgroup-uniform
  const long lo = (long)k * T / nw_eff, hi = (long)(k + 1) * T / nw_eff;
  const int n = (int)(hi - lo);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int row = lane & 15, grp = lane >> 4;
  const int gq0 = HPW * wave + row;  // query head (inside the KV head's group) of this lane's column, group 0
  const unsigned last_page = (unsigned)(a.num_pages - 1);
  const long piece_stride = (long)G * (kLV + 4);
  const uint8_t* kpool = (const uint8_t*)a.k_pool;

  // Source offset inside a (page, head) block of this lane's t-th load: LDS unit u holds 16 bytes
  // of token u / 37 at row position u % 37; position 36 is row padding and units past the page are
  // buffer padding (both load a harmless in-block address).  Recomputed per load (a few integer
  // instructions) rather than kept in registers.
  auto src_off = [&](int t) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // opaque: keeps the offsets from being hoisted into registers
    const int u = (wave * kLPW + t) * 64 + ln;
    const int tr = u / kLRowUnits;
    const int tok = min(tr, kLP - 1);
    const int q = min(u - tr * kLRowUnits, kLRowUnits - 2);
    return (q >> 2) * (kLP * kLChunk) + tok * kLChunk + (q & 3) * 16;
  };

  // unit cursor: (sequence b, KV head h, page j inside the sequence, the sequence's page count W),
  // kept wave-uniform so the page-table reads are scalar loads that do not queue behind the
  // outstanding global->LDS page loads
  struct Cursor {
    int b, h, j, W;
  };
  auto uni = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };
  auto cursor_at = [&](long g) __attribute__((always_inline)) {
    Cursor c;
    c.b = uni(sk_find_seq(px, B, Hkv, g));
    const int u0 = uni(px.unit[c.b]);
    c.W = uni(px.unit[c.b + 1]) - u0;
    const int local = (int)(g - (long)Hkv * u0);
    c.h = local / c.W;
    c.j = local - c.h * c.W;
    return c;
  };
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.j < c.W) return;
    c.j = 0;
    if (++c.h < Hkv) return;
    c.h = 0;
    do {
      ++c.b;
      c.W = c.b < B ? uni(px.unit[c.b + 1]) - uni(px.unit[c.b]) : 1;
    } while (c.W == 0);
  };
  // Page ids of this slice, 64 units at a time in a lane-distributed table (lane i: unit
  // tbase + i), loaded with vector loads well before they are needed and read with readlane.
  auto resolve = [&](int chunk) __attribute__((always_inline)) {
    const long g = lo + 64L * chunk + lane;
    int page = 0;
    if (g < hi) {
      const int b = sk_find_seq(px, B, Hkv, g);
      const int W = px.unit[b + 1] - px.unit[b];
      const int local = (int)(g - (long)Hkv * px.unit[b]);
      const int h = local / W, j = local - h * W;
      page = (int)min((unsigned)a.page_table[(size_t)b * a.pt_stride + j], last_page) * Hkv + h;
    }
    return page;  // (page, head) block index
  };
  int tcur = resolve(0), tnext = resolve(1), tbase = 0;
  auto issue = [&](lds_u8* buf, int il) __attribute__((always_inline)) {  // il: unit index in the slice
    if (il - tbase == 64) {  // units are issued in order: rotate the tables
      tbase += 64;
      tcur = tnext;
      tnext = resolve((tbase >> 6) + 1);
    }
    const int blk = __builtin_amdgcn_readlane(tcur, il - tbase);
    const uint8_t* src = kpool + (size_t)blk * kLBlock;
#pragma unroll
    for (int t = 0; t < kLPW; ++t) lds_dma16(src + src_off(t), buf + (wave * kLPW + t) * 1024);
  };

  // running softmax state and operands of the open piece, per head group: bf16 Q^T chunks (all 18
  // without QF8, the last two with it) and, with QF8, the e4m3 terms of dims 0..511 with their
  // block-scale operands
  float m[NHG], l[NHG];
  f32x4 o[NHG][kLV / 16];
  constexpr int kQB = QF8 ? 1 : kLD / 32;
  bf16x8 qop[NHG][kQB];
  i32x8 qt[NHG][QF8 ? kLQF8 + 1 : 1][kQT];  // chunk kLQF8: the packed tail (term 2 in its upper half)
  int qs[NHG][QF8 ? kLQF8 + 1 : 1];
  int cur_seg = -1, cur_part = -1, part_end = 0;
  float c_log2 = 0.0f;

  auto flush = [&]() __attribute__((always_inline)) {
    if (cur_seg < 0) return;
    const int b = cur_seg / Hkv, h = cur_seg - b * Hkv;
    const float vs = a.k_scale[h];  // shared-KV: V values are K values, with K's scale
    const int W = px.unit[b + 1] - px.unit[b];
    const int npart = px.part[b + 1] - px.part[b];
    const long seg_first = (long)Hkv * px.unit[b] + (long)h * W;
    const bool whole = npart == 1 && seg_first >= lo && seg_first + W <= hi;
    const long sg = (long)Hkv * px.part[b] + (long)h * npart + cur_part;
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      const int gq = gq0 + 16 * hg;
      const float l_tot = xor_sum(l[hg]);
      if (whole) {  // whole (sequence, head): final rows
        const float r = vs / l_tot;
        const size_t ob = ((size_t)b * a.Hq + (size_t)h * G + gq) * kLV;
#pragma unroll
        for (int dt = 0; dt < kLV / 16; ++dt) {
          const f32x4 v = o[hg][dt] * r;
          const size_t oi = ob + 16 * dt + 4 * grp;
          if (a.out_dt == DAPF8_ACT_BF16) {
            const uint32_t x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
            const uint32_t y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
            *reinterpret_cast<uint2*>((uint16_t*)a.out + oi) = make_uint2(x, y);
          } else {
            *reinterpret_cast<f32x4*>((float*)a.out + oi) = v;
          }
        }
      } else {
        float* pc = a.ws_o + (sg + k) * piece_stride + (long)gq * (kLV + 4);
#pragma unroll
        for (int dt = 0; dt < kLV / 16; ++dt) *reinterpret_cast<f32x4*>(pc + 16 * dt + 4 * grp) = o[hg][dt] * vs;
        if (grp == 0) {
          pc[kLV] = m[hg];
          pc[kLV + 1] = l_tot;
        }
      }
    }
  };

  auto open = [&](const Cursor& c) __attribute__((always_inline)) {
    flush();
    cur_seg = c.b * Hkv + c.h;
    cur_part = c.j / upp;
    part_end = (cur_part + 1) * upp;
    c_log2 = a.sm_scale * a.k_scale[c.h] * kLog2e;
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      m[hg] = -INFINITY;
      l[hg] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < kLV / 16; ++dt) o[hg][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // bf16 Q^T operand of chunk cc: dims 64(cc/2) + 16grp + 8(cc%2) .. +7 of the group's query
      // head (the same dimension order as the K operand's 16-byte reads)
      const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)c.b * a.Hq + (size_t)c.h * G + gq0 + 16 * hg) * kLD;
      if (!QF8) {
#pragma unroll
        for (int cc = 0; cc < kQB; ++cc)
          qop[hg][cc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 64 * (cc >> 1) + 16 * grp +
                                                                                        8 * (cc & 1)));
      } else {
        // e4m3 terms of chunk ch: this lane holds dims 128 ch + 16 grp .. +15 and 128 ch + 64 + 16 grp
        // .. +15 of the head, the same dims as the K operand's two 16-byte reads
#pragma unroll
        for (int ch = 0; ch < kLQF8; ++ch) {
          float x[32];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 128 * ch + 64 * (v >> 1) + 16 * grp + 8 * (v & 1));
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[8 * v + 2 * e] = __uint_as_float(u[e] << 16);
              x[8 * v + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
            }
          }
          split_q_fp8<kQT>(x, grp, qt[hg][ch], qs[hg][ch]);
        }
        // dims 512 + 16 grp .. +15 (the tail), both terms in one operand
        float y[16];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 512 + 16 * grp + 8 * v);
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[8 * v + 2 * e] = __uint_as_float(u[e] << 16);
            y[8 * v + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
          }
        }
        split_q_fp8_tail(y, grp, qt[hg][kLQF8][0], qs[hg][kLQF8]);
      }
    }
    // wait for the query here, on this (rare) path: the pages' LDS loads are older in the counter,
    // and waiting at the join instead would drain the next page's loads on every page
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  // One 32-token window (tokens 32wv .. 32wv+31 of the page in buf); nv = valid tokens in it.
  // Token groups: k-group q of the P.V product holds window tokens S_q[e] = 8q + (e ^ 4*(q&1)),
  // e < 8 (group 8q..8q+7, halves swapped for odd q); S^T tile t row 4q+i is token S_q[4t+i], so
  // lane (head, q) gets exactly S_q's scores.  This order makes every 8 lanes of the 16-byte K
  // reads and every 16 lanes of the transposed V reads hit distinct LDS bank groups.
  auto window = [&](const lds_u8* buf, int wv, int nv) __attribute__((always_inline)) {
    f32x4 acc[NHG][2];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) acc[hg][0] = acc[hg][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // this window's lane offsets are recomputed from an opaque copy of the lane id (a few integer
    // instructions): kept live across the page loop they would take registers the operands need
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = ln & 15, grp = ln >> 4;
    const int rq = row >> 2;
    // K rows of the two 16-token tiles (see the token order above)
    const lds_u8* kr0 = buf + (32 * wv + 8 * rq + 4 * (rq & 1) + (row & 3)) * kLRow;
    const lds_u8* kr1 = buf + (32 * wv + 8 * rq + 4 * (1 ^ (rq & 1)) + (row & 3)) * kLRow;
    if (QF8) {
      // dims 128 ch + 16 grp .. +15 and 128 ch + 64 + 16 grp .. +15 straight from LDS as e4m3 codes
      // (scale 2^0) against each query term of each head group.  Both tiles' operands of a chunk
      // are read together and their products alternate, so consecutive products never depend on
      // each other.
#pragma unroll
      for (int ch = 0; ch < kLQF8; ++ch) {
        i32x8 kop[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const lds_u8* kr = t ? kr1 : kr0;
          const u32x4 w0 = lds_read16(kr + 128 * ch + 16 * grp);
          const u32x4 w1 = lds_read16(kr + 128 * ch + 64 + 16 * grp);
          kop[t] = i32x8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        }
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
          for (int j = 0; j < kQT; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[hg][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop[t], qt[hg][ch][j], acc[hg][t], 0, 0, 0,
                                                                            127, 0, qs[hg][ch]);
        // keep each chunk's reads and products together: the scheduler would otherwise hoist every
        // read of the window and run out of registers
        __builtin_amdgcn_sched_barrier(0);
      }
      // the tail: dims 512 + 16 grp .. +15 in both halves of the operand, against the packed terms
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 w = lds_read16((t ? kr1 : kr0) + 512 + 16 * grp);
        const i32x8 kop = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, (int)w.x, (int)w.y, (int)w.z, (int)w.w};
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg)
          acc[hg][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qt[hg][kLQF8][0], acc[hg][t], 0, 0, 0,
                                                                        127, 0, qs[hg][kLQF8]);
      }
    } else {
      // 16 bytes = dims 64p + 16grp .. +15: the first 8 feed chunk 2p, the next 8 chunk 2p+1
#pragma unroll
      for (int pp = 0; pp < kLD / 64; ++pp) {
        bf16x8 k0[2], k1[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 w = lds_read16((t ? kr1 : kr0) + 64 * pp + 16 * grp);
          k0[t] = fp8x8_to_bf16x8(w.x, w.y);
          k1[t] = fp8x8_to_bf16x8(w.z, w.w);
        }
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[hg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0[t], qop[hg][2 * pp], acc[hg][t], 0, 0, 0);
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[hg][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1[t], qop[hg][2 * pp + 1], acc[hg][t], 0, 0, 0);
        }
      }
    }
    // this lane now holds, per head group, the scores of window tokens S_grp[i] (i < 8) for its head
    const int swz = 4 * (grp & 1);
    bf16x8 pop[NHG][PSPLIT];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      float s[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = acc[hg][0][i] * c_log2;
        s[4 + i] = acc[hg][1][i] * c_log2;
      }
      if (nv < 32) {  // the sequence's last window: tokens past the end get no weight
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (8 * grp + (i ^ swz) >= nv) s[i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mx = xor_max(mx);
      if (__builtin_expect(__any(mx > m[hg] + kRescaleSlack), 0)) {
        const float m_new = fmaxf(m[hg], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[hg] - m_new);  // 0 on the first window (m = -inf)
        m[hg] = m_new;
        l[hg] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kLV / 16; ++dt) o[hg][dt] *= alpha;
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m[hg]);
      l[hg] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      split_bf16<PSPLIT>(p, pop[hg]);
    }
    // V^T operand via the transposing read: source lane 16grp + 2e + hh addresses token S_grp[e],
    // dims 16dt + 8hh; output lane 16grp + r receives dim 16dt + r of tokens S_grp[0..7].  Each
    // operand feeds every head group.
    const int sl = lane & 15;
    const lds_u8* vr = buf + (32 * wv + 8 * grp + ((sl >> 1) ^ swz)) * kLRow + 8 * (sl & 1);
    // Operands are read four at a time, and the next four reads are issued before the current four
    // are widened and multiplied, so LDS latency overlaps the products.
    constexpr int kVB = 4;
    auto vread = [&](u32x2 (&w)[kVB], int dt0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kVB; ++u) w[u] = lds_read8_tr(vr + 16 * (dt0 + u));
    };
    auto vmul = [&](const u32x2 (&w)[kVB], int dt0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kVB; ++u) {
        // rows past the sequence end were zeroed in LDS (a stale code could be NaN, and NaN x 0 = NaN)
        const bf16x8 vop = fp8x8_to_bf16x8(w[u].x, w[u].y);
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
          for (int t = 0; t < PSPLIT; ++t)
            o[hg][dt0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[hg][t], o[hg][dt0 + u], 0, 0, 0);
      }
    };
    u32x2 wa[kVB], wb[kVB];
    vread(wa, 0);
#pragma unroll
    for (int dt0 = 0; dt0 < kLV / 16; dt0 += 2 * kVB) {
      vread(wb, dt0 + kVB);
      __builtin_amdgcn_sched_barrier(0);
      vmul(wa, dt0);
      __builtin_amdgcn_sched_barrier(0);
      if (dt0 + 2 * kVB < kLV / 16) vread(wa, dt0 + 2 * kVB);
      __builtin_amdgcn_sched_barrier(0);
      vmul(wb, dt0 + kVB);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto page = [&](const lds_u8* buf, const Cursor& c) __attribute__((always_inline)) {
    if (c.b * Hkv + c.h != cur_seg || c.j >= part_end) open(c);
    const int nv = min(kLP, uni(px.len[c.b]) - kLP * c.j);  // valid tokens of this page (>= 1)
    window(buf, 0, min(nv, 32));
    if (nv > 32) window(buf, 1, nv - 32);
  };

  // A ring of three LDS page buffers: page i + 2 is loaded while page i is computed.  At the top of
  // iteration i each wave waits for its own loads of page i (vmcnt(kLPW): page i + 1's may stay
  // outstanding); the barrier then makes every wave's loads of page i visible and guarantees every
  // wave has finished page i - 1, whose buffer page i + 2 then reuses.  One barrier per page.
  Cursor cc = cursor_at(lo);  // next unit to compute
  issue(ring, 0);
  if (n > 1) issue(ring + kBufBytes, 1);
  for (int i = 0; i < n; ++i) {
    if (i + 1 < n)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kLPW & 15) | ((kLPW >> 4) << 14));  // vmcnt(kLPW)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    {
      // A sequence's last page: rows past its end hold stale codes (possibly NaN).  Each wave zeroes
      // the stale rows among the units it loaded itself (its loads of this page have landed), before
      // the barrier publishes the page, so the P.V product needs no masking.
      const int nv = min(kLP, uni(px.len[cc.b]) - kLP * cc.j);
      if (nv < kLP) {
        lds_u8* buf = ring + (i % kLRing) * kBufBytes;
#pragma unroll
        for (int t = 0; t < kLPW; ++t) {
          const int u = (wave * kLPW + t) * 64 + lane;
          const int tr = u / kLRowUnits;
          if (tr >= nv && tr < kLP) *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(buf + 16 * u) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    wg_barrier();
    if (i + 2 < n) issue(ring + ((i + 2) % kLRing) * kBufBytes, i + 2);
    page(ring + (i % kLRing) * kBufBytes, cc);
    advance(cc);
  }
  flush();
  // A slice that ends exactly on a partition boundary inside a (sequence, head) leaves the slot of
  // (next partition, this workgroup) unused: write an empty piece there (m = -inf, l = 0, zeros).
  if (cur_seg >= 0) {
    const int b = cur_seg / Hkv, h = cur_seg - b * Hkv;
    const int W = px.unit[b + 1] - px.unit[b];
    const int npart = px.part[b + 1] - px.part[b];
    const long rel = hi - ((long)Hkv * px.unit[b] + (long)h * W);
    if (npart > 1 && rel < W && rel % upp == 0) {
      const long slot = (long)Hkv * px.part[b] + (long)h * npart + rel / upp + k;
#pragma unroll
      for (int hg = 0; hg < NHG; ++hg) {
        float* pc = a.ws_o + slot * piece_stride + (long)(gq0 + 16 * hg) * (kLV + 4);
#pragma unroll
        for (int dt = 0; dt < kLV / 16; ++dt)
          *reinterpret_cast<f32x4*>(pc + 16 * dt + 4 * grp) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (grp == 0) {
          pc[kLV] = -INFINITY;
          pc[kLV + 1] = 0.0f;
        }
      }
    }
  }
}

// Workgroups the GPU keeps resident for one instantiation (cached per device, so launches inside
// a graph capture make no runtime queries).
template <auto Kernel>
static int resident_workgroups(int threads) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0, cus = 0, wgs = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs, Kernel, threads, 0) != hipSuccess) return 0;
  const int n = cus * (wgs > 0 ? wgs : 1);
  if (dev >= 0 && dev < kMaxDev) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int launch_attn_latent(const AttnArgs& a, int max_workgroups, hipStream_t s) {
  const bool f32out = a.out_dt == DAPF8_ACT_F32;
  int nwg = 0;
#define DAPF8_LAT(NW, NHG, PS)                                                                      \
  do {                                                                                              \
    auto kern = attn_latent_kernel<NW, NHG, PS, PS == 1>;                                           \
    nwg = min(resident_workgroups<attn_latent_kernel<NW, NHG, PS, PS == 1>>(NW * 64), max_workgroups); \
    if (nwg < 1) return set_error(DAPF8_ELAUNCH, "paged_decode_attn: no resident workgroups");     \
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(NW * 64), 0, s, a, nwg);                    \
  } while (0)
  // bf16 output: P keeps 8 bits (one bf16 term) and QK runs on the FP8 matrix cores; fp32 output: P
  // keeps ~24 bits (three terms) and QK runs in bf16.  16 query heads per wave.
  switch (a.G) {
    case 16: if (f32out) DAPF8_LAT(1, 1, 3); else DAPF8_LAT(1, 1, 1); break;
    case 32: if (f32out) DAPF8_LAT(2, 1, 3); else DAPF8_LAT(2, 1, 1); break;
    case 64: if (f32out) DAPF8_LAT(4, 1, 3); else DAPF8_LAT(4, 1, 1); break;
    case 128: if (f32out) DAPF8_LAT(8, 1, 3); else DAPF8_LAT(8, 1, 1); break;
    default: return set_error(DAPF8_EUNSUPPORTED, "paged_decode_attn: latent kernel needs G in {16,32,64,128}");
  }
#undef DAPF8_LAT
  const int rc = check_launch("paged_decode_attn (latent)");
  if (rc != DAPF8_OK) return rc;
  return launch_merge_sk(a, nwg, s);
}

}  // namespace dapf8
