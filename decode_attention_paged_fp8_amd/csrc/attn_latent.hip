// attn_latent.hip -- decode attention on the matrix cores for the shared-KV ("latent") layout:
// V is the first Dv = 512 dims of each Dk = 576-dim K row, page size 64, FP8 (e4m3) storage,
// G = Hq / Hkv query heads per KV head with G a multiple of 16 up to 128.
//
// [CF §Quantize] the cache holds FP8 codes; the kernel converts them to bf16 on read (exact) and
// folds the single per-head scale into the score and the output.
//
// Why a kernel of its own: with 128 query heads sharing one 576-dim KV row the work is a real
// dense contraction (about 480 flop per cached byte), so the matrix cores -- not HBM -- set the
// pace, and every cached byte must be reused by all query heads.  One workgroup of G / 16 waves
// owns all G heads: each 64-token page is copied once into LDS (direct global->LDS loads, no
// registers), and every wave computes its 16 heads against it:
//   S^T = K Q^T   A = K tile (16 tokens x 32 dims) read from LDS, B = Q^T (32 dims x 16 heads)
//                 held in registers for the whole piece (18 operands = all 576 dims);
//   O^T = V^T P^T A = V^T tile (16 dims x 32 tokens) read from the same LDS page with the
//                 byte-transposing LDS read, B = P^T taken straight from the S^T registers (the token
//                 order inside a 32-token window is permuted so each lane holds the 8 probabilities
//                 its operand needs, as in the 128-dim kernel).
// The page's LDS rows are padded to 592 bytes so both read patterns spread over all LDS banks.
//
// Work decomposition: stream-K over (sequence, KV head, 64-token page) units, one persistent
// workgroup per CU, equal contiguous slices; a slice yields one piece per (sequence, head,
// partition) it touches, combined by merge_sk_kernel (the same piece-slot scheme as the 128-dim
// stream-K kernel).
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

// LDS pointers keep their address space, so the compiler can tell the two page buffers apart
// (a generic pointer would make every LDS read wait for every outstanding global->LDS load)
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 16 bytes per lane from global memory straight into LDS at base + 16 * lane.  Issued as inline
// assembly so the compiler does not treat the LDS writes as outstanding when the other page buffer is
// read (its LDS alias check cannot separate the two buffers and would drain every load); the kernel
// waits for these loads itself (vmcnt) and orders them with barriers.  The compiler keeps no value
// in m0 in this kernel (checked in the generated code), so setting it here is safe.
__device__ __forceinline__ void lds_dma16(const void* src, const lds_u8* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0) : "memory", "m0");
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

// zero the bf16 value e of a lane's 8 (token base + (e ^ swz)) when that token is >= nv (stale
// slots past the sequence end may hold NaN codes)
__device__ __forceinline__ bf16x8 mask_tokens(bf16x8 v, int base, int swz, int nv) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (base + (e ^ swz) >= nv) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  u = u32x4{w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8, u);
}

}  // namespace

template <int NW, int PSPLIT>
__global__ __launch_bounds__(NW * 64) void attn_latent_kernel(AttnArgs a, int nwg) {
  constexpr int kLPW = (kLWaveLoads + NW - 1) / NW;  // wave-wide loads per wave per page
  constexpr int kBufBytes = NW * kLPW * 1024;        // >= kLUnits * 16; the rest is padding
  __shared__ __attribute__((aligned(16))) uint8_t bufA_[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t bufB_[kBufBytes];
  lds_u8* const bufA = (lds_u8*)bufA_;
  lds_u8* const bufB = (lds_u8*)bufB_;
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
  const int gq = 16 * wave + row;  // query head (inside the KV head's group) of this lane's column
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

  // running softmax state and operands of the open piece
  float m = -INFINITY, l = 0.0f;
  f32x4 o[kLV / 16];
  bf16x8 qop[kLD / 32];
  int cur_seg = -1, cur_part = -1, part_end = 0;
  float c_log2 = 0.0f;

  auto flush = [&]() __attribute__((always_inline)) {
    if (cur_seg < 0) return;
    const int b = cur_seg / Hkv, h = cur_seg - b * Hkv;
    const float vs = a.k_scale[h];  // shared-KV: V values are K values, with K's scale
    const float l_tot = xor_sum(l);
    const int W = px.unit[b + 1] - px.unit[b];
    const int npart = px.part[b + 1] - px.part[b];
    const long seg_first = (long)Hkv * px.unit[b] + (long)h * W;
    if (npart == 1 && seg_first >= lo && seg_first + W <= hi) {  // whole (sequence, head): final rows
      const float r = vs / l_tot;
      const size_t ob = ((size_t)b * a.Hq + (size_t)h * G + gq) * kLV;
#pragma unroll
      for (int dt = 0; dt < kLV / 16; ++dt) {
        const f32x4 v = o[dt] * r;
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
      const long sg = (long)Hkv * px.part[b] + (long)h * npart + cur_part;
      float* pc = a.ws_o + (sg + k) * piece_stride + (long)gq * (kLV + 4);
#pragma unroll
      for (int dt = 0; dt < kLV / 16; ++dt) *reinterpret_cast<f32x4*>(pc + 16 * dt + 4 * grp) = o[dt] * vs;
      if (grp == 0) {
        pc[kLV] = m;
        pc[kLV + 1] = l_tot;
      }
    }
  };

  auto open = [&](const Cursor& c) __attribute__((always_inline)) {
    flush();
    cur_seg = c.b * Hkv + c.h;
    cur_part = c.j / upp;
    part_end = (cur_part + 1) * upp;
    c_log2 = a.sm_scale * a.k_scale[c.h] * kLog2e;
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < kLV / 16; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Q^T operand of chunk cc: dims 64(cc/2) + 16grp + 8(cc%2) .. +7 of query head gq (the same
    // dimension order as the K operand's 16-byte reads)
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)c.b * a.Hq + (size_t)c.h * G + gq) * kLD;
#pragma unroll
    for (int cc = 0; cc < kLD / 32; ++cc)
      qop[cc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 64 * (cc >> 1) + 16 * grp +
                                                                               8 * (cc & 1)));
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
    f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
    const int rq = row >> 2;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tok = 8 * rq + 4 * (t ^ (rq & 1)) + (row & 3);
      // 16 bytes = dims 64p + 16grp .. +15: the first 8 feed chunk 2p, the next 8 chunk 2p+1
      const lds_u8* kr = buf + (32 * wv + tok) * kLRow + 16 * grp;
#pragma unroll
      for (int pp = 0; pp < kLD / 64; ++pp) {
        const u32x4 w = lds_read16(kr + 64 * pp);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(w.x, w.y), qop[2 * pp], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(w.z, w.w), qop[2 * pp + 1], acc[t], 0, 0, 0);
      }
    }
    // this lane now holds the scores of window tokens S_grp[i] (i < 8) for head gq
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = acc[0][i] * c_log2;
      s[4 + i] = acc[1][i] * c_log2;
    }
    const int swz = 4 * (grp & 1);
    if (nv < 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (8 * grp + (i ^ swz) >= nv) s[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = xor_max(mx);
    if (__builtin_expect(__any(mx > m + kRescaleSlack), 0)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first window (m = -inf)
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < kLV / 16; ++dt) o[dt] *= alpha;
    }
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m);
    l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    bf16x8 pop[PSPLIT];
    split_bf16<PSPLIT>(p, pop);
    // V^T operand via the transposing read: source lane 16grp + 2e + hh addresses token S_grp[e],
    // dims 16dt + 8hh; output lane 16grp + r receives dim 16dt + r of tokens S_grp[0..7].
    const int sl = lane & 15;
    const lds_u8* vr = buf + (32 * wv + 8 * grp + ((sl >> 1) ^ swz)) * kLRow + 8 * (sl & 1);
#pragma unroll
    for (int dt = 0; dt < kLV / 16; ++dt) {
      const u32x2 w = lds_read8_tr(vr + 16 * dt);
      bf16x8 vop = fp8x8_to_bf16x8(w.x, w.y);
      if (nv < 32) vop = mask_tokens(vop, 8 * grp, swz, nv);
#pragma unroll
      for (int t = 0; t < PSPLIT; ++t) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t], o[dt], 0, 0, 0);
    }
  };

  auto page = [&](const lds_u8* buf, const Cursor& c) __attribute__((always_inline)) {
    if (c.b * Hkv + c.h != cur_seg || c.j >= part_end) open(c);
    const int nv = min(kLP, uni(px.len[c.b]) - kLP * c.j);  // valid tokens of this page (>= 1)
    window(buf, 0, min(nv, 32));
    if (nv > 32) window(buf, 1, nv - 32);
  };

  // Two LDS page buffers in ping-pong: the next page's direct loads are in flight while the
  // current page is computed.  vmcnt(kLPW) waits for this wave's loads of the current page (the
  // newer kLPW loads of the next page may stay outstanding); the barrier then makes every wave's
  // loads visible, and the barrier after the compute frees the buffer for the page after next.
  Cursor cc = cursor_at(lo);  // next unit to compute
  issue(bufA, 0);
  for (int i = 0; i < n; i += 2) {
    if (i + 1 < n) {
      issue(bufB, i + 1);
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kLPW & 15) | ((kLPW >> 4) << 14));  // vmcnt(kLPW)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    wg_barrier();
    page(bufA, cc);
    advance(cc);
    wg_barrier();
    if (i + 1 >= n) break;
    if (i + 2 < n) {
      issue(bufA, i + 2);
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kLPW & 15) | ((kLPW >> 4) << 14));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    wg_barrier();
    page(bufB, cc);
    advance(cc);
    wg_barrier();
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
      float* pc = a.ws_o + slot * piece_stride + (long)gq * (kLV + 4);
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
  const int nw = a.G / 16;
  const bool f32out = a.out_dt == DAPF8_ACT_F32;
  int nwg = 0;
#define DAPF8_LAT(NW, PS)                                                                           \
  do {                                                                                              \
    auto kern = attn_latent_kernel<NW, PS>;                                                         \
    nwg = min(resident_workgroups<attn_latent_kernel<NW, PS>>(NW * 64), max_workgroups);           \
    if (nwg < 1) return set_error(DAPF8_ELAUNCH, "paged_decode_attn: no resident workgroups");     \
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(NW * 64), 0, s, a, nwg);                    \
  } while (0)
  // P keeps 8 bits (one bf16 term) for bf16 output and ~24 bits (three terms) for fp32 output.
  switch (nw) {
    case 1: if (f32out) DAPF8_LAT(1, 3); else DAPF8_LAT(1, 1); break;
    case 2: if (f32out) DAPF8_LAT(2, 3); else DAPF8_LAT(2, 1); break;
    case 4: if (f32out) DAPF8_LAT(4, 3); else DAPF8_LAT(4, 1); break;
    case 8: if (f32out) DAPF8_LAT(8, 3); else DAPF8_LAT(8, 1); break;
    default: return set_error(DAPF8_EUNSUPPORTED, "paged_decode_attn: latent kernel needs G in {16,32,64,128}");
  }
#undef DAPF8_LAT
  const int rc = check_launch("paged_decode_attn (latent)");
  if (rc != DAPF8_OK) return rc;
  return launch_merge_sk(a, nwg, s);
}

}  // namespace dapf8
