/*
 * dapf8.h -- C ABI of the paged FP8 decode-attention library for AMD MI355X (gfx950).
 *
 * The library implements the decode-phase hot path described in Cloudflare's post
 * "Smaller, faster, safer: running Kimi and GLM at scale" (read here in its Chinese translation
 * on feinterview.poetries.top, and in the siami.tw and remio.ai write-ups of it):
 *
 *   - section "量化 KV cache" (quantize the KV cache): K and V of every processed token are
 *     stored as 8-bit floating point (FP8, e4m3) instead of BF16, halving the cache; the FP8
 *     attention kernel converts the stored values when it reads them.  A BF16 twin is kept for
 *     the comparison the pages make between the two kernels.
 *   - section "保护共享 KV cache" (protect the shared KV cache): every physical cache page has a
 *     tag that changes when the page is reallocated; the server records the pages and tags each
 *     request expects; before a supported decode operation reads the cache the mapping is checked
 *     and any mismatch aborts the affected request.  The check is a separate batched pass, not
 *     fused into attention; with checking disabled the tracker is a no-op.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers into memory the caller owns (for instance torch
 *     tensors).  The library allocates nothing on these paths and keeps no state between calls.
 *   - Every tensor pointer must be 16-byte aligned; arrays are dense and row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only enqueued; the call
 *     returns before it runs.  Calls are thread-safe.
 *   - Return value: DAPF8_OK (0) or a negative DAPF8_E* code; dapf8_last_error() then returns a
 *     message for the calling thread.  Arguments are checked on the host before any launch.
 *     Device-resident data (page ids, lengths, sequence ids) cannot be checked on the host: the
 *     kernels clamp or skip out-of-range values so that no access leaves the buffers described
 *     by the size arguments, and the results for such rows are then unspecified -- run
 *     kv_tag_verify first to turn bad page references into aborts.
 *
 * Data layout (physical page pool; P = page_size tokens per page)
 *   K pool : [num_pages][Hkv][Dk/C][P][C] elements, C = 64 bytes' worth of dimensions (64 FP8 codes
 *            or 32 bf16 values): inside a (page, head) block each token's row is cut into 64-byte
 *            dimension chunks, stored chunk by chunk (every token's chunk 0, then chunk 1, ...), so
 *            K[page][h][token t][dim d] is element ((page*Hkv + h)*P*Dk) + (d/C)*P*C + t*C + d%C.
 *            Dk must be a multiple of 64.
 *   V pool : [num_pages][Hkv][Dv][P]      elements, dimension-major inside a (page, head) block
 *   Element type: one byte per value (FP8 e4m3 code) or two bytes (bf16 bit pattern).
 *   Token t of sequence b is stored in page page_table[b * pt_stride + t / P], slot t % P.
 *   Shared-KV mode (v_pool == NULL): V of a token is the first Dv values of its K row.
 *
 * FP8 format: OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF = NaN, largest finite 448).
 * Quantisation of a value x with scale s: t = x / s as a correctly rounded fp32 division, then
 * the nearest e4m3 value with ties to even mantissa, saturating to +-448 (NaN stays NaN).
 * Dequantisation: code value * s, exactly.
 */
#ifndef DAPF8_H
#define DAPF8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* KV storage type */
#define DAPF8_KV_FP8_E4M3 0
#define DAPF8_KV_BF16 1
/* activation (query, new K/V rows, output) type */
#define DAPF8_ACT_F32 0
#define DAPF8_ACT_BF16 1

/* return codes */
#define DAPF8_OK 0
#define DAPF8_EINVAL (-1)       /* invalid argument (null pointer, bad size, misalignment) */
#define DAPF8_EUNSUPPORTED (-2) /* shape or dtype combination not supported */
#define DAPF8_EWORKSPACE (-3)   /* workspace missing or smaller than the size query returned */
#define DAPF8_ELAUNCH (-4)      /* the HIP runtime reported an error when launching */

/* Message describing the last non-zero return on the calling thread ("" if none). */
const char* dapf8_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int dapf8_version(void);

/* ---------------------------------------------------------------------------------------------
 * Scale setup (the pages say only that the cache is FP8 e4m3; the per-head scale is the
 * reading adopted: s = fp32(amax / 448) over the initial fill of that KV head, fixed afterwards).
 *
 * kv_absmax_update: amax[h] = max(amax[h], max over t, d of |x[t][h][d]|), so a fill can be
 *   processed in chunks.  x : [T][H][D] (fp32 or bf16 per x_dt); amax : [H] fp32, in/out, must
 *   hold non-negative values on entry (zeros to start).  NaN inputs are ignored.  T = 0 is a
 *   no-op.  D must be a multiple of 4.
 * kv_scale_from_absmax: scale[h] = amax[h] / 448 (correctly rounded fp32 division), or 1.0 when
 *   amax[h] == 0.  amax, scale : [H] fp32; they may alias.
 * ------------------------------------------------------------------------------------------- */
int kv_absmax_update(const void* x, int x_dt, int64_t T, int32_t H, int32_t D, float* amax, void* stream);
int kv_scale_from_absmax(const float* amax, int32_t H, float* scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kv_append -- quantize-on-append of new tokens' K/V into their page slots
 * ("量化 KV cache": the cache holds FP8 e4m3 values; BF16 for the twin).
 *
 *   k_new : [T][Hkv][Dk], v_new : [T][Hkv][Dv]   fp32 or bf16 (in_dt); v_new ignored when
 *                                                 v_pool == NULL (shared-KV mode)
 *   k_pool, v_pool : pools in the layout above, element type kv_dt (written in place)
 *   page_table : [B][pt_stride] int32 physical page ids
 *   seq_ids, positions : [T] int32 -- token i is position positions[i] of sequence seq_ids[i]
 *   k_scale, v_scale : [Hkv] fp32 per-head scales (FP8 only; may be NULL for BF16)
 *   abort_mask : [B] uint8 or NULL; tokens of sequences with a non-zero entry are not written
 * FP8: code = e4m3(fp32(x / s_head)).  BF16: the nearest bf16 value (ties to even).
 * Requirements: Dk a multiple of 64, Dv a multiple of 16; page_size >= 1; B, Hkv >= 1; T >= 0 (0 = no-op).
 * Tokens whose sequence id, position or page id is out of range are skipped.  Two tokens that
 * name the same slot race; the caller must not do that.
 * ------------------------------------------------------------------------------------------- */
int kv_append(const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool, int kv_dt,
              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_ids, const int32_t* positions,
              int32_t T, const float* k_scale, const float* v_scale, const uint8_t* abort_mask, int32_t B,
              int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_pages, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kv_tag_verify -- the batched page-tag integrity check ("保护共享 KV cache").
 *
 *   page_table, expected_tags : [B][pt_stride] (int32 page ids, uint32 tags the request expects)
 *   seq_lens : [B] int32 tokens in each request's cache;  live_tags : [num_pages] uint32
 *   abort_mask : [B] uint8 output, written for every b:
 *     abort[b] = 1 if L_b < 0, or L_b > pt_stride * page_size, or for some j < ceil(L_b / P)
 *                  page_table[b][j] is outside [0, num_pages) or
 *                  live_tags[page_table[b][j]] != expected_tags[b][j];   else 0.
 * Tags are compared for equality only (a generation counter that may wrap).  Entries past a
 * request's pages are ignored.  Deterministic: one workgroup owns each request's bit, no atomics.
 * Run it on the same stream before kv_append and paged_decode_attn and pass its mask to both.
 * With checking disabled, do not call it and pass abort_mask = NULL (no work at all).
 * ------------------------------------------------------------------------------------------- */
int kv_tag_verify(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                  const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                  int32_t B, int32_t page_size, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kv_tag_verify_append -- kv_tag_verify followed by kv_append with its mask, in one launch
 * ("保护共享 KV cache": check every page reference before the step uses it; "量化 KV cache":
 * quantize-on-append).  For a decode step's few new tokens.
 *
 *   Arguments as for kv_tag_verify and kv_append (the append's B, page_table, pt_stride,
 *   page_size and num_pages are the check's: num_pages is both the pools' page count and the
 *   length of live_tags); abort_mask : [B] uint8 output, required.
 * Results are those of kv_tag_verify(...) then kv_append(..., abort_mask) on the same stream, bit
 * for bit: the mask as defined for kv_tag_verify, and the tokens of requests whose bit is 0
 * written as kv_append writes them (tokens of aborted requests, and tokens whose sequence id,
 * position or page id is out of range, are skipped).  One workgroup per request checks its tags
 * and then writes its own tokens, so the append never waits for another workgroup.  Any T is
 * accepted; past 64 tokens of one request, or 4 * 256 (wide tables: 4 * 1024) tokens in the
 * call, a request's workgroup rescans the token list, which is slower than the two separate
 * calls.  T = 0 performs the check alone; B = 0 with T = 0 is a no-op.  Same races as kv_append
 * for tokens naming one slot.  Errors: DAPF8_EINVAL for the conditions either call rejects.
 * ------------------------------------------------------------------------------------------- */
int kv_tag_verify_append(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                         const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                         const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool, int kv_dt,
                         const int32_t* seq_ids, const int32_t* positions, int32_t T, const float* k_scale,
                         const float* v_scale, int32_t B, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size,
                         void* stream);

/* ---------------------------------------------------------------------------------------------
 * kv_transcode_pages -- copy whole pages of a BF16 pool into an FP8 pool, quantising every value
 * as kv_append does (the pages keep a BF16 cache for compute-bound prefill and an FP8 cache for
 * memory-bound decode, "量化 KV cache"; this is the handoff of a request's cache between them).
 *
 *   k_src, v_src : BF16 pools, [num_src_pages][Hkv][Dk/32][P][32] and [num_src_pages][Hkv][Dv][P]
 *   k_dst, v_dst : FP8 pools,  [num_dst_pages][Hkv][Dk/64][P][64] and [num_dst_pages][Hkv][Dv][P]
 *                  (v_src and v_dst both NULL: shared-KV pools, K only)
 *   src_pages, dst_pages : [n_pages] int32 -- page src_pages[i] is written to page dst_pages[i]
 *   k_scale, v_scale : [Hkv] fp32 per-head scales of the destination cache
 * For every pair, head h, slot t and dimension d:
 *   K_dst[dst][h][t][d] = e4m3(fp32(K_src[src][h][t][d]) / k_scale[h])   (and V with v_scale)
 * with the division and rounding of kv_append (correctly rounded fp32 division, nearest e4m3 with
 * ties to even, saturating at +-448, NaN kept).  Pairs with a page id out of range are skipped.
 * Destination pages must be distinct and the pools must not overlap (such writes race).
 * Requirements: Dk a multiple of 64, Dv a multiple of 16, page_size >= 1, n_pages >= 0 (0 = no-op).
 * ------------------------------------------------------------------------------------------- */
int kv_transcode_pages(const void* k_src, const void* v_src, void* k_dst, void* v_dst, const int32_t* src_pages,
                       const int32_t* dst_pages, int32_t n_pages, const float* k_scale, const float* v_scale,
                       int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_src_pages,
                       int32_t num_dst_pages, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Device-resident page allocator and tag tracker ("保护共享 KV cache": every physical page has a
 * tag that changes when the page is reallocated, and requests record the (page, tag) pairs they
 * expect; kv_tag_verify compares the two).  State, all caller-owned device memory:
 *   free_list : [num_pages] int32, a stack of free page ids (entries [0, *free_count) are free,
 *               the top is entry *free_count - 1);   free_count : [1] int32
 *   live_tags : [num_pages] uint32, or NULL for the no-op tracker (no tags kept, nothing checked)
 * Calls on one allocator must be ordered (one stream); each is a single-workgroup kernel, so
 * results are deterministic.
 *
 * kv_pages_init: free_list[i] = num_pages - 1 - i (page 0 on top), *free_count = num_pages,
 *   live_tags[i] = 0.
 * kv_pages_alloc: requests b = 0..B-1 ask for counts[b] pages in slots
 *   [first_slot[b], first_slot[b] + counts[b]) of row b of page_table ([B][pt_stride] int32, at
 *   least B rows).
 *   Request b is valid when counts[b] >= 0, first_slot[b] >= 0 and the slot range fits the row; it
 *   is granted (granted[b] = 1, else 0) when it is valid and the pages of all valid requests up to
 *   and including it fit in *free_count -- so the granted requests are the valid ones before the
 *   first valid request that does not fit, and nothing else is written for the others.  Granted
 *   requests take pages from the top of the stack in request order (request 0's slot 0 gets the top
 *   page); each handed-out page's live tag is incremented (wrapping) and, when expected_tags
 *   ([B][pt_stride] uint32) is given, the new tag is recorded at the same slot.  B <= 8192.
 * kv_pages_free: pushes pages[0..n) onto the stack in order.  Ids outside [0, num_pages) are
 *   rejected, as are ids beyond the stack's room; status[0] = ids pushed, status[1] = ids rejected.
 *   Tags are not changed here: a freed page keeps its tag until it is handed out again.
 *   Freeing a page that is already free, or twice, corrupts the allocator (not detected).
 * ------------------------------------------------------------------------------------------- */
int kv_pages_init(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages, void* stream);
int kv_pages_alloc(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages,
                   const int32_t* counts, const int32_t* first_slot, int32_t B, int32_t* page_table,
                   uint32_t* expected_tags, int32_t pt_stride, uint8_t* granted, void* stream);
int kv_pages_free(int32_t* free_list, int32_t* free_count, const int32_t* pages, int32_t n, int32_t num_pages,
                  int32_t* status, void* stream);

/* ---------------------------------------------------------------------------------------------
 * paged_decode_attn -- decode attention over the paged cache, dequantising on read
 * ("量化 KV cache": the FP8 kernel converts on every read; BF16 twin for comparison).
 *
 * For each request b and query head h (KV head g = h / (Hq / Hkv)), with L = seq_lens[b]:
 *   s_t = sm_scale * sum_d q[b][h][d] * K_t[d]           t in [0, L)
 *   out[b][h][:] = sum_t softmax(s)_t * V_t[:]
 * where K_t, V_t are the stored values times their per-head scales (FP8) or the bf16 values.
 * Rows of requests with abort_mask[b] != 0 and rows with L <= 0 are written as zeros.
 * Long sequences are split into parts whose partial results (max, sum, unnormalised output) are
 * combined with the log-sum-exp rule.  The fixed-partition kernels cut them into partitions of
 * split_tokens tokens (0 lets the library choose); the persistent kernels (variants
 * "mfma_streamk_*", "mfma_latent_*") give every resident wave or workgroup an equal slice of all
 * the work and their parts are those slices, so they ignore split_tokens.  The results agree to
 * rounding; paged_decode_attn_variant reports the split a call will use.
 *
 *   q   : [B][Hq][Dk] fp32 or bf16 (q_dt);   out : [B][Hq][Dv] fp32 or bf16 (out_dt, RNE)
 *   k_pool / v_pool / page_table / pt_stride : as for kv_append (v_pool NULL = shared-KV, Dv <= Dk)
 *   k_scale, v_scale : [Hkv] fp32 (FP8 only; v_scale unused in shared-KV mode)
 *   workspace : device buffer of at least paged_decode_attn_workspace_size(...) bytes with the
 *               same shape arguments (may be NULL when that size is 0); contents are scratch.
 * Requirements: Hq % Hkv == 0; Dk a multiple of 64 and Dv a multiple of 16, both <= 1024;
 * split_tokens a multiple of 32 (or 0); page_size >= 1; num_pages >= 1, num_pages * Hkv < 2^31.
 * ------------------------------------------------------------------------------------------- */
size_t paged_decode_attn_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                        int32_t page_size, int32_t pt_stride, int32_t split_tokens, int kv_dt,
                                        int shared_kv);

int paged_decode_attn(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                      const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens, const float* k_scale,
                      const float* v_scale, const uint8_t* abort_mask, void* out, int out_dt, float sm_scale,
                      int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size,
                      int32_t num_pages, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------------------------
 * paged_decode_attn_noalloc -- paged_decode_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments and results as paged_decode_attn, without workspace arguments: the kernels'
 * scratch (partial results of split sequences) is a device array of DAPF8_NOALLOC_SCRATCH_BYTES
 * bytes (64 MiB) inside the library, which every GPU the
 * library runs on holds from the first call until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).  Shapes whose workspace
 * (paged_decode_attn_workspace_size) exceeds the scratch size fail with DAPF8_EWORKSPACE before
 * anything is launched.  The calling thread's current device must be the one the stream and the
 * buffers belong to.  All calls on one GPU share its scratch array: calls that may overlap in time
 * on one GPU (other streams, other threads) race and must not be made; calls ordered on one stream
 * are safe.  No state carries from one call to the next.
 * ------------------------------------------------------------------------------------------- */
#define DAPF8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int paged_decode_attn_noalloc(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                              const float* k_scale, const float* v_scale, const uint8_t* abort_mask, void* out,
                              int out_dt, float sm_scale, int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                              int32_t page_size, int32_t num_pages, int32_t split_tokens, void* stream);

/* ---------------------------------------------------------------------------------------------
 * paged_decode_attn_checked -- the page-tag check done inside attention's page walk instead of
 * as a separate batched pass (the fused alternative the pages weigh against their separate check
 * in "保护共享 KV cache"; provided to measure the two against each other).
 *
 * Same arguments as paged_decode_attn except: no abort_mask input and no split_tokens; the tag
 * arrays of kv_tag_verify (expected_tags [B][pt_stride], live_tags [num_pages]); and
 * abort_mask_out [B] uint8, written with exactly kv_tag_verify's mask.  Rows of aborted requests
 * are zeros and every other row equals paged_decode_attn's with that mask.  Each page is checked
 * by the waves that read it, as it is read; a request's verdict is combined where its partial
 * results are.  This does not protect kv_append, which writes before attention runs: the separate
 * check is the one to use when appends must be guarded.
 * Supported: the persistent matrix-core shape only (variant "mfma_streamk_*": Dk = Dv = 128,
 * page_size 16, Hq / Hkv <= 16, separate V pool), bf16 queries; DAPF8_EUNSUPPORTED otherwise.
 * The workspace is paged_decode_attn_workspace_size(..., split_tokens = 0, ...).
 * ------------------------------------------------------------------------------------------- */
int paged_decode_attn_checked(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                              const uint32_t* expected_tags, const uint32_t* live_tags, const float* k_scale,
                              const float* v_scale, uint8_t* abort_mask_out, void* out, int out_dt, float sm_scale,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size,
                              int32_t num_pages, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * INT4 weight-only decode GEMV (the pages compress GLM's weights from 8-bit floats to 4-bit
 * integers, which speeds the memory-bound decode phase; here with synthetic weights, throughput
 * only).  Reading: symmetric 4-bit integers q in [-8, 7] with one fp32 scale per output column and
 * 128-wide group of k; activations bf16; fp32 accumulation.
 *
 * w4_pack: q [N][K] int8 (values outside [-8, 7] saturate), scales [N][K/128] fp32 ->
 *   packed [N/16][K/128][16][64] bytes (N*K/2 bytes): the 64 bytes of output column n = 16*t + c
 *   and k block kb hold k = 128*kb + 32g + 8j + e in the little-endian dword at byte 16g + 4j
 *   (g, j = 0..3; e = 0..7), element e in nibble p = e/2 (e even) or 4 + e/2 (e odd), nibble p
 *   being bits 4p..4p+3, each nibble q + 8;  packed_scales [K/128][N] fp32.
 * w4a16_gemv: y[m][n] = sum_k x[m][k] * q[n][k] * scales[n][k / 128] for m < M.
 *   x [M][K] bf16; y [M][N] fp32 or bf16 (out_dt, RNE).  M <= 16 (decode batch), N a multiple of
 *   64, K a multiple of 128.  M = 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
int w4_pack(const int8_t* q, const float* scales, int32_t N, int32_t K, uint8_t* packed, float* packed_scales,
            void* stream);
int w4a16_gemv(const void* x, const uint8_t* packed, const float* packed_scales, void* y, int out_dt, int32_t M,
               int32_t N, int32_t K, void* stream);

/* ---------------------------------------------------------------------------------------------
 * hbm_read_probe -- a plain read-only streaming kernel, the attainable HBM read rate that the
 * decode kernels are measured against (measurement only; not part of the decode path).
 *
 * Reads n_blocks blocks of block_bytes bytes (a multiple of 1024) with 16-byte non-temporal loads:
 * block i at buf + i * block_bytes (block_ids NULL: the buffer front to back) or at
 * buf + block_ids[i] * block_bytes (the scattered page-block pattern of a paged cache; the ids
 * must lie inside the buffer).  `workgroups` persistent workgroups of 256 threads share the blocks
 * round-robin; each thread writes the XOR of the words it read to sink[workgroup * 256 + thread]
 * (sink holds workgroups * 256 uint32), so that no load can be dropped.
 * ------------------------------------------------------------------------------------------- */
int hbm_read_probe(const void* buf, const int32_t* block_ids, int64_t n_blocks, int32_t block_bytes, uint32_t* sink,
                   int32_t workgroups, void* stream);

/* ---------------------------------------------------------------------------------------------
 * hbm_copy_probe -- a plain read-write streaming kernel with the byte mix of a BF16 -> FP8 page
 * transcode (two bytes read per byte written): the attainable rate of that mixed stream, beside
 * which kv_transcode_pages is measured (measurement only; not part of the decode path).
 *
 * Reads 2 * dst_bytes contiguous bytes of src and writes dst_bytes contiguous bytes of dst (the
 * XOR fold of each 32 bytes read into 16), with 16-byte non-temporal loads and stores;
 * `workgroups` persistent workgroups of 256 threads.  dst_bytes a multiple of 16, pointers 16-byte
 * aligned; the caller owns both buffers.
 * ------------------------------------------------------------------------------------------- */
int hbm_copy_probe(const void* src, void* dst, int64_t dst_bytes, int32_t workgroups, void* stream);

/* Which kernel variant paged_decode_attn would launch for these arguments, and the partition
 * size it would use (for reports and tests; no launch). Returns a static string such as
 * "mfma_g16_d128_p16" or "valu_generic"; *split_out receives the resolved split_tokens. */
const char* paged_decode_attn_variant(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                      int32_t page_size, int32_t pt_stride, int32_t split_tokens, int kv_dt,
                                      int shared_kv, int32_t* split_out);

#ifdef __cplusplus
}
#endif

#endif /* DAPF8_H */
