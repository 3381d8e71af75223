// api.hip -- the C ABI declared in include/dapf8.h: host-side argument checks, kernel-variant
// choice, partition sizing and launches on the caller's stream.  No allocation, no global state
// beyond the thread-local error message.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "common.hpp"

namespace dapf8 {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DAPF8_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return DAPF8_OK;
}

namespace {

// Scratch held by the no-allocation entry point on each device.
constexpr size_t kScratchBytes = DAPF8_NOALLOC_SCRATCH_BYTES;

// Workgroups the library aims for when it picks the partition size (256 CUs, a few waves each).
constexpr int64_t kTargetMfmaWG = 2048;
constexpr int64_t kTargetGenericWG = 2048;

struct Plan {
  Variant variant;
  const char* name;
  int32_t gb;          // generic kernel: query heads per workgroup
  int32_t alt_gb;      // latent variant: the generic plan's (fp32 queries)
  int32_t split;
  int32_t nsplit;      // fixed-partition kernels: partitions of the longest possible sequence
  int32_t max_workers; // persistent kernels: worker bound the workspace was sized for
  size_t ws_o_bytes;
  size_t ws_bytes;
  // latent variant only: the generic kernel's plan, used for fp32 queries
  int32_t alt_split;
  int32_t alt_nsplit;
  size_t alt_ws_o_bytes;
  bool alt_unsupported;  // split_tokens exceeds what the generic kernel takes (fp32 queries fail)
};

size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

bool mfma_eligible(int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t P, int shared) {
  return !shared && Dk == 128 && Dv == 128 && P == 16 && Hq / Hkv <= 16;
}

// the shared-KV latent shape on the matrix cores (FP8 storage, bf16 queries; fp32 queries take the
// generic kernel, whose workspace the plan also covers)
bool latent_eligible(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t P, int kv_dt, int shared) {
  const int32_t G = Hq / Hkv;
  return shared && kv_dt == DAPF8_KV_FP8_E4M3 && Dk == 576 && Dv == 512 && P == 64 &&
         (G == 16 || G == 32 || G == 64 || G == 128) && B <= kSkMaxBatch;
}

// Partitioning of the fixed-partition kernels (matrix-core 128-dim or generic).  The generic kernel
// serves gb of a KV head's G query heads per workgroup, with gb x split scores in LDS.
int plan_fixed(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dv, int64_t max_len, int32_t split_tokens, bool mfma,
               const char* name, int32_t* split_out, int32_t* nsplit_out, size_t* ws_o_out, size_t* ws_out,
               int32_t* gb_out) {
  // The partition length comes first (it sizes the partial results); the generic kernel then takes
  // as many of a KV head's query heads per workgroup as its LDS score buffer holds.
  const int64_t G = Hq / Hkv;
  int64_t split = split_tokens;
  if (split == 0) {
    const int64_t units = (int64_t)B * (mfma ? Hkv : Hq);
    const int64_t target = mfma ? kTargetMfmaWG : kTargetGenericWG;
    const int64_t want = (max_len * (units > 0 ? units : 1) + target - 1) / target;
    split = (int64_t)round_up((size_t)(want > 0 ? want : 1), 256);
    split = split < 256 ? 256 : (split > 4096 ? 4096 : split);
    if (split >= max_len) split = (int64_t)round_up((size_t)max_len, 32);
  }
  if (!mfma && split > kGenericMaxSplit)
    return set_error(DAPF8_EUNSUPPORTED, "split_tokens > %d is not supported for this shape (variant %s)",
                     kGenericMaxSplit, name);
  const int64_t gb = mfma ? 1 : std::max<int64_t>(1, std::min<int64_t>({G, (int64_t)kGenMaxGB, kGenScoreFloats / split}));
  const int32_t nsplit = (int32_t)((max_len + split - 1) / split);
  *split_out = (int32_t)split;
  *nsplit_out = nsplit;
  *gb_out = (int32_t)gb;
  if (nsplit > 1) {
    *ws_o_out = round_up((size_t)B * Hq * nsplit * Dv * sizeof(float), 256);
    *ws_out = *ws_o_out + round_up((size_t)B * Hq * nsplit * 2 * sizeof(float), 256);
  } else {
    *ws_o_out = *ws_out = 0;
  }
  return DAPF8_OK;
}

int make_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t P, int32_t pt_stride,
              int32_t split_tokens, int kv_dt, int shared, Plan* p) {
  DAPF8_CHECK_ARG(B >= 0 && B <= 65535, "B must be in [0, 65535] (got %d)", B);
  DAPF8_CHECK_ARG(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 && Hq <= 65535,
                  "need Hkv >= 1, Hq a multiple of Hkv, Hq <= 65535 (got Hq=%d Hkv=%d)", Hq, Hkv);
  DAPF8_CHECK_ARG(Dk >= 64 && Dk <= 1024 && Dk % 64 == 0, "Dk must be a multiple of 64 in [64, 1024] (got %d)", Dk);
  DAPF8_CHECK_ARG(Dv >= 16 && Dv <= 1024 && Dv % 16 == 0, "Dv must be a multiple of 16 in [16, 1024] (got %d)", Dv);
  DAPF8_CHECK_ARG(!shared || Dv <= Dk, "shared-KV mode needs Dv <= Dk (got Dk=%d Dv=%d)", Dk, Dv);
  DAPF8_CHECK_ARG(P >= 1, "page_size must be >= 1 (got %d)", P);
  DAPF8_CHECK_ARG(pt_stride >= 1, "pt_stride must be >= 1 (got %d)", pt_stride);
  DAPF8_CHECK_ARG((int64_t)pt_stride * P <= (1 << 30), "pt_stride * page_size too large");
  DAPF8_CHECK_ARG(kv_dt == DAPF8_KV_FP8_E4M3 || kv_dt == DAPF8_KV_BF16, "unknown kv_dt %d", kv_dt);
  DAPF8_CHECK_ARG(split_tokens >= 0 && split_tokens % 32 == 0,
                  "split_tokens must be 0 or a positive multiple of 32 (got %d)", split_tokens);
  const int64_t max_len = (int64_t)pt_stride * P;
  const bool mfma = mfma_eligible(Hq, Hkv, Dk, Dv, P, shared);
  p->max_workers = 0;
  p->gb = p->alt_gb = 1;
  p->alt_split = p->alt_nsplit = 0;
  p->alt_ws_o_bytes = 0;
  p->alt_unsupported = false;
  if (latent_eligible(B, Hq, Hkv, Dk, Dv, P, kv_dt, shared)) {
    // The persistent kernel ignores split_tokens; only fp32 queries (generic kernel) use it, so a
    // split the generic kernel cannot take fails those calls alone (the workspace is sized for the
    // generic plan at its largest split).
    size_t alt_ws = 0;
    p->alt_unsupported = split_tokens > kGenericMaxSplit;
    int rc = plan_fixed(B, Hq, Hkv, Dv, max_len, p->alt_unsupported ? kGenericMaxSplit : split_tokens, false,
                        "valu_generic", &p->alt_split, &p->alt_nsplit, &p->alt_ws_o_bytes, &alt_ws, &p->alt_gb);
    if (rc != DAPF8_OK) return rc;
    p->variant = Variant::kMfmaLatent;
    p->name = "mfma_latent_d576_p64";
    // persistent kernel: its partial results are its workgroups' slices (whole pages), whatever
    // split_tokens asks for
    const int64_t split = (int64_t)round_up((size_t)max_len, 64);
    p->split = (int32_t)split;
    p->nsplit = (int32_t)((max_len + split - 1) / split);
    p->max_workers = kLatMaxWorkgroups;
    const size_t pieces = (size_t)B * Hkv * p->nsplit + (size_t)p->max_workers;
    p->ws_o_bytes = round_up(pieces * (size_t)(Hq / Hkv) * (Dv + 4) * sizeof(float), 256);
    p->ws_bytes = p->ws_o_bytes + round_up((size_t)2 * (B + 1) * sizeof(int), 256);
    if (alt_ws > p->ws_bytes) p->ws_bytes = alt_ws;
    return DAPF8_OK;
  }
  if (mfma && B <= kSkMaxBatch) {
    // stream-K: equal slices of all windows.  The partial results are the workers' slices (whole
    // 32-token windows), merged with the log-sum-exp rule, whatever split_tokens asks for: cutting
    // a slice at partition boundaries would only add partial results to write and merge.
    p->variant = Variant::kMfmaStreamK;
    p->name = "mfma_streamk_g16_d128_p16";
    const int64_t split = (int64_t)round_up((size_t)max_len, 32);
    p->split = (int32_t)split;
    p->nsplit = (int32_t)((max_len + split - 1) / split);
    p->max_workers = kSkMaxWorkers;
    const size_t pieces = (size_t)B * Hkv * p->nsplit + (size_t)p->max_workers;
    p->ws_o_bytes = round_up(pieces * (size_t)(Hq / Hkv) * (Dv + 4) * sizeof(float), 256);
    p->ws_bytes = p->ws_o_bytes + round_up((size_t)2 * (B + 1) * sizeof(int), 256);
    return DAPF8_OK;
  }
  p->variant = mfma ? Variant::kMfmaD128P16 : Variant::kGeneric;
  p->name = mfma ? "mfma_g16_d128_p16" : "valu_generic";
  return plan_fixed(B, Hq, Hkv, Dv, max_len, split_tokens, mfma, p->name, &p->split, &p->nsplit, &p->ws_o_bytes,
                    &p->ws_bytes, &p->gb);
}

}  // namespace

}  // namespace dapf8

using namespace dapf8;

extern "C" {

const char* dapf8_last_error(void) { return g_err; }

int dapf8_version(void) { return 100; }

int kv_absmax_update(const void* x, int x_dt, int64_t T, int32_t H, int32_t D, float* amax, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(T >= 0 && H >= 1 && H <= 65535 && D >= 4 && D % 4 == 0,
                  "kv_absmax_update: need T >= 0, 1 <= H <= 65535, D a positive multiple of 4");
  DAPF8_CHECK_ARG(x_dt == DAPF8_ACT_F32 || x_dt == DAPF8_ACT_BF16, "kv_absmax_update: unknown x_dt %d", x_dt);
  DAPF8_CHECK_ARG(amax && aligned16(amax), "kv_absmax_update: amax must be a 16-byte aligned device pointer");
  if (T == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(x && aligned16(x), "kv_absmax_update: x must be a 16-byte aligned device pointer");
  return launch_absmax(x, x_dt, T, H, D, amax, (hipStream_t)stream);
}

int kv_scale_from_absmax(const float* amax, int32_t H, float* scale, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(H >= 1, "kv_scale_from_absmax: H must be >= 1");
  DAPF8_CHECK_ARG(amax && scale && aligned16(amax) && aligned16(scale),
                  "kv_scale_from_absmax: amax and scale must be 16-byte aligned device pointers");
  return launch_scale_from_absmax(amax, H, scale, (hipStream_t)stream);
}

int kv_append(const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool, int kv_dt,
              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_ids, const int32_t* positions,
              int32_t T, const float* k_scale, const float* v_scale, const uint8_t* abort_mask, int32_t B,
              int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_pages, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(T >= 0, "kv_append: T must be >= 0");
  DAPF8_CHECK_ARG(in_dt == DAPF8_ACT_F32 || in_dt == DAPF8_ACT_BF16, "kv_append: unknown in_dt %d", in_dt);
  DAPF8_CHECK_ARG(kv_dt == DAPF8_KV_FP8_E4M3 || kv_dt == DAPF8_KV_BF16, "kv_append: unknown kv_dt %d", kv_dt);
  DAPF8_CHECK_ARG(B >= 1 && Hkv >= 1 && page_size >= 1 && num_pages >= 1 && pt_stride >= 1,
                  "kv_append: B, Hkv, page_size, num_pages and pt_stride must be >= 1");
  DAPF8_CHECK_ARG(Dk >= 64 && Dk % 64 == 0 && Dk <= 4096, "kv_append: Dk must be a multiple of 64 (got %d)", Dk);
  DAPF8_CHECK_ARG(!v_pool || (Dv >= 16 && Dv % 16 == 0 && Dv <= 4096),
                  "kv_append: Dv must be a multiple of 16 (got %d)", Dv);
  DAPF8_CHECK_ARG((int64_t)pt_stride * page_size <= (1 << 30), "kv_append: pt_stride * page_size too large");
  if (T == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(k_new && k_pool && page_table && seq_ids && positions,
                  "kv_append: k_new, k_pool, page_table, seq_ids and positions are required");
  DAPF8_CHECK_ARG(!v_pool || v_new, "kv_append: v_new is required when v_pool is given");
  DAPF8_CHECK_ARG(aligned16(k_new) && aligned16(v_new) && aligned16(k_pool) && aligned16(v_pool) &&
                      aligned16(page_table) && aligned16(seq_ids) && aligned16(positions) && aligned16(k_scale) &&
                      aligned16(v_scale) && aligned16(abort_mask),
                  "kv_append: every pointer must be 16-byte aligned");
  if (kv_dt == DAPF8_KV_FP8_E4M3)
    DAPF8_CHECK_ARG(k_scale && (!v_pool || v_scale), "kv_append: FP8 storage needs k_scale (and v_scale)");
  DAPF8_CHECK_ARG((int64_t)T * Hkv * (Dk / 16 + (v_pool ? Dv / 16 : 0)) < ((int64_t)1 << 40),
                  "kv_append: too many tokens in one call");
  return launch_append(k_new, v_new, in_dt, k_pool, v_pool, kv_dt, page_table, pt_stride, seq_ids, positions, T,
                       k_scale, v_scale, abort_mask, B, Hkv, Dk, Dv, page_size, num_pages, (hipStream_t)stream);
}

int kv_tag_verify(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                  const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                  int32_t B, int32_t page_size, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(B >= 0, "kv_tag_verify: B must be >= 0");
  DAPF8_CHECK_ARG(pt_stride >= 1 && page_size >= 1 && num_pages >= 1,
                  "kv_tag_verify: pt_stride, page_size and num_pages must be >= 1");
  if (B == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(page_table && expected_tags && seq_lens && live_tags && abort_mask,
                  "kv_tag_verify: all pointers are required");
  DAPF8_CHECK_ARG(aligned16(page_table) && aligned16(expected_tags) && aligned16(seq_lens) &&
                      aligned16(live_tags) && aligned16(abort_mask),
                  "kv_tag_verify: every pointer must be 16-byte aligned");
  return launch_verify(page_table, pt_stride, expected_tags, seq_lens, live_tags, num_pages, abort_mask, B,
                       page_size, (hipStream_t)stream);
}

int kv_tag_verify_append(const int32_t* page_table, int32_t pt_stride, const uint32_t* expected_tags,
                         const int32_t* seq_lens, const uint32_t* live_tags, int32_t num_pages, uint8_t* abort_mask,
                         const void* k_new, const void* v_new, int in_dt, void* k_pool, void* v_pool, int kv_dt,
                         const int32_t* seq_ids, const int32_t* positions, int32_t T, const float* k_scale,
                         const float* v_scale, int32_t B, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size,
                         void* stream) {
  clear_error();
  // the checks of kv_tag_verify and kv_append together; no requests and no tokens is a no-op
  DAPF8_CHECK_ARG(B >= 0 && T >= 0, "kv_tag_verify_append: need B >= 0 and T >= 0");
  if (B == 0 && T == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(B >= 1, "kv_tag_verify_append: tokens to append need B >= 1");
  DAPF8_CHECK_ARG(in_dt == DAPF8_ACT_F32 || in_dt == DAPF8_ACT_BF16, "kv_tag_verify_append: unknown in_dt %d", in_dt);
  DAPF8_CHECK_ARG(kv_dt == DAPF8_KV_FP8_E4M3 || kv_dt == DAPF8_KV_BF16, "kv_tag_verify_append: unknown kv_dt %d",
                  kv_dt);
  DAPF8_CHECK_ARG(Hkv >= 1 && page_size >= 1 && num_pages >= 1 && pt_stride >= 1,
                  "kv_tag_verify_append: Hkv, page_size, num_pages and pt_stride must be >= 1");
  DAPF8_CHECK_ARG(Dk >= 64 && Dk % 64 == 0 && Dk <= 4096, "kv_tag_verify_append: Dk must be a multiple of 64 (got %d)",
                  Dk);
  DAPF8_CHECK_ARG(!v_pool || (Dv >= 16 && Dv % 16 == 0 && Dv <= 4096),
                  "kv_tag_verify_append: Dv must be a multiple of 16 (got %d)", Dv);
  DAPF8_CHECK_ARG((int64_t)pt_stride * page_size <= (1 << 30), "kv_tag_verify_append: pt_stride * page_size too large");
  DAPF8_CHECK_ARG(page_table && expected_tags && seq_lens && live_tags && abort_mask && k_pool,
                  "kv_tag_verify_append: page_table, expected_tags, seq_lens, live_tags, abort_mask and k_pool are "
                  "required");
  DAPF8_CHECK_ARG(T == 0 || (k_new && seq_ids && positions && (!v_pool || v_new)),
                  "kv_tag_verify_append: k_new, seq_ids and positions (and v_new with v_pool) are required when T > 0");
  DAPF8_CHECK_ARG(aligned16(page_table) && aligned16(expected_tags) && aligned16(seq_lens) && aligned16(live_tags) &&
                      aligned16(abort_mask) && aligned16(k_new) && aligned16(v_new) && aligned16(k_pool) &&
                      aligned16(v_pool) && aligned16(seq_ids) && aligned16(positions) && aligned16(k_scale) &&
                      aligned16(v_scale),
                  "kv_tag_verify_append: every pointer must be 16-byte aligned");
  if (kv_dt == DAPF8_KV_FP8_E4M3 && T > 0)
    DAPF8_CHECK_ARG(k_scale && (!v_pool || v_scale), "kv_tag_verify_append: FP8 storage needs k_scale (and v_scale)");
  DAPF8_CHECK_ARG((int64_t)T * Hkv * (Dk / 16 + (v_pool ? Dv / 16 : 0)) < ((int64_t)1 << 31),
                  "kv_tag_verify_append: too many tokens in one call");
  return launch_verify_append(page_table, pt_stride, expected_tags, seq_lens, live_tags, num_pages, abort_mask, B,
                              page_size, k_new, v_new, in_dt, k_pool, v_pool, kv_dt, seq_ids, positions, T, k_scale,
                              v_scale, Hkv, Dk, Dv, (hipStream_t)stream);
}

int kv_transcode_pages(const void* k_src, const void* v_src, void* k_dst, void* v_dst, const int32_t* src_pages,
                       const int32_t* dst_pages, int32_t n_pages, const float* k_scale, const float* v_scale,
                       int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_src_pages,
                       int32_t num_dst_pages, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(n_pages >= 0, "kv_transcode_pages: n_pages must be >= 0");
  DAPF8_CHECK_ARG(Hkv >= 1 && page_size >= 1 && num_src_pages >= 1 && num_dst_pages >= 1,
                  "kv_transcode_pages: Hkv, page_size, num_src_pages and num_dst_pages must be >= 1");
  DAPF8_CHECK_ARG(Dk >= 64 && Dk % 64 == 0 && Dk <= 4096, "kv_transcode_pages: Dk must be a multiple of 64 (got %d)",
                  Dk);
  DAPF8_CHECK_ARG((v_src == nullptr) == (v_dst == nullptr),
                  "kv_transcode_pages: v_src and v_dst must both be given or both be NULL (shared-KV)");
  DAPF8_CHECK_ARG(!v_dst || (Dv >= 16 && Dv % 16 == 0 && Dv <= 4096),
                  "kv_transcode_pages: Dv must be a multiple of 16 (got %d)", Dv);
  DAPF8_CHECK_ARG((int64_t)Hkv * page_size * (Dk + (v_dst ? Dv : 0)) < ((int64_t)1 << 30),
                  "kv_transcode_pages: one page (Hkv * page_size * (Dk + Dv) values) is too large");
  if (n_pages == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(k_src && k_dst && src_pages && dst_pages && k_scale && (!v_dst || v_scale),
                  "kv_transcode_pages: k_src, k_dst, src_pages, dst_pages and the scales are required");
  DAPF8_CHECK_ARG(aligned16(k_src) && aligned16(v_src) && aligned16(k_dst) && aligned16(v_dst) &&
                      aligned16(src_pages) && aligned16(dst_pages) && aligned16(k_scale) && aligned16(v_scale),
                  "kv_transcode_pages: every pointer must be 16-byte aligned");
  return launch_transcode(k_src, v_src, k_dst, v_dst, src_pages, dst_pages, n_pages, k_scale, v_scale, Hkv, Dk, Dv,
                          page_size, num_src_pages, num_dst_pages, (hipStream_t)stream);
}

int kv_pages_init(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(num_pages >= 1, "kv_pages_init: num_pages must be >= 1");
  DAPF8_CHECK_ARG(free_list && free_count && aligned16(free_list) && aligned16(free_count) && aligned16(live_tags),
                  "kv_pages_init: free_list and free_count are required; every pointer must be 16-byte aligned");
  return launch_pages_init(free_list, free_count, live_tags, num_pages, (hipStream_t)stream);
}

int kv_pages_alloc(int32_t* free_list, int32_t* free_count, uint32_t* live_tags, int32_t num_pages,
                   const int32_t* counts, const int32_t* first_slot, int32_t B, int32_t* page_table,
                   uint32_t* expected_tags, int32_t pt_stride, uint8_t* granted, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(num_pages >= 1 && pt_stride >= 1, "kv_pages_alloc: num_pages and pt_stride must be >= 1");
  DAPF8_CHECK_ARG(B >= 0 && B <= kMaxAllocRequests, "kv_pages_alloc: B must be in [0, %d] (got %d)",
                  kMaxAllocRequests, B);
  DAPF8_CHECK_ARG(!expected_tags || live_tags, "kv_pages_alloc: expected_tags needs live_tags");
  if (B == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(free_list && free_count && counts && first_slot && page_table && granted,
                  "kv_pages_alloc: free_list, free_count, counts, first_slot, page_table and granted are required");
  DAPF8_CHECK_ARG(aligned16(free_list) && aligned16(free_count) && aligned16(live_tags) && aligned16(counts) &&
                      aligned16(first_slot) && aligned16(page_table) && aligned16(expected_tags) &&
                      aligned16(granted),
                  "kv_pages_alloc: every pointer must be 16-byte aligned");
  return launch_pages_alloc(free_list, free_count, live_tags, num_pages, counts, first_slot, B, page_table,
                            expected_tags, pt_stride, granted, (hipStream_t)stream);
}

int kv_pages_free(int32_t* free_list, int32_t* free_count, const int32_t* pages, int32_t n, int32_t num_pages,
                  int32_t* status, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(num_pages >= 1 && n >= 0, "kv_pages_free: need num_pages >= 1 and n >= 0");
  DAPF8_CHECK_ARG(free_list && free_count && status && (n == 0 || pages),
                  "kv_pages_free: free_list, free_count, status and pages are required");
  DAPF8_CHECK_ARG(aligned16(free_list) && aligned16(free_count) && aligned16(pages) && aligned16(status),
                  "kv_pages_free: every pointer must be 16-byte aligned");
  return launch_pages_free(free_list, free_count, pages, n, num_pages, status, (hipStream_t)stream);
}

int w4_pack(const int8_t* q, const float* scales, int32_t N, int32_t K, uint8_t* packed, float* packed_scales,
            void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(N >= 64 && N % 64 == 0 && K >= 128 && K % 128 == 0,
                  "w4_pack: N must be a positive multiple of 64 and K a positive multiple of 128 (got %d, %d)", N, K);
  DAPF8_CHECK_ARG((int64_t)N * K / 8 < ((int64_t)1 << 31), "w4_pack: matrix too large");
  DAPF8_CHECK_ARG(q && scales && packed && packed_scales && aligned16(q) && aligned16(scales) && aligned16(packed) &&
                      aligned16(packed_scales),
                  "w4_pack: all pointers are required and must be 16-byte aligned");
  return launch_w4_pack(q, scales, N, K, packed, packed_scales, (hipStream_t)stream);
}

int w4a16_gemv(const void* x, const uint8_t* packed, const float* packed_scales, void* y, int out_dt, int32_t M,
               int32_t N, int32_t K, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(M >= 0 && M <= 16, "w4a16_gemv: M must be in [0, 16] (got %d)", M);
  DAPF8_CHECK_ARG(N >= 64 && N % 64 == 0 && K >= 128 && K % 128 == 0,
                  "w4a16_gemv: N must be a positive multiple of 64 and K a positive multiple of 128 (got %d, %d)", N,
                  K);
  DAPF8_CHECK_ARG((int64_t)N * K / 8 < ((int64_t)1 << 31), "w4a16_gemv: matrix too large");
  DAPF8_CHECK_ARG(out_dt == DAPF8_ACT_F32 || out_dt == DAPF8_ACT_BF16, "w4a16_gemv: unknown out_dt %d", out_dt);
  if (M == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(x && packed && packed_scales && y && aligned16(x) && aligned16(packed) && aligned16(packed_scales) &&
                      aligned16(y),
                  "w4a16_gemv: all pointers are required and must be 16-byte aligned");
  return launch_w4_gemv(x, packed, packed_scales, y, out_dt, M, N, K, (hipStream_t)stream);
}

int hbm_read_probe(const void* buf, const int32_t* block_ids, int64_t n_blocks, int32_t block_bytes, uint32_t* sink,
                   int32_t workgroups, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(n_blocks >= 0 && block_bytes >= 1024 && block_bytes % 1024 == 0,
                  "hbm_read_probe: need n_blocks >= 0 and block_bytes a positive multiple of 1024");
  DAPF8_CHECK_ARG(workgroups >= 1 && workgroups <= 65535, "hbm_read_probe: workgroups must be in [1, 65535]");
  DAPF8_CHECK_ARG(buf && sink && aligned16(buf) && aligned16(sink) && aligned16(block_ids),
                  "hbm_read_probe: buf and sink are required; every pointer must be 16-byte aligned");
  return launch_read_probe(buf, block_ids, n_blocks, block_bytes, sink, workgroups, (hipStream_t)stream);
}

int hbm_copy_probe(const void* src, void* dst, int64_t dst_bytes, int32_t workgroups, void* stream) {
  clear_error();
  DAPF8_CHECK_ARG(dst_bytes >= 0 && dst_bytes % 16 == 0, "hbm_copy_probe: dst_bytes must be a multiple of 16");
  DAPF8_CHECK_ARG(workgroups >= 1 && workgroups <= 65535, "hbm_copy_probe: workgroups must be in [1, 65535]");
  if (dst_bytes == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(src && dst && aligned16(src) && aligned16(dst),
                  "hbm_copy_probe: src and dst are required and must be 16-byte aligned");
  return launch_copy_probe(src, dst, dst_bytes, workgroups, (hipStream_t)stream);
}

size_t paged_decode_attn_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                        int32_t page_size, int32_t pt_stride, int32_t split_tokens, int kv_dt,
                                        int shared_kv) {
  Plan p;
  if (make_plan(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens, kv_dt, shared_kv, &p) != DAPF8_OK) return 0;
  return p.ws_bytes;
}

const char* paged_decode_attn_variant(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                                      int32_t page_size, int32_t pt_stride, int32_t split_tokens, int kv_dt,
                                      int shared_kv, int32_t* split_out) {
  clear_error();
  Plan p;
  if (make_plan(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens, kv_dt, shared_kv, &p) != DAPF8_OK)
    return "invalid";
  if (split_out) *split_out = p.split;
  return p.name;
}

}  // extern "C"

namespace dapf8 {
namespace {

// paged_decode_attn after argument checks; workspace == kUseScratch selects the library's own scratch array
void* const kUseScratch = reinterpret_cast<void*>(uintptr_t(1));
int scratch_for_current_device(void** ptr);

int attn_call(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt, const int32_t* page_table,
              int32_t pt_stride, const int32_t* seq_lens, const float* k_scale, const float* v_scale,
              const uint8_t* abort_mask, void* out, int out_dt, float sm_scale, int32_t B, int32_t Hq, int32_t Hkv,
              int32_t Dk, int32_t Dv, int32_t page_size, int32_t num_pages, int32_t split_tokens, void* workspace,
              size_t workspace_bytes, void* stream) {
  const int shared = v_pool == nullptr;
  Plan p;
  int rc = make_plan(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens, kv_dt, shared, &p);
  if (rc != DAPF8_OK) return rc;
  DAPF8_CHECK_ARG(q_dt == DAPF8_ACT_F32 || q_dt == DAPF8_ACT_BF16, "paged_decode_attn: unknown q_dt %d", q_dt);
  DAPF8_CHECK_ARG(out_dt == DAPF8_ACT_F32 || out_dt == DAPF8_ACT_BF16, "paged_decode_attn: unknown out_dt %d",
                  out_dt);
  DAPF8_CHECK_ARG(num_pages >= 1, "paged_decode_attn: num_pages must be >= 1");
  DAPF8_CHECK_ARG((int64_t)num_pages * Hkv <= INT32_MAX,
                  "paged_decode_attn: num_pages * Hkv must fit in 32 bits (got %d * %d)", num_pages, Hkv);
  DAPF8_CHECK_ARG(std::isfinite(sm_scale), "paged_decode_attn: sm_scale must be finite");
  if (B == 0) return DAPF8_OK;
  DAPF8_CHECK_ARG(q && k_pool && page_table && seq_lens && out,
                  "paged_decode_attn: q, k_pool, page_table, seq_lens and out are required");
  if (kv_dt == DAPF8_KV_FP8_E4M3)
    DAPF8_CHECK_ARG(k_scale && (shared || v_scale), "paged_decode_attn: FP8 storage needs k_scale (and v_scale)");
  const bool own = workspace == kUseScratch;
  DAPF8_CHECK_ARG(aligned16(q) && aligned16(k_pool) && aligned16(v_pool) && aligned16(page_table) &&
                      aligned16(seq_lens) && aligned16(k_scale) && aligned16(v_scale) && aligned16(abort_mask) &&
                      aligned16(out) && (own || aligned16(workspace)),
                  "paged_decode_attn: every pointer must be 16-byte aligned");
  if (own) {
    if (p.ws_bytes > kScratchBytes)
      return set_error(DAPF8_EWORKSPACE,
                       "paged_decode_attn_noalloc: this shape needs %zu bytes of scratch; the library holds %zu "
                       "(use paged_decode_attn with a workspace)", p.ws_bytes, kScratchBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (p.ws_bytes > 0) {
      rc = scratch_for_current_device(&workspace);
      if (rc != DAPF8_OK) return rc;
      workspace_bytes = kScratchBytes;
    }
  }
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes))
    return set_error(DAPF8_EWORKSPACE, "paged_decode_attn: workspace of %zu bytes needed, %zu given", p.ws_bytes,
                     workspace ? workspace_bytes : (size_t)0);
  AttnArgs a;
  a.q = q;
  a.q_dt = q_dt;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.kv_dt = kv_dt;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.abort_mask = abort_mask;
  a.out = out;
  a.out_dt = out_dt;
  a.sm_scale = sm_scale;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Dk = Dk;
  a.Dv = Dv;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.split = p.split;
  a.nsplit = p.nsplit;
  a.gb = p.gb;
  a.ws_o = p.ws_bytes ? (float*)workspace : nullptr;
  a.ws_ml = p.ws_bytes ? (float*)((char*)workspace + p.ws_o_bytes) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (p.variant == Variant::kMfmaStreamK) return launch_attn_sk(a, p.max_workers, s);
  if (p.variant == Variant::kMfmaLatent) {
    if (q_dt == DAPF8_ACT_BF16) return launch_attn_latent(a, p.max_workers, s);
    // fp32 queries: the generic kernel with its own partitioning (the workspace covers both)
    if (p.alt_unsupported)
      return set_error(DAPF8_EUNSUPPORTED,
                       "paged_decode_attn: fp32 queries on this shape run the generic kernel, which takes "
                       "split_tokens <= %d (got %d)", kGenericMaxSplit, split_tokens);
    p.variant = Variant::kGeneric;
    a.split = p.alt_split;
    a.nsplit = p.alt_nsplit;
    a.gb = p.alt_gb;
    a.ws_o = p.alt_nsplit > 1 ? (float*)workspace : nullptr;
    a.ws_ml = p.alt_nsplit > 1 ? (float*)((char*)workspace + p.alt_ws_o_bytes) : nullptr;
    p.nsplit = p.alt_nsplit;
  }
  rc = p.variant == Variant::kMfmaD128P16 ? launch_attn_mfma(a, s) : launch_attn_generic(a, s);
  if (rc != DAPF8_OK) return rc;
  if (p.nsplit > 1) rc = launch_merge(a, s);
  return rc;
}

}  // namespace

// The no-allocation entry point's scratch: a file-scope device array, which each GPU holds once the
// library's code is loaded on it (until the process ends).  Host code never uses the array's name as
// an address (on the host it is only a stand-in); it takes each device's address of it once, with
// that device current, and passes that address to the kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(DAPF8_ELAUNCH, "paged_decode_attn_noalloc: no usable current device (%d)", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return set_error(DAPF8_ELAUNCH, "paged_decode_attn_noalloc: hipGetSymbolAddress of the scratch array "
                                        "failed on device %d: %s", dev, hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return DAPF8_OK;
}

}  // namespace
}  // namespace dapf8

extern "C" {

int paged_decode_attn(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                      const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens, const float* k_scale,
                      const float* v_scale, const uint8_t* abort_mask, void* out, int out_dt, float sm_scale,
                      int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size,
                      int32_t num_pages, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                      void* stream) {
  clear_error();
  if (workspace == kUseScratch) return set_error(DAPF8_EINVAL, "paged_decode_attn: invalid workspace pointer");
  return attn_call(q, q_dt, k_pool, v_pool, kv_dt, page_table, pt_stride, seq_lens, k_scale, v_scale, abort_mask,
                   out, out_dt, sm_scale, B, Hq, Hkv, Dk, Dv, page_size, num_pages, split_tokens, workspace,
                   workspace_bytes, stream);
}

int paged_decode_attn_noalloc(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                              const float* k_scale, const float* v_scale, const uint8_t* abort_mask, void* out,
                              int out_dt, float sm_scale, int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv,
                              int32_t page_size, int32_t num_pages, int32_t split_tokens, void* stream) {
  clear_error();
  return attn_call(q, q_dt, k_pool, v_pool, kv_dt, page_table, pt_stride, seq_lens, k_scale, v_scale, abort_mask,
                   out, out_dt, sm_scale, B, Hq, Hkv, Dk, Dv, page_size, num_pages, split_tokens, kUseScratch, 0,
                   stream);
}

int paged_decode_attn_checked(const void* q, int q_dt, const void* k_pool, const void* v_pool, int kv_dt,
                              const int32_t* page_table, int32_t pt_stride, const int32_t* seq_lens,
                              const uint32_t* expected_tags, const uint32_t* live_tags, const float* k_scale,
                              const float* v_scale, uint8_t* abort_mask_out, void* out, int out_dt, float sm_scale,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t page_size,
                              int32_t num_pages, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const int shared = v_pool == nullptr;
  Plan p;
  int rc = make_plan(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, 0, kv_dt, shared, &p);
  if (rc != DAPF8_OK) return rc;
  if (B == 0) return DAPF8_OK;
  if (p.variant != Variant::kMfmaStreamK)
    return set_error(DAPF8_EUNSUPPORTED,
                     "paged_decode_attn_checked: only the persistent matrix-core shape (Dk = Dv = 128, page 16, "
                     "Hq/Hkv <= 16, separate V) is supported (this shape uses %s)", p.name);
  DAPF8_CHECK_ARG(q_dt == DAPF8_ACT_BF16, "paged_decode_attn_checked: bf16 queries only");
  DAPF8_CHECK_ARG(out_dt == DAPF8_ACT_F32 || out_dt == DAPF8_ACT_BF16, "paged_decode_attn_checked: unknown out_dt %d",
                  out_dt);
  DAPF8_CHECK_ARG(num_pages >= 1 && (int64_t)num_pages * Hkv <= INT32_MAX,
                  "paged_decode_attn_checked: need num_pages >= 1 and num_pages * Hkv < 2^31");
  DAPF8_CHECK_ARG(std::isfinite(sm_scale), "paged_decode_attn_checked: sm_scale must be finite");
  DAPF8_CHECK_ARG(q && k_pool && page_table && seq_lens && expected_tags && live_tags && abort_mask_out && out,
                  "paged_decode_attn_checked: q, k_pool, page_table, seq_lens, the tags, abort_mask_out and out "
                  "are required");
  if (kv_dt == DAPF8_KV_FP8_E4M3)
    DAPF8_CHECK_ARG(k_scale && v_scale, "paged_decode_attn_checked: FP8 storage needs k_scale and v_scale");
  DAPF8_CHECK_ARG(aligned16(q) && aligned16(k_pool) && aligned16(v_pool) && aligned16(page_table) &&
                      aligned16(seq_lens) && aligned16(expected_tags) && aligned16(live_tags) &&
                      aligned16(k_scale) && aligned16(v_scale) && aligned16(abort_mask_out) && aligned16(out) &&
                      aligned16(workspace),
                  "paged_decode_attn_checked: every pointer must be 16-byte aligned");
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes))
    return set_error(DAPF8_EWORKSPACE, "paged_decode_attn_checked: workspace of %zu bytes needed, %zu given",
                     p.ws_bytes, workspace ? workspace_bytes : (size_t)0);
  AttnArgs a;
  a.q = q;
  a.q_dt = q_dt;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.kv_dt = kv_dt;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.seq_lens = seq_lens;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.abort_mask = nullptr;
  a.out = out;
  a.out_dt = out_dt;
  a.sm_scale = sm_scale;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Dk = Dk;
  a.Dv = Dv;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.split = p.split;
  a.nsplit = p.nsplit;
  a.ws_o = (float*)workspace;
  a.ws_ml = (float*)((char*)workspace + p.ws_o_bytes);
  a.live_tags = live_tags;
  a.expected_tags = expected_tags;
  a.abort_out = abort_mask_out;
  return launch_attn_sk(a, p.max_workers, (hipStream_t)stream);
}

}  // extern "C"
