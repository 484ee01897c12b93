// C ABI of the MTLA hot path: argument validation, workspace sizing and
// kernel dispatch.  Every check runs before anything is enqueued; no HIP API
// is called on a failed check.
#include <algorithm>
#include <climits>
#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mtla.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int32_t ok() {
  g_err[0] = '\0';
  return MTLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int kMaxS = 256;
constexpr int kMaxWidth = 1024;
constexpr int kMaxDh = 256;
constexpr int64_t kMaxElems = int64_t(1) << 40;

// Element stride between W_hyp rows: 0 when every token takes the one row,
// d_c when W_hyp has one row per place in the block.
int gate_stride(const mtla_dims* d) { return (d->flags & MTLA_FLAG_GATE_PER_POSITION) ? d->d_c : 0; }
int gate_rows(const mtla_dims* d) { return (d->flags & MTLA_FLAG_GATE_PER_POSITION) ? d->stride_s : 1; }

int32_t check_dims(const mtla_dims* d) {
  if (!d) return fail(MTLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 0) return fail(MTLA_ERR_INVALID_ARG, "batch=%d < 0", d->batch);
  if (d->heads < 1) return fail(MTLA_ERR_INVALID_ARG, "heads=%d < 1", d->heads);
  if (d->d_h < 1) return fail(MTLA_ERR_INVALID_ARG, "d_h=%d < 1", d->d_h);
  if (d->d_c < 1) return fail(MTLA_ERR_INVALID_ARG, "d_c=%d < 1", d->d_c);
  if (d->d_r < 0) return fail(MTLA_ERR_INVALID_ARG, "d_r=%d < 0", d->d_r);
  if (d->stride_s < 1) return fail(MTLA_ERR_INVALID_ARG, "stride_s=%d < 1", d->stride_s);
  if (d->max_slots < 1) return fail(MTLA_ERR_INVALID_ARG, "max_slots=%d < 1", d->max_slots);
  if (d->dtype != MTLA_FP32 && d->dtype != MTLA_BF16)
    return fail(MTLA_ERR_INVALID_ARG, "dtype=%d is neither MTLA_FP32 nor MTLA_BF16", d->dtype);
  if (!(isfinite(d->softmax_scale) && d->softmax_scale > 0.f))
    return fail(MTLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (d->flags & ~(MTLA_FLAG_PORTABLE | MTLA_FLAG_GATE_PER_POSITION))
    return fail(MTLA_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
  if (d->decode_splits < 0 || d->decode_splits > 64)
    return fail(MTLA_ERR_INVALID_ARG, "decode_splits=%d is outside 0..64", d->decode_splits);
  if (d->step_groups < 0) return fail(MTLA_ERR_INVALID_ARG, "step_groups=%d < 0", d->step_groups);
  if (d->stride_s > kMaxS) return fail(MTLA_ERR_UNSUPPORTED, "stride_s=%d > %d", d->stride_s, kMaxS);
  if (d->d_c + d->d_r > kMaxWidth)
    return fail(MTLA_ERR_UNSUPPORTED, "d_c + d_r = %d > %d", d->d_c + d->d_r, kMaxWidth);
  if (d->d_h > kMaxDh) return fail(MTLA_ERR_UNSUPPORTED, "d_h=%d > %d", d->d_h, kMaxDh);
  if (d->d_c % 8 != 0 || d->d_r % 8 != 0)
    return fail(MTLA_ERR_UNSUPPORTED, "d_c=%d and d_r=%d must be multiples of 8", d->d_c, d->d_r);
  if ((8 * int64_t(d->d_c) + int64_t(d->d_h) * 65) * 4 > 65536)
    return fail(MTLA_ERR_UNSUPPORTED, "d_c=%d with d_h=%d exceeds the up-projection kernel's LDS", d->d_c, d->d_h);
  const int64_t W = d->d_c + d->d_r;
  // one sequence's rows are addressed through a buffer resource whose size
  // is a 32-bit byte count
  if (int64_t(d->max_slots) * W * 4 > INT32_MAX)
    return fail(MTLA_ERR_UNSUPPORTED, "max_slots=%d rows of %lld elements exceed 2^31 bytes per sequence",
                d->max_slots, static_cast<long long>(W));
  if (int64_t(d->batch) * d->max_slots * W > kMaxElems)
    return fail(MTLA_ERR_UNSUPPORTED, "cache of %lld elements is too large",
                static_cast<long long>(int64_t(d->batch) * d->max_slots * W));
  return MTLA_OK;
}

#define CHECK_PTR(p)                                                                   \
  do {                                                                                 \
    if (!(p)) return fail(MTLA_ERR_INVALID_ARG, "%s is NULL", #p);                     \
    if (!aligned16(p)) return fail(MTLA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

// Pointers only read or written element by element need their element
// alignment; tensors that kernels move in 16-byte vectors need 16 bytes.
#define CHECK_PTR_ALIGN(p, n)                                                          \
  do {                                                                                 \
    if (!(p)) return fail(MTLA_ERR_INVALID_ARG, "%s is NULL", #p);                     \
    if (!aligned_to(p, n)) return fail(MTLA_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, n); \
  } while (0)

#define CHECK_OPT_PTR_ALIGN(p, n)                                                      \
  do {                                                                                 \
    if ((p) && !aligned_to(p, n))                                                      \
      return fail(MTLA_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, n);           \
  } while (0)

int32_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MTLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t elem_bytes(const mtla_dims* d) { return d->dtype == MTLA_FP32 ? 4 : 2; }

bool decode_fast(const mtla_dims* d) {
  return d->dtype == MTLA_BF16 && !(d->flags & MTLA_FLAG_PORTABLE) &&
         mtla::decode_mfma_supported(d->heads, d->d_c, d->d_r);
}

bool prefill_fast(const mtla_dims* d) {
  return d->dtype == MTLA_BF16 && !(d->flags & MTLA_FLAG_PORTABLE) &&
         mtla::prefill_mfma_supported(d->heads, d->d_h, d->d_c, d->d_r);
}

int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }
int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Splits of the slot range.  The MFMA kernel gives each split at least ~512
// slots (a short cache is one workgroup per sequence, with no merge pass) and
// otherwise aims at one workgroup per CU over the chip's 256 CUs; the
// portable kernel gives each split ~128 slots.  A nonzero dims->decode_splits
// replaces the default, within the same limits.
int decode_splits(const mtla_dims* d) {
  if (decode_fast(d)) {
    const int cap = clampi(ceil_div(d->max_slots, 512), 1, 64);
    if (d->decode_splits > 0) return clampi(d->decode_splits, 1, cap);
    // one workgroup per compute unit: the split kernel's registers allow one
    // 256-thread workgroup per CU, so a second round of workgroups would run
    // on a quarter-full chip
    const int want = ceil_div(256, d->batch > 0 ? d->batch : 1);
    return clampi(want, 1, cap);
  }
  const int cap = clampi(ceil_div(d->max_slots, 128), 1, 32);
  return d->decode_splits > 0 ? clampi(d->decode_splits, 1, cap) : cap;
}

// One workgroup per sequence runs the whole step (merge, absorb, attention,
// up-projection) when the cache needs a single split and the weights are small.
bool decode_fused(const mtla_dims* d) {
  return decode_fast(d) && decode_splits(d) == 1 &&
         mtla::decode_step_supported(d->heads, d->d_h, d->d_c, d->d_r);
}

int prefill_splits(const mtla_dims* d, int n_tokens) {
  return clampi(ceil_div(n_tokens / d->stride_s + 1, 128), 1, 16);
}

// Workspace of the latent attention: the split partials.
struct AttnWs {
  size_t pm, pl, pacc, total;
};

AttnWs attn_ws(const mtla_dims* d, size_t rows, int splits, size_t off) {
  const size_t H = d->heads, S = splits;
  AttnWs w;
  w.pm = off;
  w.pl = w.pm + align_up(rows * S * H * 4);
  w.pacc = w.pl + align_up(rows * S * H * 4);
  w.total = w.pacc + align_up(rows * S * H * d->d_c * 4);
  return w;
}

struct DecodeWs {
  size_t qlat, olat;
  AttnWs attn;
  size_t total;
};

DecodeWs decode_ws(const mtla_dims* d) {
  const size_t B = d->batch, H = d->heads, W = d->d_c + d->d_r;
  DecodeWs w;
  w.qlat = 0;
  w.olat = w.qlat + align_up(B * H * W * 4);
  w.attn = attn_ws(d, B, decode_splits(d), w.olat + align_up(B * H * d->d_c * 4));
  w.total = w.attn.total;
  return w;
}

struct PrefillWs {
  size_t P, kc, v, qlat, olat;
  AttnWs attn;
  size_t total;
};

// Completed slots that some query of tokens t0+1 .. t0+n attends: query
// token i sees slots 1 .. ceil(i/s) - 1.
int prefill_slot_keys(const mtla_dims* d, int n, int t0) { return n > 0 ? (t0 + n - 1) / d->stride_s : 0; }

// Workspace of a prefill of n tokens after t0 cached ones.  The MFMA path
// holds K^C and V of the completed slots the queries attend ([B, H, slots,
// d_h] each); each query's own diagonal key is formed in the attention kernel.
PrefillWs prefill_ws(const mtla_dims* d, int n, int t0 = 0) {
  const size_t B = d->batch, H = d->heads, W = d->d_c + d->d_r, N = n;
  const size_t e = elem_bytes(d);
  PrefillWs w{};
  w.P = 0;
  size_t off = align_up(B * N * W * e);
  if (prefill_fast(d)) {
    const size_t S = prefill_slot_keys(d, n, t0);
    w.kc = off;
    off += align_up(B * H * S * d->d_h * e);
    w.v = off;
    off += align_up(B * H * S * d->d_h * e);
    w.total = off;
  } else {
    const size_t R = B * N;
    w.qlat = off;
    off += align_up(R * H * W * 4);
    w.olat = off;
    off += align_up(R * H * d->d_c * 4);
    w.attn = attn_ws(d, R, prefill_splits(d, t0 + n), off);
    w.total = w.attn.total;
  }
  return w;
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

}  // namespace

extern "C" {

int32_t mtla_version(void) { return 10100; }

const char* mtla_status_string(int32_t s) {
  switch (s) {
    case MTLA_OK: return "MTLA_OK";
    case MTLA_ERR_INVALID_ARG: return "MTLA_ERR_INVALID_ARG";
    case MTLA_ERR_UNSUPPORTED: return "MTLA_ERR_UNSUPPORTED";
    case MTLA_ERR_WORKSPACE: return "MTLA_ERR_WORKSPACE";
    case MTLA_ERR_HIP: return "MTLA_ERR_HIP";
    default: return "MTLA_UNKNOWN_STATUS";
  }
}

const char* mtla_last_error(void) { return g_err; }

int32_t mtla_sinusoidal_pe(int32_t rows, int32_t d, float* pe, void* stream) {
  if (rows < 1 || d < 1) return fail(MTLA_ERR_INVALID_ARG, "rows=%d, d=%d must be >= 1", rows, d);
  if (int64_t(rows) * d > kMaxElems) return fail(MTLA_ERR_UNSUPPORTED, "table too large");
  CHECK_PTR_ALIGN(pe, 4);
  return hip_status(mtla::launch_sinusoidal_pe(rows, d, pe, static_cast<hipStream_t>(stream)),
                    "sinusoidal_pe launch");
}

int32_t mtla_merge_append(const mtla_dims* dims, const int32_t* pos0, int32_t n_tokens,
                          const void* c, const void* k_r, const float* w_hyp, const float* pe,
                          int32_t pe_rows, void* cache, float* open_acc, float* gate_out,
                          void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if (pe_rows < 1) return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < 1", pe_rows);
  if (n_tokens > pe_rows)
    return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d exceeds pe_rows=%d", n_tokens, pe_rows);
  if (int64_t(n_tokens) > int64_t(dims->max_slots) * dims->stride_s)
    return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d exceeds the cache capacity s*max_slots", n_tokens);
  if (dims->batch == 0 || n_tokens == 0) return ok();
  CHECK_PTR_ALIGN(pos0, 4);
  CHECK_PTR(c);
  if (dims->d_r > 0) CHECK_PTR(k_r);
  CHECK_PTR_ALIGN(w_hyp, 4);
  CHECK_PTR_ALIGN(pe, 4);
  CHECK_PTR(cache);
  CHECK_PTR(open_acc);
  CHECK_OPT_PTR_ALIGN(gate_out, 4);
  mtla::MergeArgs a{dims->batch, n_tokens, dims->d_c, dims->d_r, dims->stride_s, dims->max_slots,
                    pe_rows, pos0, c, k_r, w_hyp, pe, cache, open_acc, gate_out, nullptr};
  a.wh_stride = gate_stride(dims);
  return hip_status(mtla::launch_merge(a, dims->dtype, static_cast<hipStream_t>(stream)),
                    "merge launch");
}

int32_t mtla_reorder_state(const mtla_dims* dims, const int32_t* src, const int32_t* pos,
                           const void* cache_in, const float* open_in, void* cache_out, float* open_out,
                           int32_t* pos_out, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (dims->batch == 0) return ok();
  CHECK_PTR_ALIGN(src, 4);
  CHECK_PTR_ALIGN(pos, 4);
  CHECK_PTR(cache_in);
  CHECK_PTR(cache_out);
  CHECK_PTR_ALIGN(open_in, 4);
  CHECK_PTR_ALIGN(open_out, 4);
  CHECK_OPT_PTR_ALIGN(pos_out, 4);
  if (cache_in == cache_out || open_in == open_out || (pos_out && pos_out == pos))
    return fail(MTLA_ERR_INVALID_ARG, "the reorder is out of place: outputs must not be the inputs");
  const int W = dims->d_c + dims->d_r;
  const int row_bytes = W * static_cast<int>(elem_bytes(dims));
  mtla::ReorderArgs a{dims->batch, dims->stride_s, dims->max_slots, row_bytes, 2 * W, src, pos,
                      cache_in, cache_out, open_in, open_out, pos_out};
  return hip_status(mtla::launch_reorder(a, static_cast<hipStream_t>(stream)), "reorder launch");
}

int32_t mtla_absorb_query(const mtla_dims* dims, int32_t n_rows, const void* q_c, const void* q_r,
                          const void* w_uk, float* q_lat, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (n_rows < 0) return fail(MTLA_ERR_INVALID_ARG, "n_rows=%d < 0", n_rows);
  if (n_rows == 0) return ok();
  CHECK_PTR(q_c);
  if (dims->d_r > 0) CHECK_PTR(q_r);
  CHECK_PTR(w_uk);
  CHECK_PTR_ALIGN(q_lat, 4);
  return hip_status(mtla::launch_absorb(n_rows, dims->heads, dims->d_h, dims->d_c, dims->d_r, q_c,
                                        q_r, w_uk, q_lat, dims->dtype,
                                        static_cast<hipStream_t>(stream)),
                    "absorb launch");
}

int32_t mtla_up_project(const mtla_dims* dims, int32_t n_rows, const float* o_lat,
                        const void* w_uv, void* out, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (n_rows < 0) return fail(MTLA_ERR_INVALID_ARG, "n_rows=%d < 0", n_rows);
  if (n_rows == 0) return ok();
  CHECK_PTR_ALIGN(o_lat, 4);
  CHECK_PTR(w_uv);
  CHECK_PTR(out);
  return hip_status(mtla::launch_up_project(n_rows, dims->heads, dims->d_h, dims->d_c, o_lat, w_uv,
                                            out, dims->dtype, static_cast<hipStream_t>(stream)),
                    "up-projection launch");
}

int32_t mtla_decode_plan(const mtla_dims* dims, int32_t* splits, int32_t* fused) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (!splits || !fused) return fail(MTLA_ERR_INVALID_ARG, "splits and fused must be non-NULL");
  *splits = decode_splits(dims);
  *fused = decode_fused(dims) ? 1 : 0;
  return ok();
}

int32_t mtla_decode_attention_workspace_bytes(const mtla_dims* dims, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = attn_ws(dims, dims->batch, decode_splits(dims), 0).total;
  return ok();
}

namespace {

mtla::Partials attn_partials(void* ws, const AttnWs& w) {
  return mtla::Partials{reinterpret_cast<float*>(at(ws, w.pm)), reinterpret_cast<float*>(at(ws, w.pl)),
                        reinterpret_cast<float*>(at(ws, w.pacc))};
}

// Latent attention into o_lat; with merge_splits false (MFMA path, several
// splits) the split partials are left in the workspace for the caller.
hipError_t run_decode_attention(const mtla_dims* dims, const int32_t* pos, const float* q_lat,
                                const void* cache, float* o_lat, void* ws, const AttnWs& w,
                                hipStream_t s, bool merge_splits = true) {
  const int splits = decode_splits(dims);
  mtla::AttendArgs a{dims->batch, 0, dims->heads, dims->d_c, dims->d_r, dims->stride_s,
                     dims->max_slots, splits, dims->softmax_scale, pos, q_lat, cache, nullptr,
                     attn_partials(ws, w), o_lat};
  return decode_fast(dims) ? mtla::launch_decode_mfma(a, s, merge_splits)
                           : mtla::launch_attend_portable(a, dims->dtype, s);
}

}  // namespace

int32_t mtla_decode_attention(const mtla_dims* dims, const int32_t* pos, const float* q_lat,
                              const void* cache, float* o_lat, void* workspace, size_t ws_bytes,
                              void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (dims->batch == 0) return ok();
  CHECK_PTR_ALIGN(pos, 4);
  CHECK_PTR_ALIGN(q_lat, 4);
  CHECK_PTR(cache);
  CHECK_PTR_ALIGN(o_lat, 4);
  const AttnWs w = attn_ws(dims, dims->batch, decode_splits(dims), 0);
  if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", w.total);
  if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < w.total)
    return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, w.total);
  return hip_status(run_decode_attention(dims, pos, q_lat, cache, o_lat, workspace, w,
                                         static_cast<hipStream_t>(stream)),
                    "decode attention launch");
}

int32_t mtla_decode_workspace_bytes(const mtla_dims* dims, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = decode_ws(dims).total;
  return ok();
}

namespace {

mtla::StepArgs step_args(const mtla_dims* d, const int32_t* pos, const void* c, const void* k_r,
                         const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                         const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                         float* open_acc, void* out, int merge) {
  return mtla::StepArgs{d->batch, d->heads, d->d_h, d->d_c, d->d_r, d->stride_s, d->max_slots,
                        pe_rows, merge, /*groups requested (0: the launcher chooses)*/ d->step_groups,
                        d->softmax_scale, pos,
                        static_cast<const uint16_t*>(c), static_cast<const uint16_t*>(k_r), w_hyp,
                        pe, static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
                        static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
                        static_cast<uint16_t*>(cache), open_acc, static_cast<uint16_t*>(out)};
}

// absorb -> latent attention (-> split merge) -> up-projection.  With a
// merge (`merge` non-null: the token of a decode step) whose shapes allow it,
// the merge and the absorb run as one launch.
hipError_t run_decode_pipeline(const mtla_dims* dims, const int32_t* pos, const void* q_c,
                               const void* q_r, const void* w_uk, const void* w_uv,
                               const void* cache, void* out, void* workspace, const DecodeWs& ws,
                               hipStream_t s, const mtla::MergeArgs* merge = nullptr) {
  const int B = dims->batch, H = dims->heads;
  float* q_lat = reinterpret_cast<float*>(at(workspace, ws.qlat));
  float* o_lat = reinterpret_cast<float*>(at(workspace, ws.olat));
  hipError_t e;
  if (merge && mtla::merge_absorb_supported(dims->d_h, dims->d_c, dims->dtype)) {
    e = mtla::launch_merge_absorb(*merge, H, dims->d_h, dims->d_r, q_c, q_r, w_uk, q_lat, s);
  } else {
    if (merge && (e = mtla::launch_merge(*merge, dims->dtype, s)) != hipSuccess) return e;
    e = mtla::launch_absorb(B, H, dims->d_h, dims->d_c, dims->d_r, q_c, q_r, w_uk, q_lat, dims->dtype, s);
  }
  if (e != hipSuccess) return e;
  // several MFMA splits: their merge runs inside the up-projection's launch
  const int splits = decode_splits(dims);
  const bool combine = decode_fast(dims) && mtla::combine_up_project_supported(dims->d_h, dims->d_c, splits,
                                                                              dims->dtype);
  e = run_decode_attention(dims, pos, q_lat, cache, o_lat, workspace, ws.attn, s, !combine);
  if (e != hipSuccess) return e;
  if (combine)
    return mtla::launch_combine_up_project(B, H, dims->d_h, dims->d_c, splits, attn_partials(workspace, ws.attn),
                                           w_uv, out, s);
  return mtla::launch_up_project(B, H, dims->d_h, dims->d_c, o_lat, w_uv, out, dims->dtype, s);
}

}  // namespace

int32_t mtla_decode(const mtla_dims* dims, const int32_t* pos, const void* q_c, const void* q_r,
                    const void* w_uk, const void* w_uv, const void* cache, void* out,
                    void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (dims->batch == 0) return ok();
  CHECK_PTR_ALIGN(pos, 4);
  CHECK_PTR(q_c);
  if (dims->d_r > 0) CHECK_PTR(q_r);
  CHECK_PTR(w_uk);
  CHECK_PTR(w_uv);
  CHECK_PTR(cache);
  CHECK_PTR(out);
  const DecodeWs ws = decode_ws(dims);
  if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws.total);
  if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < ws.total)
    return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, ws.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (decode_fused(dims)) {
    const mtla::StepArgs a = step_args(dims, pos, nullptr, nullptr, nullptr, nullptr, 0, q_c, q_r,
                                       w_uk, w_uv, const_cast<void*>(cache), nullptr, out, 0);
    return hip_status(mtla::launch_decode_step(a, s), "decode step launch");
  }
  return hip_status(run_decode_pipeline(dims, pos, q_c, q_r, w_uk, w_uv, cache, out, workspace, ws, s),
                    "decode launch");
}

static int32_t decode_step_impl(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                                const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                                const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                                float* open_acc, void* out, void* workspace, size_t ws_bytes, void* stream,
                                bool check_only, const void* w_uv_tiles,
                                unsigned long long* timeline = nullptr);

int32_t mtla_decode_step(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                         const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                         const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                         float* open_acc, void* out, void* workspace, size_t ws_bytes,
                         void* stream) {
  return decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, out,
                          workspace, ws_bytes, stream, false, nullptr);
}

int32_t mtla_w_uv_tiles_bytes(const mtla_dims* dims, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  if (dims->dtype != MTLA_BF16) return fail(MTLA_ERR_UNSUPPORTED, "W_UV tiles are bf16 only");
  if (dims->d_c % 32 != 0) return fail(MTLA_ERR_UNSUPPORTED, "d_c=%d is not a multiple of 32", dims->d_c);
  *bytes = mtla::w_uv_tiles_elems(dims->heads, dims->d_h, dims->d_c) * sizeof(uint16_t);
  return ok();
}

int32_t mtla_pack_w_uv_tiles(const mtla_dims* dims, const void* w_uv, void* w_uv_tiles, void* stream) {
  size_t bytes = 0;
  int32_t st = mtla_w_uv_tiles_bytes(dims, &bytes);
  if (st != MTLA_OK) return st;
  if (!w_uv || !aligned16(w_uv)) return fail(MTLA_ERR_INVALID_ARG, "w_uv is NULL or not 16-byte aligned");
  if (!w_uv_tiles || !aligned16(w_uv_tiles))
    return fail(MTLA_ERR_INVALID_ARG, "w_uv_tiles is NULL or not 16-byte aligned");
  return hip_status(mtla::launch_pack_w_uv_tiles(dims->heads, dims->d_h, dims->d_c, static_cast<const uint16_t*>(w_uv),
                                                 static_cast<uint16_t*>(w_uv_tiles), static_cast<hipStream_t>(stream)),
                    "W_UV tile pack launch");
}

int32_t mtla_decode_step_tiles(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                               const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                               const void* q_r, const void* w_uk, const void* w_uv, const void* w_uv_tiles,
                               void* cache, float* open_acc, void* out, void* workspace, size_t ws_bytes,
                               void* stream) {
  size_t bytes = 0;
  int32_t st = mtla_w_uv_tiles_bytes(dims, &bytes);
  if (st != MTLA_OK) return st;
  if (!w_uv_tiles || !aligned16(w_uv_tiles))
    return fail(MTLA_ERR_INVALID_ARG, "w_uv_tiles is NULL or not 16-byte aligned");
  return decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, out,
                          workspace, ws_bytes, stream, false, w_uv_tiles);
}

// The timeline instance of the fused step (measurement): the same checks and
// work as mtla_decode_step_tiles on the shapes that run the one-kernel step
// for 256-wide latents with one W_hyp row.
int32_t mtla_calib_step_timeline(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                                 const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                                 const void* q_r, const void* w_uk, const void* w_uv, const void* w_uv_tiles,
                                 void* cache, float* open_acc, void* out, void* workspace, size_t ws_bytes,
                                 uint64_t* timeline, size_t timeline_entries, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (dims->dtype != MTLA_BF16 || dims->d_c != 256 || dims->d_r != 32 || !decode_fused(dims) ||
      gate_stride(dims) != 0)
    return fail(MTLA_ERR_UNSUPPORTED,
                "the step timeline covers the one-kernel bf16 step with d_c=256, d_r=32 and one W_hyp row");
  const int groups = mtla::decode_step_groups(dims->batch, dims->heads, dims->d_h, dims->d_c, dims->step_groups);
  if (groups < 1) return fail(MTLA_ERR_UNSUPPORTED, "no head grouping of the fused step fits these dims");
  const size_t need = static_cast<size_t>(8) * groups * ((dims->batch + 7) / 8) * mtla::kStepTimelineSlots;
  if (!timeline || !aligned_to(timeline, 8)) return fail(MTLA_ERR_INVALID_ARG, "timeline is NULL or not 8-byte aligned");
  if (timeline_entries < need)
    return fail(MTLA_ERR_INVALID_ARG, "timeline holds %zu entries < %zu needed", timeline_entries, need);
  size_t bytes = 0;
  if ((st = mtla_w_uv_tiles_bytes(dims, &bytes)) != MTLA_OK) return st;
  if (!w_uv_tiles || !aligned16(w_uv_tiles))
    return fail(MTLA_ERR_INVALID_ARG, "w_uv_tiles is NULL or not 16-byte aligned");
  return decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, out,
                          workspace, ws_bytes, stream, false, w_uv_tiles,
                          reinterpret_cast<unsigned long long*>(timeline));
}

static int32_t decode_step_impl(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                                const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                                const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                                float* open_acc, void* out, void* workspace, size_t ws_bytes, void* stream,
                                bool check_only, const void* w_uv_tiles, unsigned long long* timeline) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (pe_rows < 1) return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < 1", pe_rows);
  if (dims->batch == 0) return ok();
  CHECK_PTR_ALIGN(pos, 4);
  CHECK_PTR(c);
  if (dims->d_r > 0) CHECK_PTR(k_r);
  CHECK_PTR_ALIGN(w_hyp, 4);
  CHECK_PTR_ALIGN(pe, 4);
  CHECK_PTR(q_c);
  if (dims->d_r > 0) CHECK_PTR(q_r);
  CHECK_PTR(w_uk);
  CHECK_PTR(w_uv);
  CHECK_PTR(cache);
  CHECK_PTR(open_acc);
  CHECK_PTR(out);
  const DecodeWs ws = decode_ws(dims);
  if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws.total);
  if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < ws.total)
    return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, ws.total);
  if (check_only) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the fused step kernels merge with one W_hyp row per place in the block
  // only for 256-wide latents; otherwise that merge runs first, on its own
  const bool per_place = gate_stride(dims) != 0;
  if (decode_fused(dims) && (!per_place || dims->d_c == 256)) {
    mtla::StepArgs a = step_args(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv,
                                 cache, open_acc, out, 1);
    a.wh_stride = gate_stride(dims);
    if (dims->d_c == 256) a.w_uv_tiles = static_cast<const uint16_t*>(w_uv_tiles);
    a.timeline = timeline;
    return hip_status(mtla::launch_decode_step(a, s), "decode step launch");
  }
  mtla::MergeArgs m{dims->batch, 1, dims->d_c, dims->d_r, dims->stride_s, dims->max_slots, pe_rows,
                    pos, c, k_r, w_hyp, pe, cache, open_acc, nullptr, nullptr};
  m.wh_stride = gate_stride(dims);
  if (decode_fused(dims)) {
    hipError_t e = mtla::launch_merge(m, dims->dtype, s);
    if (e != hipSuccess) return hip_status(e, "merge launch");
    const mtla::StepArgs a = step_args(dims, pos, nullptr, nullptr, nullptr, nullptr, 0, q_c, q_r, w_uk, w_uv,
                                       cache, nullptr, out, 0);
    return hip_status(mtla::launch_decode_step(a, s), "decode step launch");
  }
  return hip_status(run_decode_pipeline(dims, pos, q_c, q_r, w_uk, w_uv, cache, out, workspace, ws, s, &m),
                    "decode launch");
}

// ---------------------------------------------------------------------------
// Allocation-free decode step.  Its workspace is this file-scope device
// array (every GPU the library runs on holds its own copy until the process
// ends).  In host code `scratch` names a host-side stand-in, not device
// memory: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MTLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of `scratch` on the current device (resolved on the first
// call made with that device current).
int32_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MTLA_ERR_UNSUPPORTED, "device %d is past the %d supported", dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_status(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  if (!g_scratch_ptr[dev]) return fail(MTLA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
  *ptr = g_scratch_ptr[dev];
  return ok();
}
}  // namespace

int32_t mtla_decode_step_noalloc(const mtla_dims* dims, const int32_t* pos, const void* c, const void* k_r,
                                 const float* w_hyp, const float* pe, int32_t pe_rows, const void* q_c,
                                 const void* q_r, const void* w_uk, const void* w_uv, void* cache,
                                 float* open_acc, void* out, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  const size_t need = decode_ws(dims).total;
  if (need > MTLA_NOALLOC_SCRATCH_BYTES)
    return fail(MTLA_ERR_WORKSPACE,
                "these dims need %zu bytes of workspace, more than the %zu bytes of static scratch "
                "(use mtla_decode_step with a workspace)",
                need, static_cast<size_t>(MTLA_NOALLOC_SCRATCH_BYTES));
  // every other argument check, before any HIP call (a stand-in workspace
  // address: only its non-null, aligned value is checked)
  st = decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, out,
                        reinterpret_cast<void*>(static_cast<uintptr_t>(256)), MTLA_NOALLOC_SCRATCH_BYTES,
                        stream, true, nullptr);
  if (st != MTLA_OK || dims->batch == 0) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MTLA_OK) return st;
  return decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, out,
                          ws, MTLA_NOALLOC_SCRATCH_BYTES, stream, false, nullptr);
}

int32_t mtla_prefill_workspace_bytes(const mtla_dims* dims, int32_t n_tokens, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = prefill_ws(dims, n_tokens).total;
  return ok();
}

// Prefill of tokens t0+1 .. t0+n_tokens of every sequence (t0 = 0: from an
// empty cache).
static int32_t prefill_impl(const mtla_dims* dims, int32_t t0, int32_t n_tokens, const void* q_c,
                            const void* q_r, const void* c, const void* k_r, const float* w_hyp,
                            const float* pe, int32_t pe_rows, const void* w_uk, const void* w_uv,
                            void* cache, float* open_acc, void* out, void* workspace, size_t ws_bytes,
                            void* stream, bool check_only = false) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (t0 < 0) return fail(MTLA_ERR_INVALID_ARG, "t0=%d < 0", t0);
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  const int64_t t_end = int64_t(t0) + n_tokens;
  if (pe_rows < t_end)
    return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < t0 + n_tokens = %lld", pe_rows, static_cast<long long>(t_end));
  if (t_end > int64_t(dims->max_slots) * dims->stride_s)
    return fail(MTLA_ERR_INVALID_ARG, "t0 + n_tokens = %lld exceeds the cache capacity s*max_slots",
                static_cast<long long>(t_end));
  if (int64_t(dims->batch) * n_tokens * dims->heads * (dims->d_c + dims->d_r) > kMaxElems)
    return fail(MTLA_ERR_UNSUPPORTED, "prefill too large");
  // the partial merges [B, N, W] are read through a buffer resource (32-bit size)
  if (int64_t(dims->batch) * n_tokens * (dims->d_c + dims->d_r) * 4 > INT32_MAX)
    return fail(MTLA_ERR_UNSUPPORTED, "prefill of %d x %d tokens exceeds the 2^31-byte partial-merge buffer",
                dims->batch, n_tokens);
  // with t0 > 0 the cache rows of all sequences are one GEMM operand (32-bit size)
  if (t0 > 0 && int64_t(dims->batch) * dims->max_slots * (dims->d_c + dims->d_r) * 2 > INT32_MAX)
    return fail(MTLA_ERR_UNSUPPORTED, "cache of %d x %d slots exceeds the 2^31-byte operand buffer",
                dims->batch, dims->max_slots);
  if (dims->batch == 0 || n_tokens == 0) return ok();
  CHECK_PTR(q_c);
  if (dims->d_r > 0) CHECK_PTR(q_r);
  CHECK_PTR(c);
  if (dims->d_r > 0) CHECK_PTR(k_r);
  CHECK_PTR_ALIGN(w_hyp, 4);
  CHECK_PTR_ALIGN(pe, 4);
  CHECK_PTR(w_uk);
  CHECK_PTR(w_uv);
  CHECK_PTR(cache);
  CHECK_PTR(open_acc);
  CHECK_PTR(out);
  const PrefillWs ws = prefill_ws(dims, n_tokens, t0);
  if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws.total);
  if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < ws.total)
    return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, ws.total);
  if (check_only) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = dims->batch, H = dims->heads, N = n_tokens;
  void* P = at(workspace, ws.P);
  mtla::MergeArgs m{B, N, dims->d_c, dims->d_r, dims->stride_s, dims->max_slots, pe_rows,
                    nullptr, c, k_r, w_hyp, pe, cache, open_acc, nullptr, P, t0 + 1};
  m.wh_stride = gate_stride(dims);
  hipError_t e = mtla::launch_merge(m, dims->dtype, s);
  if (e != hipSuccess) return hip_status(e, "prefill merge launch");
  if (prefill_fast(dims)) {
    // K^C and V of the completed slots the queries attend, then the attention
    // (which forms each query's diagonal key itself).  From token 1 the slot
    // keys are the partial merges at block ends (rows s*j + s - 1), as in the
    // staged calls; after t0 cached tokens they are the cache rows, which the
    // merge has just completed.
    void* kc = at(workspace, ws.kc);
    void* v = at(workspace, ws.v);
    const int nsl = prefill_slot_keys(dims, N, t0);
    const int S = dims->stride_s;
    mtla::PrefillAttnArgs pa{B, N, H, dims->d_h, dims->d_c, dims->d_r, S, 0, dims->softmax_scale,
                             q_c, q_r, P, w_uk, w_uv, out, t0, kc, v, nsl};
    if (t0 == 0) {
      e = mtla::launch_prefill_kv(B, nsl, N, S, S - 1, H, dims->d_h, dims->d_c, dims->d_r, P, w_uk, w_uv, kc, v,
                                  true, s);
      pa.rslot = P;
      pa.rslot_rows = N;
      pa.rslot_mul = S;
      pa.rslot_add = S - 1;
    } else {
      e = mtla::launch_prefill_kv(B, nsl, dims->max_slots, 1, 0, H, dims->d_h, dims->d_c, dims->d_r, cache, w_uk,
                                  w_uv, kc, v, true, s);
      pa.rslot = cache;
      pa.rslot_rows = dims->max_slots;
      pa.rslot_mul = 1;
      pa.rslot_add = 0;
    }
    if (e != hipSuccess) return hip_status(e, "slot up-projection launch");
    return hip_status(mtla::launch_prefill_attn(pa, s), "prefill attention launch");
  }
  const int R = B * N;
  const int splits = prefill_splits(dims, t0 + N);
  float* q_lat = reinterpret_cast<float*>(at(workspace, ws.qlat));
  float* o_lat = reinterpret_cast<float*>(at(workspace, ws.olat));
  mtla::Partials p{reinterpret_cast<float*>(at(workspace, ws.attn.pm)),
                   reinterpret_cast<float*>(at(workspace, ws.attn.pl)),
                   reinterpret_cast<float*>(at(workspace, ws.attn.pacc))};
  e = mtla::launch_absorb(R, H, dims->d_h, dims->d_c, dims->d_r, q_c, q_r, w_uk, q_lat,
                          dims->dtype, s);
  if (e != hipSuccess) return hip_status(e, "prefill absorb launch");
  mtla::AttendArgs a{R, N, H, dims->d_c, dims->d_r, dims->stride_s, dims->max_slots, splits,
                     dims->softmax_scale, nullptr, q_lat, cache, P, p, o_lat, t0};
  e = mtla::launch_attend_portable(a, dims->dtype, s);
  if (e != hipSuccess) return hip_status(e, "prefill attention launch");
  e = mtla::launch_up_project(R, H, dims->d_h, dims->d_c, o_lat, w_uv, out, dims->dtype, s);
  return hip_status(e, "prefill up-projection launch");
}

int32_t mtla_prefill(const mtla_dims* dims, int32_t n_tokens, const void* q_c, const void* q_r,
                     const void* c, const void* k_r, const float* w_hyp, const float* pe,
                     int32_t pe_rows, const void* w_uk, const void* w_uv, void* cache,
                     float* open_acc, void* out, void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(dims, 0, n_tokens, q_c, q_r, c, k_r, w_hyp, pe, pe_rows, w_uk, w_uv, cache, open_acc,
                      out, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Staged prefill (t0 = 0): partial merges, K/V up-projection, attention.
// ---------------------------------------------------------------------------
namespace {
int32_t check_staged_prefill(const mtla_dims* dims, int32_t n_tokens) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if (!prefill_fast(dims))
    return fail(MTLA_ERR_UNSUPPORTED, "the staged prefill needs bf16 storage and a shape with the MFMA path");
  if (int64_t(n_tokens) > int64_t(dims->max_slots) * dims->stride_s)
    return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d exceeds the cache capacity s*max_slots", n_tokens);
  if (int64_t(dims->batch) * n_tokens * (dims->d_c + dims->d_r) * 4 > INT32_MAX)
    return fail(MTLA_ERR_UNSUPPORTED, "prefill of %d x %d tokens exceeds the 2^31-byte partial-merge buffer",
                dims->batch, n_tokens);
  return MTLA_OK;
}
}  // namespace

int32_t mtla_prefill_partials(const mtla_dims* dims, int32_t n_tokens, const void* c, const void* k_r,
                              const float* w_hyp, const float* pe, int32_t pe_rows, void* cache, float* open_acc,
                              void* partials, void* stream) {
  int32_t st = check_staged_prefill(dims, n_tokens);
  if (st != MTLA_OK) return st;
  if (pe_rows < n_tokens) return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < n_tokens=%d", pe_rows, n_tokens);
  if (dims->batch == 0 || n_tokens == 0) return ok();
  CHECK_PTR(c);
  if (dims->d_r > 0) CHECK_PTR(k_r);
  CHECK_PTR_ALIGN(w_hyp, 4);
  CHECK_PTR_ALIGN(pe, 4);
  CHECK_PTR(cache);
  CHECK_PTR(open_acc);
  CHECK_PTR(partials);
  mtla::MergeArgs m{dims->batch, n_tokens, dims->d_c, dims->d_r, dims->stride_s, dims->max_slots, pe_rows,
                    nullptr, c, k_r, w_hyp, pe, cache, open_acc, nullptr, partials, 1};
  m.wh_stride = gate_stride(dims);
  return hip_status(mtla::launch_merge(m, dims->dtype, static_cast<hipStream_t>(stream)), "prefill merge launch");
}

int32_t mtla_prefill_keys(const mtla_dims* dims, int32_t n_tokens, const void* partials, const void* w_uk,
                          const void* w_uv, void* k_c, void* v, void* stream) {
  int32_t st = check_staged_prefill(dims, n_tokens);
  if (st != MTLA_OK) return st;
  const int nsl = prefill_slot_keys(dims, n_tokens, 0);
  if (dims->batch == 0 || nsl == 0) return ok();
  CHECK_PTR(partials);
  CHECK_PTR(w_uk);
  CHECK_PTR(w_uv);
  CHECK_PTR(k_c);
  CHECK_PTR(v);
  const int S = dims->stride_s;
  return hip_status(mtla::launch_prefill_kv(dims->batch, nsl, n_tokens, S, S - 1, dims->heads, dims->d_h, dims->d_c,
                                            dims->d_r, partials, w_uk, w_uv, k_c, v, true,
                                            static_cast<hipStream_t>(stream)),
                    "up-projection launch");
}

int32_t mtla_prefill_attention(const mtla_dims* dims, int32_t n_tokens, const void* q_c, const void* q_r,
                               const void* partials, const void* w_uk, const void* w_uv, const void* k_c,
                               const void* v, void* out, void* stream) {
  int32_t st = check_staged_prefill(dims, n_tokens);
  if (st != MTLA_OK) return st;
  if (dims->batch == 0 || n_tokens == 0) return ok();
  const int nsl = prefill_slot_keys(dims, n_tokens, 0);
  CHECK_PTR(q_c);
  if (dims->d_r > 0) CHECK_PTR(q_r);
  CHECK_PTR(partials);
  CHECK_PTR(w_uk);
  CHECK_PTR(w_uv);
  if (nsl > 0) {
    CHECK_PTR(k_c);
    CHECK_PTR(v);
  }
  CHECK_PTR(out);
  const int S = dims->stride_s;
  mtla::PrefillAttnArgs pa{dims->batch, n_tokens, dims->heads, dims->d_h, dims->d_c, dims->d_r, S, 0,
                           dims->softmax_scale, q_c, q_r, partials, w_uk, w_uv, out, 0, k_c, v, nsl,
                           partials, n_tokens, S, S - 1};
  return hip_status(mtla::launch_prefill_attn(pa, static_cast<hipStream_t>(stream)), "prefill attention launch");
}

int32_t mtla_prefill_at_workspace_bytes(const mtla_dims* dims, int32_t t0, int32_t n_tokens, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (t0 < 0) return fail(MTLA_ERR_INVALID_ARG, "t0=%d < 0", t0);
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = prefill_ws(dims, n_tokens, t0).total;
  return ok();
}

int32_t mtla_prefill_at(const mtla_dims* dims, int32_t t0, int32_t n_tokens, const void* q_c,
                        const void* q_r, const void* c, const void* k_r, const float* w_hyp,
                        const float* pe, int32_t pe_rows, const void* w_uk, const void* w_uv, void* cache,
                        float* open_acc, void* out, void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(dims, t0, n_tokens, q_c, q_r, c, k_r, w_hyp, pe, pe_rows, w_uk, w_uv, cache, open_acc,
                      out, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// The decoder layer around the core: input and output projections, and a
// whole layer step / prefill from h.
// ---------------------------------------------------------------------------

static int32_t check_layer(const mtla_dims* d, int32_t d_model) {
  if (d_model < 8 || d_model % 8 != 0)
    return fail(MTLA_ERR_UNSUPPORTED, "d_model=%d must be a positive multiple of 8", d_model);
  if ((int64_t(d->heads) * d->d_h) % 8 != 0)
    return fail(MTLA_ERR_UNSUPPORTED, "heads*d_h=%lld must be a multiple of 8",
                static_cast<long long>(int64_t(d->heads) * d->d_h));
  if (d->d_h % 2 != 0) return fail(MTLA_ERR_UNSUPPORTED, "d_h=%d must be even", d->d_h);
  return ok();
}

static mtla::LayerGemmArgs input_gemm(const mtla_dims* d, int32_t d_model, int32_t n_tokens,
                                      const int32_t* pos0, int32_t p0_all, const void* h, const void* w_dkv,
                                      const void* w_q, const void* w_r, void* c, void* k_r, void* q_c,
                                      void* q_r) {
  mtla::LayerGemmArgs g{};
  g.M = d->batch * n_tokens;
  g.N = d->d_c + d->heads * (d->d_h + d->d_r) + d->d_r;
  g.K = d_model;
  g.A = h;
  g.w0 = w_dkv;
  g.n0 = d->d_c;
  g.w1 = w_q;
  g.n1 = d->heads * (d->d_h + d->d_r);
  g.w2 = w_r;
  g.mode = 1;
  g.T = n_tokens;
  g.H = d->heads;
  g.d_h = d->d_h;
  g.d_r = d->d_r;
  g.d_c = d->d_c;
  g.pos0 = pos0;
  g.p0_all = p0_all;
  g.c = c;
  g.k_r = k_r;
  g.q_c = q_c;
  g.q_r = q_r;
  return g;
}

static mtla::LayerGemmArgs output_gemm(const mtla_dims* d, int32_t d_model, int32_t n_rows, const void* o,
                                       const void* w_o, void* y) {
  mtla::LayerGemmArgs g{};
  g.M = n_rows;
  g.N = d_model;
  g.K = d->heads * d->d_h;
  g.A = o;
  g.w0 = w_o;
  g.n0 = d_model;
  g.w1 = w_o;
  g.w2 = w_o;
  g.mode = 0;
  g.out = y;
  return g;
}

static int32_t check_rows(const mtla_dims* d, int64_t rows, int32_t d_model) {
  const int64_t width = std::max<int64_t>(d_model, d->d_c + int64_t(d->heads) * (d->d_h + d->d_r) + d->d_r);
  if (rows > INT32_MAX || rows * width > kMaxElems)
    return fail(MTLA_ERR_UNSUPPORTED, "%lld rows of width %lld are too many", static_cast<long long>(rows),
                static_cast<long long>(width));
  return ok();
}

int32_t mtla_project_inputs(const mtla_dims* dims, int32_t d_model, int32_t n_tokens, const int32_t* pos0,
                            const void* h, const void* w_dkv, const void* w_q, const void* w_r, void* c,
                            void* k_r, void* q_c, void* q_r, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if ((st = check_layer(dims, d_model)) != MTLA_OK) return st;
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if ((st = check_rows(dims, int64_t(dims->batch) * n_tokens, d_model)) != MTLA_OK) return st;
  if (dims->batch == 0 || n_tokens == 0) return ok();
  CHECK_PTR_ALIGN(pos0, 4);
  CHECK_PTR(h);
  CHECK_PTR(w_dkv);
  CHECK_PTR(w_q);
  if (dims->d_r > 0) {
    CHECK_PTR(w_r);
    CHECK_PTR_ALIGN(k_r, 4);
    CHECK_PTR_ALIGN(q_r, 4);
  }
  CHECK_PTR_ALIGN(c, 4);
  CHECK_PTR_ALIGN(q_c, 4);
  const mtla::LayerGemmArgs g = input_gemm(dims, d_model, n_tokens, pos0, 1, h, w_dkv, w_q, w_r, c, k_r, q_c, q_r);
  return hip_status(mtla::launch_layer_gemm(g, dims->dtype, static_cast<hipStream_t>(stream)),
                    "input projection launch");
}

int32_t mtla_output_project(const mtla_dims* dims, int32_t d_model, int32_t n_rows, const void* o,
                            const void* w_o, void* y, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if ((st = check_layer(dims, d_model)) != MTLA_OK) return st;
  if (n_rows < 0) return fail(MTLA_ERR_INVALID_ARG, "n_rows=%d < 0", n_rows);
  if ((st = check_rows(dims, n_rows, d_model)) != MTLA_OK) return st;
  if (n_rows == 0) return ok();
  CHECK_PTR(o);
  CHECK_PTR(w_o);
  CHECK_PTR_ALIGN(y, 4);
  const mtla::LayerGemmArgs g = output_gemm(dims, d_model, n_rows, o, w_o, y);
  return hip_status(mtla::launch_layer_gemm(g, dims->dtype, static_cast<hipStream_t>(stream)),
                    "output projection launch");
}

namespace {
// Workspace of a layer call over R rows: c, k_r, q_c, q_r and the heads'
// outputs o (storage dtype), then the core call's own workspace.
struct LayerWs {
  size_t c, k_r, q_c, q_r, o, core, total;
};
LayerWs layer_ws(const mtla_dims* d, size_t R, size_t core_bytes) {
  const size_t e = elem_bytes(d), H = d->heads;
  LayerWs w;
  size_t off = 0;
  w.c = off;
  off += align_up(R * d->d_c * e);
  w.k_r = off;
  off += align_up(R * d->d_r * e);
  w.q_c = off;
  off += align_up(R * H * d->d_h * e);
  w.q_r = off;
  off += align_up(R * H * d->d_r * e);
  w.o = off;
  off += align_up(R * H * d->d_h * e);
  w.core = off;
  w.total = off + core_bytes;
  return w;
}
}  // namespace

int32_t mtla_layer_decode_workspace_bytes(const mtla_dims* dims, int32_t d_model, size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if ((st = check_layer(dims, d_model)) != MTLA_OK) return st;
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layer_ws(dims, dims->batch, decode_ws(dims).total).total;
  return ok();
}

static int32_t layer_decode_step_impl(const mtla_dims* dims, int32_t d_model, const int32_t* pos, const void* h,
                                     const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                                     const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                                     const void* w_uv, const void* w_uv_tiles, void* cache, float* open_acc,
                                     void* y, void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if ((st = check_layer(dims, d_model)) != MTLA_OK) return st;
  if (pe_rows < 1) return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < 1", pe_rows);
  if ((st = check_rows(dims, dims->batch, d_model)) != MTLA_OK) return st;
  if (dims->batch == 0) return ok();
  CHECK_PTR(h);
  CHECK_PTR(w_o);
  CHECK_PTR_ALIGN(y, 4);
  const DecodeWs dw = decode_ws(dims);
  const LayerWs lw = layer_ws(dims, dims->batch, dw.total);
  if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", lw.total);
  if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < lw.total)
    return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, lw.total);
  void *c = at(workspace, lw.c), *k_r = at(workspace, lw.k_r), *q_c = at(workspace, lw.q_c),
       *q_r = at(workspace, lw.q_r), *o = at(workspace, lw.o);
  // the core's own checks run before anything is enqueued
  if ((st = decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, o,
                             at(workspace, lw.core), dw.total, nullptr, true, nullptr)) != MTLA_OK)
    return st;
  if ((st = mtla_project_inputs(dims, d_model, 1, pos, h, w_dkv, w_q, w_r, c, k_r, q_c, q_r, stream)) != MTLA_OK)
    return st;
  if ((st = decode_step_impl(dims, pos, c, k_r, w_hyp, pe, pe_rows, q_c, q_r, w_uk, w_uv, cache, open_acc, o,
                             at(workspace, lw.core), dw.total, stream, false, w_uv_tiles)) != MTLA_OK)
    return st;
  return mtla_output_project(dims, d_model, dims->batch, o, w_o, y, stream);
}

int32_t mtla_layer_decode_step(const mtla_dims* dims, int32_t d_model, const int32_t* pos, const void* h,
                               const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                               const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                               const void* w_uv, void* cache, float* open_acc, void* y, void* workspace,
                               size_t ws_bytes, void* stream) {
  return layer_decode_step_impl(dims, d_model, pos, h, w_dkv, w_q, w_r, w_o, w_hyp, pe, pe_rows, w_uk, w_uv,
                                nullptr, cache, open_acc, y, workspace, ws_bytes, stream);
}

int32_t mtla_layer_decode_step_tiles(const mtla_dims* dims, int32_t d_model, const int32_t* pos, const void* h,
                                     const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                                     const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                                     const void* w_uv, const void* w_uv_tiles, void* cache, float* open_acc,
                                     void* y, void* workspace, size_t ws_bytes, void* stream) {
  size_t bytes = 0;
  int32_t st = mtla_w_uv_tiles_bytes(dims, &bytes);
  if (st != MTLA_OK) return st;
  if (!w_uv_tiles || !aligned16(w_uv_tiles))
    return fail(MTLA_ERR_INVALID_ARG, "w_uv_tiles is NULL or not 16-byte aligned");
  return layer_decode_step_impl(dims, d_model, pos, h, w_dkv, w_q, w_r, w_o, w_hyp, pe, pe_rows, w_uk, w_uv,
                                w_uv_tiles, cache, open_acc, y, workspace, ws_bytes, stream);
}

int32_t mtla_layer_prefill_workspace_bytes(const mtla_dims* dims, int32_t d_model, int32_t t0, int32_t n_tokens,
                                           size_t* bytes) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if ((st = check_layer(dims, d_model)) != MTLA_OK) return st;
  if (t0 < 0) return fail(MTLA_ERR_INVALID_ARG, "t0=%d < 0", t0);
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layer_ws(dims, size_t(dims->batch) * n_tokens, prefill_ws(dims, n_tokens, t0).total).total;
  return ok();
}

int32_t mtla_layer_prefill(const mtla_dims* dims, int32_t d_model, int32_t t0, int32_t n_tokens, const void* h,
                           const void* w_dkv, const void* w_q, const void* w_r, const void* w_o,
                           const float* w_hyp, const float* pe, int32_t pe_rows, const void* w_uk,
                           const void* w_uv, void* cache, float* open_acc, void* y, void* workspace,
                           size_t ws_bytes, void* stream) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if ((st = check_layer(dims, d_model)) != MTLA_OK) return st;
  if (t0 < 0) return fail(MTLA_ERR_INVALID_ARG, "t0=%d < 0", t0);
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if ((st = check_rows(dims, int64_t(dims->batch) * n_tokens, d_model)) != MTLA_OK) return st;
  // (before the workspace check: the workspace size depends on t0)
  if (pe_rows < int64_t(t0) + n_tokens)
    return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < t0 + n_tokens = %lld", pe_rows,
                static_cast<long long>(int64_t(t0) + n_tokens));
  if (int64_t(t0) + n_tokens > int64_t(dims->max_slots) * dims->stride_s)
    return fail(MTLA_ERR_INVALID_ARG, "t0 + n_tokens = %lld exceeds the cache capacity s*max_slots",
                static_cast<long long>(int64_t(t0) + n_tokens));
  if (dims->batch == 0 || n_tokens == 0) return ok();
  CHECK_PTR(h);
  CHECK_PTR(w_dkv);
  CHECK_PTR(w_q);
  if (dims->d_r > 0) CHECK_PTR(w_r);
  CHECK_PTR(w_o);
  CHECK_PTR_ALIGN(y, 4);
  const size_t R = size_t(dims->batch) * n_tokens;
  const PrefillWs pw = prefill_ws(dims, n_tokens, t0);
  const LayerWs lw = layer_ws(dims, R, pw.total);
  if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", lw.total);
  if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < lw.total)
    return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, lw.total);
  void *c = at(workspace, lw.c), *k_r = at(workspace, lw.k_r), *q_c = at(workspace, lw.q_c),
       *q_r = at(workspace, lw.q_r), *o = at(workspace, lw.o);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // run the core's own checks before anything is enqueued
  if ((st = prefill_impl(dims, t0, n_tokens, q_c, q_r, c, k_r, w_hyp, pe, pe_rows, w_uk, w_uv, cache, open_acc,
                         o, at(workspace, lw.core), pw.total, nullptr, /*check_only=*/true)) != MTLA_OK)
    return st;
  const mtla::LayerGemmArgs g =
      input_gemm(dims, d_model, n_tokens, nullptr, t0 + 1, h, w_dkv, w_q, w_r, c, k_r, q_c, q_r);
  hipError_t e = mtla::launch_layer_gemm(g, dims->dtype, s);
  if (e != hipSuccess) return hip_status(e, "input projection launch");
  if ((st = prefill_impl(dims, t0, n_tokens, q_c, q_r, c, k_r, w_hyp, pe, pe_rows, w_uk, w_uv, cache, open_acc,
                         o, at(workspace, lw.core), pw.total, stream)) != MTLA_OK)
    return st;
  return mtla_output_project(dims, d_model, n_tokens * dims->batch, o, w_o, y, stream);
}

// ---------------------------------------------------------------------------
// Training backward of the parallel pass.
// ---------------------------------------------------------------------------
namespace {
struct BwdWs {
  size_t P, gate, KV, lse, D, dKV, Wt, dPc, wg_part, du, wh_part, total;
  size_t kc, v, pd, dsd;  // MFMA path
  int wg_splits, wh_parts;
  bool fast;
};

// The MFMA attention backward runs where the forward's MFMA prefill does,
// with d_h = 64 and d_r = 32.
bool backward_fast(const mtla_dims* d) { return prefill_fast(d) && mtla::bwd_mfma_supported(d->d_h, d->d_r); }

BwdWs bwd_ws(const mtla_dims* d, int n) {
  const size_t B = d->batch, H = d->heads, N = n, R = B * N, W = d->d_c + d->d_r;
  const size_t KV2 = 2 * H * d->d_h, e = elem_bytes(d);
  BwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  w.fast = backward_fast(d);
  w.P = take(R * W * e);
  w.gate = take(R * 4);
  if (w.fast) {
    w.kc = take(B * H * N * d->d_h * e);
    w.v = take(B * H * N * d->d_h * e);
    w.pd = take(B * H * N * 4);
    w.dsd = take(B * H * N * 4);
  } else {
    w.KV = take(R * KV2 * e);
  }
  w.lse = take(B * H * N * 4);
  w.D = take(B * H * N * 4);
  w.dKV = take(R * (KV2 + H * d->d_r) * e);
  w.Wt = take(size_t(d->d_c) * KV2 * e);
  w.dPc = take(R * d->d_c * 4);
  // split the weight-gradient product over rows so that ~1024 workgroups run
  const size_t tiles = mtla::bwd_wgrad_tiles(static_cast<int>(KV2), d->d_c, d->dtype);
  w.wg_splits = static_cast<int>(std::max<size_t>(1, std::min<size_t>((1024 + tiles - 1) / tiles, (R + 255) / 256)));
  w.wg_part = take(size_t(w.wg_splits) * KV2 * d->d_c * 4);
  w.du = take(R * 4);
  // dW_hyp: partial sums over chunks of ~256 rows
  w.wh_parts = static_cast<int>(std::max<size_t>(1, std::min<size_t>((R + 255) / 256, 4096)));
  w.wh_part = take(size_t(w.wh_parts) * gate_rows(d) * d->d_c * 4);
  w.total = off;
  return w;
}

int32_t check_backward(const mtla_dims* dims, int32_t n_tokens) {
  int32_t st = check_dims(dims);
  if (st != MTLA_OK) return st;
  if (n_tokens < 0) return fail(MTLA_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if ((int64_t(dims->heads) * dims->d_h) % 4 != 0)
    return fail(MTLA_ERR_UNSUPPORTED, "heads*d_h=%lld must be a multiple of 4",
                static_cast<long long>(int64_t(dims->heads) * dims->d_h));
  if (dims->batch > 65535 || dims->heads > 65535)
    return fail(MTLA_ERR_UNSUPPORTED, "batch=%d and heads=%d must be <= 65535", dims->batch, dims->heads);
  if (2 * int64_t(dims->heads) * dims->d_h * dims->d_c > INT32_MAX)
    return fail(MTLA_ERR_UNSUPPORTED, "W_UK and W_UV of %d x %d x %d are too large", dims->heads, dims->d_h,
                dims->d_c);
  const int64_t R = int64_t(dims->batch) * n_tokens;
  const int64_t width = 2 * int64_t(dims->heads) * dims->d_h + int64_t(dims->heads) * dims->d_r;
  // one sequence's query rows are addressed through 32-bit byte offsets
  if (int64_t(n_tokens) * dims->heads * (dims->d_h + dims->d_r) * 4 > INT32_MAX ||
      int64_t(n_tokens) * (dims->d_c + dims->d_r) * 4 > INT32_MAX)
    return fail(MTLA_ERR_UNSUPPORTED, "n_tokens=%d is too long for one sequence's 2^31-byte rows", n_tokens);
  if (R > INT32_MAX || R * std::max<int64_t>(width, dims->d_c + dims->d_r) > kMaxElems)
    return fail(MTLA_ERR_UNSUPPORTED, "%lld token rows are too many", static_cast<long long>(R));
  return ok();
}
}  // namespace

int32_t mtla_prefill_backward_workspace_bytes(const mtla_dims* dims, int32_t n_tokens, size_t* bytes) {
  int32_t st = check_backward(dims, n_tokens);
  if (st != MTLA_OK) return st;
  if (!bytes) return fail(MTLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_ws(dims, n_tokens).total;
  return ok();
}

int32_t mtla_prefill_backward(const mtla_dims* dims, int32_t n_tokens, const void* q_c, const void* q_r,
                              const void* c, const void* k_r, const float* w_hyp, const float* pe,
                              int32_t pe_rows, const void* w_uk, const void* w_uv, const void* grad_out,
                              void* grad_q_c, void* grad_q_r, void* grad_c, void* grad_k_r, float* grad_w_hyp,
                              float* grad_w_uk, float* grad_w_uv, void* workspace, size_t ws_bytes, void* stream) {
  int32_t st = check_backward(dims, n_tokens);
  if (st != MTLA_OK) return st;
  if (pe_rows < n_tokens) return fail(MTLA_ERR_INVALID_ARG, "pe_rows=%d < n_tokens=%d", pe_rows, n_tokens);
  CHECK_PTR_ALIGN(w_hyp, 4);
  CHECK_PTR(w_uk);
  CHECK_PTR(w_uv);
  CHECK_PTR_ALIGN(grad_w_hyp, 4);
  CHECK_PTR_ALIGN(grad_w_uk, 4);
  CHECK_PTR_ALIGN(grad_w_uv, 4);
  const BwdWs ws = bwd_ws(dims, n_tokens);
  const bool empty = dims->batch == 0 || n_tokens == 0;
  if (!empty) {
    CHECK_PTR(q_c);
    CHECK_PTR(c);
    CHECK_PTR_ALIGN(pe, 4);
    CHECK_PTR(grad_out);
    CHECK_PTR(grad_q_c);
    CHECK_PTR(grad_c);
    if (dims->d_r > 0) {
      CHECK_PTR(q_r);
      CHECK_PTR(k_r);
      CHECK_PTR(grad_q_r);
      CHECK_PTR(grad_k_r);
    }
    if (!workspace) return fail(MTLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws.total);
    if (!aligned16(workspace)) return fail(MTLA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (ws_bytes < ws.total)
      return fail(MTLA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, ws.total);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = dims->heads, d_h = dims->d_h, dc = dims->d_c, dr = dims->d_r, W = dc + dr;
  const int KV2 = 2 * H * d_h;
  hipError_t e;
  if (empty) {
    // the gradients of the weights are sums over no tokens
    if ((e = mtla::launch_sum_parts(nullptr, 0, gate_rows(dims) * dc, grad_w_hyp, s)) != hipSuccess)
      return hip_status(e, "backward zero-fill launch");
    if ((e = mtla::launch_sum_parts(nullptr, 0, H * d_h * dc, grad_w_uk, s)) != hipSuccess)
      return hip_status(e, "backward zero-fill launch");
    return hip_status(mtla::launch_sum_parts(nullptr, 0, H * d_h * dc, grad_w_uv, s), "backward zero-fill launch");
  }
  const int R = dims->batch * n_tokens;
  mtla::BwdArgs a{};
  a.B = dims->batch;
  a.N = n_tokens;
  a.H = H;
  a.d_h = d_h;
  a.d_c = dc;
  a.d_r = dr;
  a.s = dims->stride_s;
  a.scale = dims->softmax_scale;
  a.q_c = q_c;
  a.q_r = q_r;
  a.c = c;
  a.k_r = k_r;
  a.w_hyp = w_hyp;
  a.pe = pe;
  a.d_o = grad_out;
  a.P = at(workspace, ws.P);
  a.gate = reinterpret_cast<float*>(at(workspace, ws.gate));
  a.KV = at(workspace, ws.KV);
  a.lse = reinterpret_cast<float*>(at(workspace, ws.lse));
  a.D = reinterpret_cast<float*>(at(workspace, ws.D));
  a.dKV = at(workspace, ws.dKV);
  a.dPc = reinterpret_cast<float*>(at(workspace, ws.dPc));
  a.g_q_c = grad_q_c;
  a.g_q_r = grad_q_r;
  a.g_c = grad_c;
  a.g_k_r = grad_k_r;
  a.du = reinterpret_cast<float*>(at(workspace, ws.du));
  a.wh_part = reinterpret_cast<float*>(at(workspace, ws.wh_part));
  a.wh_parts = ws.wh_parts;
  a.wh_stride = gate_stride(dims);
  a.wh_rows = gate_rows(dims);
  const int ldk = KV2 + H * dr;
  // forward recomputation: gates and partial merges, then K^C and V of every token
  if ((e = mtla::launch_bwd_partials(a, dims->dtype, s)) != hipSuccess)
    return hip_status(e, "backward partials launch");
  if (ws.fast) {
    // the forward's own K/V GEMM gives K^C and V of every token; then the
    // MFMA dQ kernel (which also forms lse and D) and the dK/dV kernel
    a.kc = at(workspace, ws.kc);
    a.v = at(workspace, ws.v);
    a.pd = reinterpret_cast<float*>(at(workspace, ws.pd));
    a.dsd = reinterpret_cast<float*>(at(workspace, ws.dsd));
    if ((e = mtla::launch_prefill_kv(a.B, n_tokens, n_tokens, 1, 0, H, d_h, dc, dr, a.P, w_uk, w_uv,
                                     at(workspace, ws.kc), at(workspace, ws.v), false, s)) != hipSuccess)
      return hip_status(e, "backward K/V up-projection launch");
    if ((e = mtla::launch_bwd_attention_mfma(a, s)) != hipSuccess)
      return hip_status(e, "backward attention launch");
  } else {
    mtla::LayerGemmArgs kv{};
    kv.M = R;
    kv.N = KV2;
    kv.K = dc;
    kv.A = a.P;
    kv.lda = W;
    kv.w0 = w_uk;
    kv.n0 = H * d_h;
    kv.w1 = w_uv;
    kv.n1 = H * d_h;
    kv.w2 = w_uv;
    kv.mode = 0;
    kv.out = at(workspace, ws.KV);
    if ((e = mtla::launch_layer_gemm(kv, dims->dtype, s)) != hipSuccess)
      return hip_status(e, "backward K/V up-projection launch");
    // attention backward: dq (with lse and D), then dK^C, dK^R, dV of every key token
    if ((e = mtla::launch_bwd_attention(a, dims->dtype, s)) != hipSuccess)
      return hip_status(e, "backward attention launch");
  }
  // dP^c = [dK^C | dV] [W_UK ; W_UV]
  void* wt = at(workspace, ws.Wt);
  if ((e = mtla::launch_bwd_transpose_w(H * d_h, dc, w_uk, w_uv, wt, dims->dtype, s)) != hipSuccess)
    return hip_status(e, "backward weight transpose launch");
  mtla::LayerGemmArgs dp{};
  dp.M = R;
  dp.N = dc;
  dp.K = KV2;
  dp.A = a.dKV;
  dp.lda = ldk;
  dp.w0 = wt;
  dp.n0 = dc;
  dp.w1 = wt;
  dp.w2 = wt;
  dp.mode = 0;
  dp.out = at(workspace, ws.dPc);
  dp.out_f32 = 1;
  if ((e = mtla::launch_layer_gemm(dp, dims->dtype, s)) != hipSuccess)
    return hip_status(e, "backward dP launch");
  // dW_UK, dW_UV = [dK^C | dV]^T P^c, summed over every token of the batch
  if ((e = mtla::launch_bwd_wgrad(R, KV2, dc, a.dKV, ldk, a.P, W, reinterpret_cast<float*>(at(workspace, ws.wg_part)),
                                  ws.wg_splits, grad_w_uk, H * d_h, grad_w_uv, dims->dtype, s)) != hipSuccess)
    return hip_status(e, "backward weight-gradient launch");
  // reverse in-block sums, gate backward, dc, dk^R and dW_hyp
  if ((e = mtla::launch_bwd_scan(a, dims->dtype, s)) != hipSuccess) return hip_status(e, "backward scan launch");
  return hip_status(mtla::launch_bwd_dwhyp(a, grad_w_hyp, dims->dtype, s), "backward dW_hyp launch");
}

int32_t mtla_debug_stride_mask(int32_t n, int32_t s, uint8_t* mask, void* stream) {
  if (n < 1 || s < 1) return fail(MTLA_ERR_INVALID_ARG, "n=%d, s=%d must be >= 1", n, s);
  if (int64_t(n) * n > kMaxElems) return fail(MTLA_ERR_UNSUPPORTED, "mask too large");
  if (!mask) return fail(MTLA_ERR_INVALID_ARG, "mask is NULL");
  return hip_status(mtla::launch_debug_mask(n, s, mask, static_cast<hipStream_t>(stream)),
                    "debug mask launch");
}

int32_t mtla_debug_slot_limits(int32_t n, int32_t s, int32_t* hi, void* stream) {
  if (n < 1 || s < 1) return fail(MTLA_ERR_INVALID_ARG, "n=%d, s=%d must be >= 1", n, s);
  if (!hi) return fail(MTLA_ERR_INVALID_ARG, "hi is NULL");
  return hip_status(mtla::launch_debug_limits(n, s, hi, static_cast<hipStream_t>(stream)),
                    "debug limits launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Measurement hooks
// ---------------------------------------------------------------------------
int32_t mtla_calib_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!src || !aligned16(src)) return fail(MTLA_ERR_INVALID_ARG, "src is NULL or not 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0) return fail(MTLA_ERR_INVALID_ARG, "bytes=%zu is not a positive multiple of 16", bytes);
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(MTLA_ERR_INVALID_ARG, "workgroups=%d outside 1..2^20", workgroups);
  CHECK_PTR_ALIGN(sink, 4);
  return hip_status(mtla::launch_calib_read(src, bytes, workgroups, sink, static_cast<hipStream_t>(stream)),
                    "stream-read launch");
}

int32_t mtla_calib_mfma(int32_t f16, int32_t workgroups, int32_t iters, float* out, double* flops, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(MTLA_ERR_INVALID_ARG, "workgroups=%d outside 1..2^20", workgroups);
  if (iters < 1) return fail(MTLA_ERR_INVALID_ARG, "iters=%d < 1", iters);
  CHECK_PTR_ALIGN(out, 4);
  if (flops) *flops = mtla::calib_mfma_flops(workgroups, iters);
  return hip_status(mtla::launch_calib_mfma(f16 != 0, workgroups, iters, out, static_cast<hipStream_t>(stream)),
                    "MFMA-loop launch");
}

int32_t mtla_calib_tile_stream(const void* rows, int32_t seqs, int32_t rows_per_seq, int32_t splits, int32_t flags,
                               uint32_t* sink, void* stream) {
  if (!rows || !aligned16(rows)) return fail(MTLA_ERR_INVALID_ARG, "rows is NULL or not 16-byte aligned");
  if (seqs < 1 || seqs > 65535) return fail(MTLA_ERR_INVALID_ARG, "seqs=%d outside 1..65535", seqs);
  if (rows_per_seq < 1 || int64_t(rows_per_seq) * 1152 > INT32_MAX)
    return fail(MTLA_ERR_INVALID_ARG, "rows_per_seq=%d outside 1..%d", rows_per_seq, INT32_MAX / 1152);
  if (splits < 1 || splits > 64) return fail(MTLA_ERR_INVALID_ARG, "splits=%d outside 1..64", splits);
  if (flags & ~3) return fail(MTLA_ERR_INVALID_ARG, "flags=%d has bits other than 0 and 1", flags);
  CHECK_PTR_ALIGN(sink, 4);
  return hip_status(mtla::launch_calib_tile_stream(rows, seqs, rows_per_seq, splits, (flags & 1) != 0,
                                                   (flags & 2) != 0, sink, static_cast<hipStream_t>(stream)),
                    "tile-stream launch");
}

int32_t mtla_calib_load_pattern(int32_t pattern, int32_t workgroups, const void* buf, size_t bytes,
                                uint32_t* cycles, void* stream) {
  if (pattern != 0 && pattern != 1) return fail(MTLA_ERR_INVALID_ARG, "pattern=%d is not 0 or 1", pattern);
  if (workgroups < 1 || workgroups > 65535)
    return fail(MTLA_ERR_INVALID_ARG, "workgroups=%d outside 1..65535", workgroups);
  if (!buf || !aligned16(buf)) return fail(MTLA_ERR_INVALID_ARG, "buf is NULL or not 16-byte aligned");
  if (bytes < 131072 || bytes > (size_t(1) << 31))
    return fail(MTLA_ERR_INVALID_ARG, "bytes=%zu outside 128 KiB..2 GiB", bytes);
  CHECK_PTR_ALIGN(cycles, 4);
  return hip_status(mtla::launch_calib_load_pattern(pattern, workgroups, buf, bytes, cycles,
                                                    static_cast<hipStream_t>(stream)),
                    "load-pattern launch");
}

int32_t mtla_calib_empty(void* stream) {
  return hip_status(mtla::launch_calib_empty(static_cast<hipStream_t>(stream)), "empty-kernel launch");
}
