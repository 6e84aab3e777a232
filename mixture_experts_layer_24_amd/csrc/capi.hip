// C ABI entry points: argument validation on the host, then kernel launches.
// Nothing here allocates or synchronizes; see include/moe.h for the contract.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQ(cond, code, ...) \
  do {                        \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)
#define PTR(p) REQ((p) != nullptr && al16(p), MOE_ERR_ARG, "%s must be a non-NULL 16-byte aligned pointer", #p)
#define OPT(p) REQ((p) == nullptr || al16(p), MOE_ERR_ARG, "%s must be 16-byte aligned", #p)

int launched(int rc, const char* what) {
  if (rc == MOE_OK) return MOE_OK;
  if (rc == MOE_ERR_HIP) return fail(rc, "%s: HIP launch failed (%s)", what, moe_launch::last_hip_error());
  return fail(rc, "%s failed", what);
}

thread_local const char* g_hip_err = "";

size_t esize(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

}  // namespace

namespace moe_launch {
void clear_status() { (void)hipGetLastError(); }
int launch_status() {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) return MOE_OK;
  g_hip_err = hipGetErrorString(e);
  return MOE_ERR_HIP;
}
const char* last_hip_error() { return g_hip_err; }

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
}  // namespace moe_launch

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_version(void) { return 4; }

size_t moe_packed_weight_bytes(int which, int E, int h, int h_ffn, int dtype) {
  if (E <= 0 || h <= 0 || h_ffn <= 0 || dtype < MOE_F32 || dtype > MOE_FP8_E4M3) return 0;
  size_t e = size_t(E), hh = size_t(h), hf = size_t(h_ffn);
  switch (which) {
    case 0: return e * 2 * hf * hh * esize(dtype);
    case 1: return e * hh * hf * esize(dtype);
    case 2: return dtype == MOE_FP8_E4M3 ? e * 2 * hf * 4 : 0;
    case 3: return dtype == MOE_FP8_E4M3 ? e * hh * 4 : 0;
    case 4: return dtype == MOE_F32 ? 0 : e * hh * 2 * hf * esize(dtype);
    case 5: return dtype == MOE_F32 ? 0 : e * hf * hh * esize(dtype);
    case 6: return dtype == MOE_FP8_E4M3 ? e * hh * 4 : 0;
    case 7: return dtype == MOE_FP8_E4M3 ? e * hf * 4 : 0;
  }
  return 0;
}

int moe_pack_weights(const void* w1, const void* w3, const void* w2, int in_dtype, int E, int h,
                     int h_ffn, int out_dtype, void* w13, void* w2_packed, float* w13_scale,
                     float* w2_scale, void* w13_bwd, void* w2_bwd, float* w13_bwd_scale,
                     float* w2_bwd_scale, void* stream) {
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(h > 0 && h % 128 == 0 && h_ffn > 0 && h_ffn % 128 == 0, MOE_ERR_SHAPE,
      "h=%d and h_ffn=%d must be positive multiples of 128", h, h_ffn);
  bool ok = (in_dtype == MOE_F32 && out_dtype == MOE_F32) ||
            (in_dtype == MOE_BF16 && (out_dtype == MOE_BF16 || out_dtype == MOE_FP8_E4M3));
  REQ(ok, MOE_ERR_DTYPE, "unsupported pack %d -> %d", in_dtype, out_dtype);
  PTR(w1); PTR(w3); PTR(w2); PTR(w13); PTR(w2_packed);
  if (out_dtype == MOE_FP8_E4M3) { PTR(w13_scale); PTR(w2_scale); }
  OPT(w13_bwd); OPT(w2_bwd); OPT(w13_bwd_scale); OPT(w2_bwd_scale);
  REQ((w13_bwd == nullptr && w2_bwd == nullptr) || out_dtype != MOE_F32, MOE_ERR_DTYPE,
      "backward weight layouts are produced for bf16 and fp8");
  if (out_dtype == MOE_FP8_E4M3) {
    REQ(w13_bwd == nullptr || w13_bwd_scale != nullptr, MOE_ERR_ARG, "FP8 w13_bwd needs w13_bwd_scale");
    REQ(w2_bwd == nullptr || w2_bwd_scale != nullptr, MOE_ERR_ARG, "FP8 w2_bwd needs w2_bwd_scale");
  }
  moe_launch::clear_status();
  return launched(moe_launch::pack_weights(w1, w3, w2, in_dtype, E, h, h_ffn, out_dtype, w13,
                                           w2_packed, w13_scale, w2_scale, w13_bwd, w2_bwd,
                                           w13_bwd_scale, w2_bwd_scale, (hipStream_t)stream),
                  "moe_pack_weights");
}

int moe_route(const void* x, const void* w_gate, const float* bias, float* logits, int T, int h,
              int E, int k, int dtype, int32_t* topk_idx, float* topk_w, void* stream) {
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(k >= 1 && k <= E && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  PTR(topk_idx); PTR(topk_w); OPT(bias); OPT(logits);
  if (x == nullptr) {
    REQ(logits != nullptr, MOE_ERR_ARG, "logits must be given when x is NULL");
  } else {
    PTR(x); PTR(w_gate);
    REQ(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_DTYPE, "router dtype %d unsupported", dtype);
    REQ(h > 0 && (dtype == MOE_F32 || h % 64 == 0), MOE_ERR_SHAPE,
        "h=%d must be a positive multiple of 64 for bf16", h);
  }
  if (T == 0) return MOE_OK;
  moe_launch::clear_status();
  return launched(moe_launch::route(x, w_gate, bias, logits, T, h, E, k, dtype, topk_idx, topk_w,
                                    (hipStream_t)stream),
                  "moe_route");
}

size_t moe_permute_workspace_size(int T, int E, int k) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return moe_launch::index_ws_bytes(T, E);
}

}  // extern "C"

// Scratch of moe_permute_noalloc: the index builder's per-block histograms,
// in a file-scope device array instead of a caller's workspace.  Each device
// holds its own copy until the process ends.  Host code uses the address
// hipGetSymbolAddress returns for the current device, never the array's name.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// This device's copy of `scratch`, looked up on the first call on the device.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  REQ(e == hipSuccess && dev >= 0 && dev < 64, MOE_ERR_HIP, "no usable current device (%s)",
      hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    REQ(e == hipSuccess && p != nullptr, MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s",
        dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_permute_noalloc(const void* src, int src_dtype, const int32_t* topk_idx, const float* row_scale,
                        int T, int h, int E, int k, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                        int32_t* src_tok, void* dst, int dst_dtype, float* dst_scale, void* stream) {
  if (topk_idx == nullptr)  // no index to build: moe_permute needs no workspace then
    return moe_permute(src, src_dtype, topk_idx, row_scale, T, h, E, k, counts, offsets, dst_row,
                       src_tok, dst, dst_dtype, dst_scale, nullptr, 0, stream);
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  const size_t need = moe_launch::index_ws_bytes(T, E);
  REQ(need <= MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
      "moe_permute_noalloc: T=%d, E=%d need %zu bytes of scratch, more than its %d", T, E, need,
      MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc) return rc;
  return moe_permute(src, src_dtype, topk_idx, row_scale, T, h, E, k, counts, offsets, dst_row,
                     src_tok, dst, dst_dtype, dst_scale, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_permute(const void* src, int src_dtype, const int32_t* topk_idx, const float* row_scale,
                int T, int h, int E, int k, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                int32_t* src_tok, void* dst, int dst_dtype, float* dst_scale, void* ws,
                size_t ws_bytes, void* stream) {
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(k >= 1 && k <= E && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  REQ(h > 0 && h % 8 == 0, MOE_ERR_SHAPE, "h=%d must be a positive multiple of 8", h);
  bool ok = (src_dtype == MOE_F32 && dst_dtype == MOE_F32) ||
            (src_dtype == MOE_BF16 && (dst_dtype == MOE_BF16 || dst_dtype == MOE_FP8_E4M3));
  REQ(ok, MOE_ERR_DTYPE, "unsupported permute %d -> %d", src_dtype, dst_dtype);
  if (dst_dtype == MOE_FP8_E4M3) PTR(dst_scale);
  PTR(src); PTR(dst); PTR(dst_row); OPT(row_scale);
  if (topk_idx) {
    PTR(topk_idx); PTR(counts); PTR(offsets); PTR(src_tok);
    size_t need = moe_launch::index_ws_bytes(T, E);
    REQ(T == 0 || (ws != nullptr && ws_bytes >= need), MOE_ERR_WORKSPACE,
        "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : size_t(0));
    OPT(ws);
    moe_launch::clear_status();
    int rc = moe_launch::index_build(topk_idx, T, E, k, counts, offsets, dst_row, src_tok, ws,
                                     (hipStream_t)stream);
    if (rc) return launched(rc, "moe_permute (index)");
  }
  if (T == 0) return MOE_OK;
  moe_launch::clear_status();
  return launched(moe_launch::permute_rows(src, src_dtype, dst_row, row_scale, T, h, k, dst,
                                           dst_dtype, dst_scale, (hipStream_t)stream),
                  "moe_permute");
}

size_t moe_permute_local_workspace_size(int T, int e_count, int k) {
  if (T < 0 || e_count < 1 || k < 1) return 0;
  return ((size_t(T) * k * 4 + 255) & ~size_t(255)) + moe_launch::index_ws_bytes(T, e_count);
}

int moe_permute_local(const void* src, int src_dtype, const int32_t* topk_idx, const float* row_scale,
                      int T, int h, int E, int k, int e_lo, int e_count, int32_t* counts,
                      int32_t* offsets, int32_t* dst_row, int32_t* src_tok, void* dst, int dst_dtype,
                      float* dst_scale, void* ws, size_t ws_bytes, void* stream) {
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(k >= 1 && k <= E && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  REQ(e_count >= 1 && e_lo >= 0 && e_lo + e_count <= E, MOE_ERR_ARG,
      "expert range [%d, %d) not inside [0, %d)", e_lo, e_lo + e_count, E);
  PTR(topk_idx);
  const size_t need = moe_permute_local_workspace_size(T, e_count, k);
  REQ(T == 0 || (ws != nullptr && ws_bytes >= need), MOE_ERR_WORKSPACE,
      "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : size_t(0));
  if (T == 0)  // the empty batch still clears counts / offsets
    return moe_permute(src, src_dtype, topk_idx, row_scale, 0, h, e_count, e_count < k ? e_count : k,
                       counts, offsets, dst_row, src_tok, dst, dst_dtype, dst_scale, ws, ws_bytes,
                       stream);
  // k may exceed e_count (a token meets at most one slot per local expert):
  // the share is validated with the global E
  REQ(h > 0 && h % 8 == 0, MOE_ERR_SHAPE, "h=%d must be a positive multiple of 8", h);
  bool ok = (src_dtype == MOE_F32 && dst_dtype == MOE_F32) ||
            (src_dtype == MOE_BF16 && (dst_dtype == MOE_BF16 || dst_dtype == MOE_FP8_E4M3));
  REQ(ok, MOE_ERR_DTYPE, "unsupported permute %d -> %d", src_dtype, dst_dtype);
  if (dst_dtype == MOE_FP8_E4M3) PTR(dst_scale);
  PTR(src); PTR(dst); PTR(dst_row); OPT(row_scale); PTR(counts); PTR(offsets); PTR(src_tok);
  unsigned char* w = static_cast<unsigned char*>(ws);
  int32_t* local = reinterpret_cast<int32_t*>(w);
  const size_t lb = (size_t(T) * k * 4 + 255) & ~size_t(255);
  moe_launch::clear_status();
  int rc = moe_launch::local_ids(topk_idx, T * k, e_lo, e_count, local, (hipStream_t)stream);
  if (rc) return launched(rc, "moe_permute_local (ids)");
  rc = moe_launch::index_build(local, T, e_count, k, counts, offsets, dst_row, src_tok, w + lb,
                               (hipStream_t)stream);
  if (rc) return launched(rc, "moe_permute_local (index)");
  return launched(moe_launch::permute_rows(src, src_dtype, dst_row, row_scale, T, h, k, dst, dst_dtype,
                                           dst_scale, (hipStream_t)stream),
                  "moe_permute_local");
}

size_t moe_capacity_drop_workspace_size(int T, int E, int k) {
  if (T <= 0 || E < 1 || k < 1) return 0;
  return moe_launch::capacity_ws_bytes(T, E, k);
}

int moe_capacity_drop(const int32_t* topk_idx, const float* logits, int T, int E, int k, int group,
                      int capacity, int32_t* topk_idx_out, void* ws, size_t ws_bytes, void* stream) {
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(k >= 1 && k <= E && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  REQ(group >= 1 && E % group == 0, MOE_ERR_ARG, "group=%d must divide E=%d", group, E);
  REQ(capacity >= 0, MOE_ERR_ARG, "capacity=%d is negative", capacity);
  PTR(topk_idx); PTR(logits); PTR(topk_idx_out);
  if (T == 0) return MOE_OK;
  const size_t need = moe_launch::capacity_ws_bytes(T, E, k);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  moe_launch::clear_status();
  return launched(moe_launch::capacity_drop(topk_idx, logits, T, E, k, group, capacity, topk_idx_out,
                                            ws, (hipStream_t)stream),
                  "moe_capacity_drop");
}

static int check_weights(const moe_weights* W) {
  REQ(W != nullptr, MOE_ERR_ARG, "W must not be NULL");
  REQ(W->dtype == MOE_F32 || W->dtype == MOE_BF16 || W->dtype == MOE_FP8_E4M3, MOE_ERR_DTYPE,
      "weight dtype %d unsupported", W->dtype);
  REQ(W->E >= 1 && W->E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", W->E,
      MOE_MAX_EXPERTS);
  REQ(W->h > 0 && W->h % 128 == 0 && W->h_ffn > 0 && W->h_ffn % 128 == 0, MOE_ERR_SHAPE,
      "h=%d and h_ffn=%d must be positive multiples of 128", W->h, W->h_ffn);
  const void* w13 = W->w13;
  const void* w2 = W->w2;
  PTR(w13); PTR(w2);
  if (W->dtype == MOE_FP8_E4M3) {
    const float* w13_scale = W->w13_scale;
    const float* w2_scale = W->w2_scale;
    PTR(w13_scale); PTR(w2_scale);
  }
  return MOE_OK;
}

size_t moe_grouped_workspace_size(int rows, int h, int h_ffn, int E, int dtype) {
  if (rows < 0 || h <= 0 || h_ffn <= 0 || E < 1) return 0;
  return moe_launch::grouped_fwd_ws_bytes(rows, h, h_ffn, E, dtype);
}

int moe_grouped_swiglu_fwd(const void* xp, const float* xp_scale, const moe_weights* W,
                           const int32_t* offsets, int rows, void* h13_save, void* yp, int yp_dtype,
                           void* ws, size_t ws_bytes, void* stream) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQ(yp_dtype == MOE_F32 || (yp_dtype == MOE_BF16 && W->dtype != MOE_F32), MOE_ERR_DTYPE,
      "yp_dtype %d with weight dtype %d (fp32 always; bf16 with bf16 or fp8 weights)", yp_dtype,
      int(W->dtype));
  REQ(rows >= 0, MOE_ERR_ARG, "rows=%d is negative", rows);
  PTR(xp); PTR(offsets); PTR(yp); OPT(h13_save);
  if (W->dtype == MOE_FP8_E4M3) PTR(xp_scale);
  REQ(h13_save == nullptr || W->dtype != MOE_F32, MOE_ERR_DTYPE,
      "h13_save is only supported with bf16 and fp8 weights");
  if (rows == 0) return MOE_OK;
  size_t need = moe_launch::grouped_fwd_ws_bytes(rows, W->h, W->h_ffn, W->E, W->dtype);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  OPT(ws);
  moe_launch::clear_status();
  return launched(moe_launch::grouped_fwd(xp, xp_scale, W, offsets, rows, h13_save, yp, yp_dtype,
                                          ws, (hipStream_t)stream),
                  "moe_grouped_swiglu_fwd");
}

size_t moe_grouped_bwd_workspace_size(int rows, int h, int h_ffn, int E, int dtype) {
  if (rows < 0 || h <= 0 || h_ffn <= 0 || E < 1) return 0;
  return moe_launch::grouped_bwd_ws_bytes(rows, h, h_ffn, E, dtype);
}

int moe_grouped_swiglu_bwd(const void* dyp, const void* xp, const void* h13_save,
                           const moe_weights* W, const int32_t* offsets, int rows, void* dxp,
                           float* dw1, float* dw3, float* dw2, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQ(W->dtype == MOE_BF16, MOE_ERR_DTYPE, "backward needs bf16 weights");
  {
    const void* w13_bwd = W->w13_bwd;
    const void* w2_bwd = W->w2_bwd;
    PTR(w13_bwd); PTR(w2_bwd);
  }
  REQ(rows >= 0, MOE_ERR_ARG, "rows=%d is negative", rows);
  PTR(dyp); PTR(xp); PTR(h13_save); PTR(offsets); PTR(dxp); PTR(dw1); PTR(dw3); PTR(dw2);
  size_t need = moe_launch::grouped_bwd_ws_bytes(rows, W->h, W->h_ffn, W->E, W->dtype);
  REQ(need == 0 || (ws != nullptr && ws_bytes >= need), MOE_ERR_WORKSPACE,
      "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : size_t(0));
  OPT(ws);
  moe_launch::clear_status();
  return launched(moe_launch::grouped_bwd(dyp, xp, h13_save, W, offsets, rows, dxp, dw1, dw3, dw2,
                                          ws, (hipStream_t)stream),
                  "moe_grouped_swiglu_bwd");
}

int moe_combine(const void* yp, int yp_dtype, const int32_t* dst_row, const float* topk_w, int T,
                int h, int k, void* y, int y_dtype, void* stream) {
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(k >= 1 && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  REQ(h > 0 && h % 8 == 0, MOE_ERR_SHAPE, "h=%d must be a positive multiple of 8", h);
  REQ((yp_dtype == MOE_F32 || yp_dtype == MOE_BF16) && (y_dtype == MOE_F32 || y_dtype == MOE_BF16),
      MOE_ERR_DTYPE, "combine dtypes %d -> %d unsupported", yp_dtype, y_dtype);
  PTR(yp); PTR(dst_row); PTR(y); OPT(topk_w);
  if (T == 0) return MOE_OK;
  moe_launch::clear_status();
  return launched(moe_launch::combine_rows(yp, yp_dtype, dst_row, topk_w, T, h, k, y, y_dtype,
                                           (hipStream_t)stream),
                  "moe_combine");
}

size_t moe_grouped_bwd_fp8_workspace_size(int rows, int h, int h_ffn, int E) {
  if (rows < 0 || h <= 0 || h_ffn <= 0 || E <= 0) return 0;
  return moe_launch::grouped_bwd_fp8_ws_bytes(rows > 0 ? rows : 1, h, h_ffn, E);
}

int moe_grouped_swiglu_bwd_fp8(const void* dyp_q, const float* dyp_scale, const void* dyp,
                               const void* xp, const void* h13_save, const moe_weights* W,
                               const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3,
                               float* dw2, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQ(W->dtype == MOE_FP8_E4M3, MOE_ERR_DTYPE, "the FP8 backward needs FP8 weights");
  REQ(W->w13_bwd && W->w2_bwd && W->w13_bwd_scale && W->w2_bwd_scale, MOE_ERR_ARG,
      "FP8 backward weight layouts and scales are required");
  REQ(rows >= 0, MOE_ERR_ARG, "rows=%d is negative", rows);
  PTR(dyp_q); PTR(dyp_scale); PTR(dyp); PTR(xp); PTR(h13_save); PTR(offsets); PTR(dxp);
  PTR(dw1); PTR(dw3); PTR(dw2);
  const size_t need = moe_launch::grouped_bwd_fp8_ws_bytes(rows > 0 ? rows : 1, W->h, W->h_ffn, W->E);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  moe_launch::clear_status();
  return launched(moe_launch::grouped_bwd_fp8(dyp_q, dyp_scale, dyp, xp, h13_save, W, offsets, rows,
                                              dxp, dw1, dw3, dw2, ws, (hipStream_t)stream),
                  "moe_grouped_swiglu_bwd_fp8");
}

int moe_grouped_swiglu_bwd_fp8_tok(const void* dyp_q, const float* dyp_scale, const void* dy,
                                   const void* x, const int32_t* dst_row, const float* topk_w, int T,
                                   int k, const void* h13_save, const moe_weights* W,
                                   const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3,
                                   float* dw2, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQ(W->dtype == MOE_FP8_E4M3, MOE_ERR_DTYPE, "the FP8 backward needs FP8 weights");
  REQ(W->w13_bwd && W->w2_bwd && W->w13_bwd_scale && W->w2_bwd_scale, MOE_ERR_ARG,
      "FP8 backward weight layouts and scales are required");
  REQ(rows >= 0, MOE_ERR_ARG, "rows=%d is negative", rows);
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(k >= 1 && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, %d]", k, MOE_MAX_TOPK);
  REQ(rows <= T * k, MOE_ERR_ARG, "rows=%d exceeds T*k=%d", rows, T * k);
  PTR(dyp_q); PTR(dyp_scale); PTR(dy); PTR(x); PTR(dst_row); PTR(topk_w); PTR(h13_save); PTR(offsets);
  PTR(dxp); PTR(dw1); PTR(dw3); PTR(dw2);
  const size_t need = moe_launch::grouped_bwd_fp8_ws_bytes(rows > 0 ? rows : 1, W->h, W->h_ffn, W->E);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  moe_launch::clear_status();
  return launched(moe_launch::grouped_bwd_fp8(dyp_q, dyp_scale, dy, x, h13_save, W, offsets, rows, dxp,
                                              dw1, dw3, dw2, ws, (hipStream_t)stream, dst_row, topk_w,
                                              T, k),
                  "moe_grouped_swiglu_bwd_fp8_tok");
}

size_t moe_dispatch_swiglu_fwd_workspace_size(int T, int k, int h, int h_ffn, int E) {
  if (T < 0 || k < 1 || h <= 0 || h_ffn <= 0 || E < 1) return 0;
  return moe_launch::arrival_ws_bytes(T, k, h, h_ffn, E);
}

static int dispatch_swiglu_fwd_checked(const void* x, const int32_t* topk_idx, int T, int k,
                                       int32_t* counts, int32_t* offsets, int32_t* dst_row,
                                       int32_t* src_tok, const moe_weights* W, void* xp, void* h13_save,
                                       void* yp, int yp_dtype, int32_t* status, void* ws, size_t ws_bytes,
                                       void* stream, int spin_limit, bool copy, const char* name) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQ(W->dtype == MOE_BF16, MOE_ERR_DTYPE, "the tile-arrival forward needs BF16 weights");
  REQ(yp_dtype == MOE_BF16 || yp_dtype == MOE_F32, MOE_ERR_DTYPE, "yp dtype %d unsupported", yp_dtype);
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(k >= 1 && k <= W->E && k <= MOE_MAX_TOPK, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  PTR(x); PTR(topk_idx); PTR(counts); PTR(offsets); PTR(dst_row); PTR(src_tok); PTR(xp); PTR(yp);
  PTR(status); OPT(h13_save);
  const size_t need = moe_launch::arrival_ws_bytes(T, k, W->h, W->h_ffn, W->E);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  moe_launch::clear_status();
  return launched(moe_launch::dispatch_swiglu_fwd(x, topk_idx, T, k, counts, offsets, dst_row, src_tok, W,
                                                  xp, h13_save, yp, yp_dtype == MOE_F32, status, ws,
                                                  (hipStream_t)stream, spin_limit, copy),
                  name);
}

int moe_dispatch_swiglu_fwd(const void* x, const int32_t* topk_idx, int T, int k, int32_t* counts,
                            int32_t* offsets, int32_t* dst_row, int32_t* src_tok, const moe_weights* W,
                            void* xp, void* h13_save, void* yp, int yp_dtype, int32_t* status, void* ws,
                            size_t ws_bytes, void* stream) {
  return dispatch_swiglu_fwd_checked(x, topk_idx, T, k, counts, offsets, dst_row, src_tok, W, xp, h13_save,
                                     yp, yp_dtype, status, ws, ws_bytes, stream, 1 << 20, true,
                                     "moe_dispatch_swiglu_fwd");
}

int moe_dispatch_swiglu_fwd_wait_selftest(const void* x, const int32_t* topk_idx, int T, int k,
                                          int32_t* counts, int32_t* offsets, int32_t* dst_row,
                                          int32_t* src_tok, const moe_weights* W, void* xp,
                                          void* h13_save, void* yp, int yp_dtype, int32_t* status,
                                          void* ws, size_t ws_bytes, void* stream) {
  return dispatch_swiglu_fwd_checked(x, topk_idx, T, k, counts, offsets, dst_row, src_tok, W, xp, h13_save,
                                     yp, yp_dtype, status, ws, ws_bytes, stream, 64, false,
                                     "moe_dispatch_swiglu_fwd_wait_selftest");
}

size_t moe_router_bwd_workspace_size(int T, int h, int E) {
  if (T <= 0 || h <= 0 || E <= 0) return 0;
  return moe_launch::router_bwd_ws_bytes(T, h, E);
}

int moe_router_bwd(const void* dy, const void* yp, int yp_dtype, const int32_t* dst_row,
                   const int32_t* topk_idx,
                   const float* topk_w, const float* logits, const int32_t* counts, int T, int h,
                   int E, int k, float alpha, int dtype, const void* x, const void* w_gate,
                   const float* dx_in, void* dx, float* dlogits, float* dw_gate, float* dbias,
                   void* ws, size_t ws_bytes, void* stream) {
  REQ(T >= 0, MOE_ERR_ARG, "T=%d is negative", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(k >= 1 && k <= MOE_MAX_TOPK && k <= E, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  REQ(h > 0 && h % 64 == 0, MOE_ERR_SHAPE, "h=%d must be a positive multiple of 64", h);
  REQ(dtype == MOE_F32 || dtype == MOE_BF16, MOE_ERR_DTYPE, "router backward dtype %d unsupported",
      dtype);
  REQ(yp_dtype == MOE_F32 || yp_dtype == MOE_BF16, MOE_ERR_DTYPE, "yp dtype %d unsupported", yp_dtype);
  REQ(alpha == alpha, MOE_ERR_ARG, "alpha is NaN");
  PTR(dy); PTR(yp); PTR(dst_row); PTR(topk_idx); PTR(topk_w); PTR(logits); PTR(counts);
  PTR(x); PTR(w_gate); PTR(dx); PTR(dw_gate); OPT(dx_in); OPT(dlogits); OPT(dbias);
  REQ(static_cast<const void*>(dx_in) != dx, MOE_ERR_ARG, "dx may not alias dx_in");
  if (T == 0) return MOE_OK;
  const size_t need = moe_launch::router_bwd_ws_bytes(T, h, E);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  moe_launch::clear_status();
  return launched(moe_launch::router_bwd(dy, yp, yp_dtype, dst_row, topk_idx, topk_w, logits, counts, T, h, E,
                                         k, alpha, dtype, x, w_gate, dx_in, dx, dlogits, dw_gate,
                                         dbias, ws, (hipStream_t)stream),
                  "moe_router_bwd");
}

size_t moe_router_aux_workspace_size(int T, int E) {
  if (T <= 0 || E <= 0) return 0;
  return moe_launch::router_aux_ws_bytes(T, E);
}

int moe_router_aux_loss(const float* logits, const int32_t* counts, int T, int E, int k,
                        float alpha, float* loss, void* ws, size_t ws_bytes, void* stream) {
  REQ(T >= 1, MOE_ERR_ARG, "T=%d must be positive", T);
  REQ(E >= 1 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
  REQ(k >= 1 && k <= MOE_MAX_TOPK && k <= E, MOE_ERR_ARG, "k=%d outside [1, min(E, %d)]", k,
      MOE_MAX_TOPK);
  PTR(logits); PTR(counts); PTR(loss);
  const size_t need = moe_launch::router_aux_ws_bytes(T, E);
  REQ(ws != nullptr && ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
      need, ws ? ws_bytes : size_t(0));
  moe_launch::clear_status();
  return launched(moe_launch::router_aux(logits, counts, T, E, k, alpha, loss, ws, (hipStream_t)stream),
                  "moe_router_aux_loss");
}

int moe_fp8_convert_selftest(unsigned long long* mismatches, void* stream) {
  PTR(mismatches);
  moe_launch::clear_status();
  return launched(moe_launch::fp8_convert_selftest(mismatches, (hipStream_t)stream),
                  "moe_fp8_convert_selftest");
}

}  // extern "C"
