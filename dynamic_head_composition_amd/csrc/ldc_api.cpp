// C ABI of the Lightweight DC library: argument validation and dispatch.
// Validation happens before any HIP call, so every error path below runs on
// a machine without a GPU.
#include "../../include/ldc.h"

#include <hip/hip_runtime.h>

#include "ldc_internal.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_supported(int dtype, int d) {
  if (dtype == LDC_BF16) return d == 16 || d == 64 || d == 128;
  return d == 16 || d == 64 || d == 128;
}

bool scale_ok(float scale) { return scale > 0.f && scale < 3.0e38f; }  // positive and finite

int check_common(int dtype, int64_t T, int H, int d, int window) {
  if (dtype != LDC_BF16 && dtype != LDC_F32) return LDC_ERR_DTYPE;
  if (T < 0 || H < 1 || window < 1 || window > 128) return LDC_ERR_SHAPE;
  if (d < 1) return LDC_ERR_SHAPE;
  // T*H*d elements must index with 32-bit rows; keep a margin of one tile.
  const int64_t elems = T * (int64_t)H * (int64_t)d;
  if (T > (int64_t)1 << 30 || elems + 512LL * H * d >= ((int64_t)1 << 31)) return LDC_ERR_SHAPE;
  if (!head_dim_supported(dtype, d)) return LDC_ERR_UNSUPPORTED;
  // float32 rows of 128 leave no LDS for the 10-block band's longer halo
  if (dtype == LDC_F32 && d == 128 && window > 113) return LDC_ERR_UNSUPPORTED;
  return LDC_OK;
}

}  // namespace

extern "C" {

int ldc_version(void) { return kVersion; }

const char* ldc_status_str(int status) {
  switch (status) {
    case LDC_OK: return "LDC_OK";
    case LDC_ERR_NULL: return "LDC_ERR_NULL: a required pointer is NULL";
    case LDC_ERR_SHAPE: return "LDC_ERR_SHAPE: size or window out of range";
    case LDC_ERR_DTYPE: return "LDC_ERR_DTYPE: unknown dtype";
    case LDC_ERR_ALIGN: return "LDC_ERR_ALIGN: pointer not 16-byte aligned";
    case LDC_ERR_UNSUPPORTED:
      return "LDC_ERR_UNSUPPORTED: head dim (or, for float32 d=128, a window above 113) not available "
             "for this dtype";
    case LDC_ERR_WORKSPACE: return "LDC_ERR_WORKSPACE: workspace missing or too small";
    case LDC_ERR_HIP: return "LDC_ERR_HIP: a HIP launch failed";
    case LDC_ERR_SCRATCH:
      return "LDC_ERR_SCRATCH: the call needs more workspace than ldc_bwd_noalloc's static scratch "
             "(ldc_bwd_noalloc_max_workspace() bytes)";
    default: return "unknown ldc status";
  }
}

size_t ldc_saved_bytes(int dtype, int64_t T, int H, int d, int window) {
  if (check_common(dtype, T, H, d, window) != LDC_OK) return 0;
  return ldc::saved_band_bytes(T, window) + (size_t)T * (size_t)H * sizeof(float2);
}

// The backward pass's own scratch (the dPbar band), after room for the saved
// state it recomputes when the caller passes none (256-byte aligned).
static size_t bwd_own_bytes(int64_t T, int window) { return ldc::saved_band_bytes(T, window); }
static size_t state_room(size_t saved) { return (saved + 255) & ~(size_t)255; }

size_t ldc_bwd_workspace_bytes(int dtype, int64_t T, int H, int d, int window) {
  if (check_common(dtype, T, H, d, window) != LDC_OK) return 0;
  if (T == 0) return 0;
  return state_room(ldc_saved_bytes(dtype, T, H, d, window)) + bwd_own_bytes(T, window);
}

int ldc_fwd(int dtype, int64_t T, int H, int d, int window, float scale, const void* q,
            const void* k, const void* v, const float* c, const float* g, const int32_t* doc_ids,
            float* o, void* saved, size_t saved_bytes, void* stream) {
  int st = check_common(dtype, T, H, d, window);
  if (st != LDC_OK) return st;
  if (!scale_ok(scale)) return LDC_ERR_SHAPE;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {q, k, v, c, g, doc_ids, o};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  if (saved) {
    if (saved_bytes < ldc_saved_bytes(dtype, T, H, d, window)) return LDC_ERR_WORKSPACE;
    if (!aligned16(saved)) return LDC_ERR_ALIGN;
  }
  uint32_t* band = static_cast<uint32_t*>(saved);
  float2* stats = saved ? reinterpret_cast<float2*>(static_cast<char*>(saved) + ldc::saved_band_bytes(T, window))
                        : nullptr;
  ldc::FwdArgs a{(int)T, H, window, scale, q, k, v, c, g, doc_ids, o, band, stats};
  hipError_t e = ldc::fwd_dispatch(dtype, d, a, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LDC_OK : LDC_ERR_HIP;
}

// Validation shared by the backward entry points (everything but the
// workspace).  On LDC_OK, *need_ws holds the workspace bytes the call needs.
static int bwd_validate(int dtype, int64_t T, int H, int d, int window, float scale,
                        const void* q, const void* k, const void* v, const float* c,
                        const float* g, const int32_t* doc_ids, const void* saved,
                        size_t saved_bytes, const void* dO, float* dq, float* dk, float* dv,
                        float* dc, float* dg, size_t* need_ws) {
  int st = check_common(dtype, T, H, d, window);
  if (st != LDC_OK) return st;
  if (!scale_ok(scale)) return LDC_ERR_SHAPE;
  *need_ws = 0;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {q, k, v, c, g, doc_ids, dO, dq, dk, dv, dc, dg};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  const size_t need_saved = ldc_saved_bytes(dtype, T, H, d, window);
  if (saved) {
    if (saved_bytes < need_saved) return LDC_ERR_WORKSPACE;
    if (!aligned16(saved)) return LDC_ERR_ALIGN;
  }
  // Without saved state the workspace first holds the recomputed state.
  *need_ws = (saved ? 0 : state_room(need_saved)) + bwd_own_bytes(T, window);
  return LDC_OK;
}

// Enqueues the backward kernels on validated arguments and a large enough workspace.
static int bwd_run(int parts, int dtype, int64_t T, int H, int d, int window, float scale,
                   const void* q, const void* k, const void* v, const float* c, const float* g,
                   const int32_t* doc_ids, const void* saved, const void* dO, float* dq,
                   float* dk, float* dv, float* dc, float* dg, char* ws, hipStream_t hs) {
  const size_t need_saved = ldc_saved_bytes(dtype, T, H, d, window);
  const void* state = saved;
  if (!saved) {
    state = ws;
    ws += state_room(need_saved);
    // The query-side kernel is the first reader of the state: recompute it
    // there (the forward's score phase, band and statistics only).
    if (parts & 1) {
      ldc::FwdArgs f{(int)T, H, window, scale, q, k, v, c, g, doc_ids, nullptr,
                     static_cast<uint32_t*>(const_cast<void*>(state)),
                     reinterpret_cast<float2*>(static_cast<char*>(const_cast<void*>(state)) +
                                               ldc::saved_band_bytes(T, window))};
      if (ldc::fwd_dispatch(dtype, d, f, false, hs) != hipSuccess) return LDC_ERR_HIP;
    }
  }
  const uint32_t* band = static_cast<const uint32_t*>(state);
  const float2* stats =
      reinterpret_cast<const float2*>(static_cast<const char*>(state) + ldc::saved_band_bytes(T, window));
  ldc::BwdArgs a{(int)T, H, window, scale, q, k, v, dO, c, g, doc_ids,
                 dq, dk, dv, dc, dg, band, stats, reinterpret_cast<float*>(ws)};
  hipError_t e = ldc::bwd_dispatch(dtype, d, a, parts, hs);
  return e == hipSuccess ? LDC_OK : LDC_ERR_HIP;
}

static int bwd_parts(int parts, int dtype, int64_t T, int H, int d, int window, float scale,
                     const void* q, const void* k, const void* v, const float* c, const float* g,
                     const int32_t* doc_ids, const void* saved, size_t saved_bytes, const void* dO,
                     float* dq, float* dk, float* dv, float* dc, float* dg, void* workspace,
                     size_t workspace_bytes, void* stream) {
  size_t need_ws = 0;
  int st = bwd_validate(dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, saved, saved_bytes,
                        dO, dq, dk, dv, dc, dg, &need_ws);
  if (st != LDC_OK || T == 0) return st;
  if (!workspace || workspace_bytes < need_ws) return LDC_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LDC_ERR_ALIGN;
  return bwd_run(parts, dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, saved, dO, dq, dk,
                 dv, dc, dg, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

#define LDC_BWD_PARAMS                                                                          \
  int dtype, int64_t T, int H, int d, int window, float scale, const void *q, const void *k,    \
      const void *v, const float *c, const float *g, const int32_t *doc_ids, const void *saved, \
      size_t saved_bytes, const void *dO, float *dq, float *dk, float *dv, float *dc, float *dg, \
      void *workspace, size_t workspace_bytes, void *stream
#define LDC_BWD_ARGS                                                                           \
  dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, saved, saved_bytes, dO, dq, dk, dv, dc, \
      dg, workspace, workspace_bytes, stream

int ldc_bwd(LDC_BWD_PARAMS) { return bwd_parts(3, LDC_BWD_ARGS); }
int ldc_bwd_q(LDC_BWD_PARAMS) { return bwd_parts(1, LDC_BWD_ARGS); }
int ldc_bwd_kv(LDC_BWD_PARAMS) { return bwd_parts(2, LDC_BWD_ARGS); }

int ldc_bwd_noalloc(int dtype, int64_t T, int H, int d, int window, float scale, const void* q,
                    const void* k, const void* v, const float* c, const float* g,
                    const int32_t* doc_ids, const void* saved, size_t saved_bytes, const void* dO,
                    float* dq, float* dk, float* dv, float* dc, float* dg, void* stream) {
  size_t need_ws = 0;
  int st = bwd_validate(dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, saved, saved_bytes,
                        dO, dq, dk, dv, dc, dg, &need_ws);
  if (st != LDC_OK || T == 0) return st;
  if (need_ws > ldc::kStaticScratchBytes) return LDC_ERR_SCRATCH;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // The stream's device decides which copy of the static scratch the kernels use.
  int dev = 0;
  if (hipStreamGetDevice(hs, &dev) != hipSuccess) return LDC_ERR_HIP;
  void* ws = nullptr;
  if (ldc::static_scratch(dev, &ws) != hipSuccess) return LDC_ERR_HIP;
  return bwd_run(3, dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, saved, dO, dq, dk, dv,
                 dc, dg, static_cast<char*>(ws), hs);
}

size_t ldc_bwd_noalloc_max_workspace(void) { return ldc::kStaticScratchBytes; }

}  // extern "C"
