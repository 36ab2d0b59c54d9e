// C ABI of the DCMHA composition: argument validation and dispatch.  Every
// validation precedes any HIP call, so the error paths run without a GPU.
#include "../../include/dcmha.h"

#include <hip/hip_runtime.h>

#include "dcmha_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool scale_ok(float scale) { return scale > 0.f && scale < 3.0e38f; }

int check_common(int dtype, int64_t T, int H, int d, int window) {
  if (dtype != LDC_BF16 && dtype != LDC_F32) return LDC_ERR_DTYPE;
  if (T < 0 || H < 1 || window < 1 || window > 113 || d < 1) return LDC_ERR_SHAPE;
  const int64_t elems = T * (int64_t)H * (int64_t)d;
  if (T > (int64_t)1 << 30 || elems + 512LL * H * d >= ((int64_t)1 << 31)) return LDC_ERR_SHAPE;
  if (H > ldc::kDcMaxHeads) return LDC_ERR_UNSUPPORTED;
  if (dtype == LDC_BF16 ? !(d == 64 || d == 128) : d != 64) return LDC_ERR_UNSUPPORTED;
  return LDC_OK;
}

size_t room(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

size_t dcmha_saved_bytes(int dtype, int64_t T, int H, int d, int window) {
  if (check_common(dtype, T, H, d, window) != LDC_OK) return 0;
  return 2 * ldc::dc_bands_bytes(T, H);  // P bands, then R bands
}

size_t dcmha_bwd_workspace_bytes(int dtype, int64_t T, int H, int d, int window) {
  if (check_common(dtype, T, H, d, window) != LDC_OK || T == 0) return 0;
  return room(dcmha_saved_bytes(dtype, T, H, d, window)) + ldc::dc_bands_bytes(T, H);
}

int dcmha_fwd(int dtype, int64_t T, int H, int d, int window, float scale, const void* q,
              const void* k, const void* v, const float* cs, const float* cw,
              const int32_t* doc_ids, float* o, void* saved, size_t saved_bytes, void* stream) {
  int st = check_common(dtype, T, H, d, window);
  if (st != LDC_OK) return st;
  if (!scale_ok(scale)) return LDC_ERR_SHAPE;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {q, k, v, cs, cw, doc_ids, o};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  if (saved) {
    if (saved_bytes < dcmha_saved_bytes(dtype, T, H, d, window)) return LDC_ERR_WORKSPACE;
    if (!aligned16(saved)) return LDC_ERR_ALIGN;
  }
  uint32_t* pband = static_cast<uint32_t*>(saved);
  uint32_t* rband = saved ? pband + ldc::dc_bands_bytes(T, H) / 4 : nullptr;
  ldc::DcFwdArgs a{(int)T, H, window, scale, q, k, v, cs, cw, doc_ids, o, pband, rband};
  return ldc::dcmha_fwd_dispatch(dtype, d, a, true, static_cast<hipStream_t>(stream)) == hipSuccess
             ? LDC_OK
             : LDC_ERR_HIP;
}

static int bwd_parts(int parts, int dtype, int64_t T, int H, int d, int window, float scale,
                     const void* q, const void* k, const void* v, const float* cs, const float* cw,
                     const int32_t* doc_ids, const void* saved, size_t saved_bytes, const void* dO,
                     float* dq, float* dk, float* dv, float* dcs, float* dcw, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_common(dtype, T, H, d, window);
  if (st != LDC_OK) return st;
  if (!scale_ok(scale)) return LDC_ERR_SHAPE;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {q, k, v, cs, cw, doc_ids, dO, dq, dk, dv, dcs, dcw};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  const size_t need_saved = dcmha_saved_bytes(dtype, T, H, d, window);
  if (saved) {
    if (saved_bytes < need_saved) return LDC_ERR_WORKSPACE;
    if (!aligned16(saved)) return LDC_ERR_ALIGN;
  }
  const size_t need_ws = (saved ? 0 : room(need_saved)) + ldc::dc_bands_bytes(T, H);
  if (!workspace || workspace_bytes < need_ws) return LDC_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LDC_ERR_ALIGN;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const uint32_t* state = static_cast<const uint32_t*>(saved);
  if (!saved) {
    // recompute the saved state (the forward without O) into the workspace
    uint32_t* p = reinterpret_cast<uint32_t*>(ws);
    state = p;
    ws += room(need_saved);
    if (parts & 1) {
      ldc::DcFwdArgs f{(int)T, H, window, scale, q, k, v, cs, cw, doc_ids, nullptr, p,
                       p + ldc::dc_bands_bytes(T, H) / 4};
      if (ldc::dcmha_fwd_dispatch(dtype, d, f, false, hs) != hipSuccess) return LDC_ERR_HIP;
    }
  }
  ldc::DcBwdArgs a{(int)T, H, window, scale, q, k, v, dO, cs, cw, doc_ids, dq, dk, dv, dcs, dcw,
                   state, state + ldc::dc_bands_bytes(T, H) / 4, reinterpret_cast<uint32_t*>(ws)};
  return ldc::dcmha_bwd_dispatch(dtype, d, a, parts, hs) == hipSuccess ? LDC_OK : LDC_ERR_HIP;
}

#define DC_BWD_PARAMS                                                                             \
  int dtype, int64_t T, int H, int d, int window, float scale, const void *q, const void *k,       \
      const void *v, const float *cs, const float *cw, const int32_t *doc_ids, const void *saved,  \
      size_t saved_bytes, const void *dO, float *dq, float *dk, float *dv, float *dcs, float *dcw, \
      void *workspace, size_t workspace_bytes, void *stream
#define DC_BWD_ARGS                                                                              \
  dtype, T, H, d, window, scale, q, k, v, cs, cw, doc_ids, saved, saved_bytes, dO, dq, dk, dv, dcs, \
      dcw, workspace, workspace_bytes, stream

int dcmha_bwd(DC_BWD_PARAMS) { return bwd_parts(3, DC_BWD_ARGS); }
int dcmha_bwd_q(DC_BWD_PARAMS) { return bwd_parts(1, DC_BWD_ARGS); }
int dcmha_bwd_kv(DC_BWD_PARAMS) { return bwd_parts(2, DC_BWD_ARGS); }

}  // extern "C"
