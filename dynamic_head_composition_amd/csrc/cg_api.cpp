// C ABI of the generator of the Lightweight DC weights: validation and
// dispatch.  Every validation precedes any HIP call.
#include "../../include/ldc_cg.h"

#include <hip/hip_runtime.h>

#include "cg_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check(int dtype, int64_t T, int dm, int H) {
  if (dtype != LDC_BF16 && dtype != LDC_F32) return LDC_ERR_DTYPE;
  if (T < 0 || H < 1 || dm < 1) return LDC_ERR_SHAPE;
  if (T > ((int64_t)1 << 30) || T * (int64_t)dm >= ((int64_t)1 << 31)) return LDC_ERR_SHAPE;
  if (H > 8 || dm % 64 != 0 || dm > (dtype == LDC_BF16 ? 1024 : 768)) return LDC_ERR_UNSUPPORTED;
  return LDC_OK;
}

}  // namespace

extern "C" {

size_t ldc_cg_bwd_workspace_bytes(int dtype, int64_t T, int dm, int H) {
  if (check(dtype, T, dm, H) != LDC_OK || T == 0) return 0;
  return ldc::cg_partial_bytes(T, dm);
}

int ldc_cg_fwd(int dtype, int64_t T, int dm, int H, const void* x, const void* wc, const void* wg,
               float* c, float* g, void* stream) {
  int st = check(dtype, T, dm, H);
  if (st != LDC_OK) return st;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {x, wc, wg, c, g};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  ldc::CgArgs a{(int)T, dm, H, x, wc, wg, c, g};
  return ldc::cg_fwd_dispatch(dtype, a, static_cast<hipStream_t>(stream)) == hipSuccess ? LDC_OK : LDC_ERR_HIP;
}

int ldc_cg_bwd(int dtype, int64_t T, int dm, int H, const void* x, const void* wc, const void* wg,
               const float* dc, const float* dg, float* dx, float* dwc, float* dwg, void* workspace,
               size_t workspace_bytes, void* stream) {
  int st = check(dtype, T, dm, H);
  if (st != LDC_OK) return st;
  const void* ptrs[] = {x, wc, wg, dc, dg, dx, dwc, dwg};
  for (const void* p : ptrs)
    if (!p && T > 0) return LDC_ERR_NULL;
  if (!dwc || !dwg) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return LDC_ERR_ALIGN;
  if (T > 0) {
    if (!workspace || workspace_bytes < ldc::cg_partial_bytes(T, dm)) return LDC_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LDC_ERR_ALIGN;
  }
  ldc::CgBwdArgs a{(int)T, dm, H, x, wc, wg, dc, dg, dx, dwc, dwg, static_cast<float*>(workspace)};
  return ldc::cg_bwd_dispatch(dtype, a, static_cast<hipStream_t>(stream)) == hipSuccess ? LDC_OK : LDC_ERR_HIP;
}

}  // extern "C"
