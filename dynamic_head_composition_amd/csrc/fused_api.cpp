// C ABI of the fused block: argument validation and dispatch.  Every
// validation precedes any HIP call, so the error paths run without a GPU.
#include "../../include/ldc_fused.h"

#include <hip/hip_runtime.h>

#include "fused_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool scale_ok(float scale) { return scale > 0.f && scale < 3.0e38f; }

int check(int dtype, int64_t T, int H, int d, int window, float scale) {
  if (dtype != LDC_BF16 && dtype != LDC_F32) return LDC_ERR_DTYPE;
  if (T < 0 || H < 1 || window < 1 || window > 113 || d < 1 || !scale_ok(scale)) return LDC_ERR_SHAPE;
  const int64_t elems = T * (int64_t)H * (int64_t)d;
  if (T > (int64_t)1 << 30 || elems + 512LL * H * d >= ((int64_t)1 << 31)) return LDC_ERR_SHAPE;
  if (dtype != LDC_BF16 || !(d == 64 || d == 128)) return LDC_ERR_UNSUPPORTED;
  return LDC_OK;
}

int run(bool ldc, int dtype, int64_t T, int H, int d, int window, float scale, const void* q, const void* k,
        const void* v, const float* c, const float* g, const int32_t* doc_ids, float* o, void* stream) {
  const int st = check(dtype, T, H, d, window, scale);
  if (st != LDC_OK) return st;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {q, k, v, doc_ids, o, ldc ? (const void*)c : q, ldc ? (const void*)g : q};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  ldc::FusedArgs a{(int)T, H, window, scale, q, k, v, c, g, doc_ids, o};
  return ldc::fused_fwd_dispatch(d, a, ldc, static_cast<hipStream_t>(stream)) == hipSuccess ? LDC_OK
                                                                                          : LDC_ERR_HIP;
}

}  // namespace

extern "C" {

int ldc_fused_fwd(int dtype, int64_t T, int H, int d, int window, float scale, const void* q, const void* k,
                  const void* v, const float* c, const float* g, const int32_t* doc_ids, float* o, void* stream) {
  return run(true, dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, o, stream);
}

int ldc_main_attention_fwd(int dtype, int64_t T, int H, int d, float scale, const void* q, const void* k,
                           const void* v, const int32_t* doc_ids, float* o, void* stream) {
  // the window is not used: any valid value
  return run(false, dtype, T, H, d, 1, scale, q, k, v, nullptr, nullptr, doc_ids, o, stream);
}

}  // extern "C"
