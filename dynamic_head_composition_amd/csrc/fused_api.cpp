// C ABI of the fused block: argument validation, workspace layout and the
// launch sequence.  Every validation precedes any HIP call, so the error paths
// run without a GPU.
#include "../../include/ldc_fused.h"

#include <hip/hip_runtime.h>

#include "fused_internal.h"
#include "ldc_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool scale_ok(float scale) { return scale > 0.f && scale < 3.0e38f; }

size_t room(size_t x) { return (x + 255) & ~(size_t)255; }

int check(int dtype, int64_t T, int H, int d, int window, float scale) {
  if (dtype != LDC_BF16 && dtype != LDC_F32) return LDC_ERR_DTYPE;
  if (T < 0 || H < 1 || window < 1 || window > 128 || d < 1 || !scale_ok(scale)) return LDC_ERR_SHAPE;
  const int64_t elems = T * (int64_t)H * (int64_t)d;
  if (T > (int64_t)1 << 30 || elems + 512LL * H * d >= ((int64_t)1 << 31)) return LDC_ERR_SHAPE;
  if (dtype != LDC_BF16 || !(d == 64 || d == 128)) return LDC_ERR_UNSUPPORTED;
  return LDC_OK;
}

// run-start arrays: the block summaries, then one int per token
size_t runs_bytes(int64_t T) {
  return room(ldc::run_blocks(T) * 4) + room((size_t)T * 4) + ldc::order_ints(T) * 4;
}

int run(bool ldc_on, int dtype, int64_t T, int H, int d, int window, float scale, const void* q,
        const void* k, const void* v, const float* c, const float* g, const int32_t* doc_ids, float* o,
        void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check(dtype, T, H, d, window, scale);
  if (st != LDC_OK) return st;
  if (T == 0) return LDC_OK;
  const void* ptrs[] = {q, k, v, doc_ids, o, ldc_on ? (const void*)c : q, ldc_on ? (const void*)g : q};
  for (const void* p : ptrs)
    if (!p) return LDC_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return LDC_ERR_ALIGN;
  const size_t saved = ldc_on ? ldc_saved_bytes(dtype, T, H, d, window) : 0;
  const size_t need = (ldc_on ? room(saved) : 0) + runs_bytes(T);
  if (!workspace || workspace_bytes < need) return LDC_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LDC_ERR_ALIGN;

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint32_t* band = nullptr;
  if (ldc_on) {
    // the Lightweight DC score pass: the layer's saved state at the start of
    // the workspace (band, then statistics), no output
    band = reinterpret_cast<uint32_t*>(ws);
    float2* stats = reinterpret_cast<float2*>(ws + ldc::saved_band_bytes(T, window));
    ldc::FwdArgs f{(int)T, H, window, scale, q, k, v, c, g, doc_ids, nullptr, band, stats};
    if (ldc::fwd_dispatch(dtype, d, f, false, hs) != hipSuccess) return LDC_ERR_HIP;
    ws += room(saved);
  }
  int* last = reinterpret_cast<int*>(ws);
  int* rs = reinterpret_cast<int*>(ws + room(ldc::run_blocks(T) * 4));
  int* order = reinterpret_cast<int*>(ws + room(ldc::run_blocks(T) * 4) + room((size_t)T * 4));
  if (ldc::run_starts_dispatch(doc_ids, (int)T, last, rs, order, hs) != hipSuccess) return LDC_ERR_HIP;
  ldc::AttnArgs a{(int)T, H, window, scale, q, k, v, g, band, rs, order + ldc::order_list_offset(), o};
  return ldc::attn_fwd_dispatch(d, a, ldc_on, hs) == hipSuccess ? LDC_OK : LDC_ERR_HIP;
}

}  // namespace

extern "C" {

size_t ldc_fused_fwd_workspace_bytes(int dtype, int64_t T, int H, int d, int window) {
  if (check(dtype, T, H, d, window, 1.f) != LDC_OK || T == 0) return 0;
  return room(ldc_saved_bytes(dtype, T, H, d, window)) + runs_bytes(T);
}

size_t ldc_main_attention_workspace_bytes(int64_t T) {
  if (T <= 0 || T > (int64_t)1 << 30) return 0;
  return runs_bytes(T);
}

int ldc_fused_fwd(int dtype, int64_t T, int H, int d, int window, float scale, const void* q, const void* k,
                  const void* v, const float* c, const float* g, const int32_t* doc_ids, float* o,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return run(true, dtype, T, H, d, window, scale, q, k, v, c, g, doc_ids, o, workspace, workspace_bytes,
             stream);
}

int ldc_main_attention_fwd(int dtype, int64_t T, int H, int d, float scale, const void* q, const void* k,
                           const void* v, const int32_t* doc_ids, float* o, void* workspace,
                           size_t workspace_bytes, void* stream) {
  // the window is not used: any valid value
  return run(false, dtype, T, H, d, 1, scale, q, k, v, nullptr, nullptr, doc_ids, o, workspace,
             workspace_bytes, stream);
}

}  // extern "C"
