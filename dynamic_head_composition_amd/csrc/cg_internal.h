// Internal interface between the generator's C ABI (cg_api.cpp) and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

struct CgArgs {
  int T, dm, H;
  const void *x, *wc, *wg;  // [T, dm], [dm, H], [dm, H] in the storage dtype
  float *c, *g;             // [T, H]
};

struct CgBwdArgs {
  int T, dm, H;
  const void *x, *wc, *wg;
  const float *dc, *dg;     // [T, H]
  float* dx;                // [T, dm]
  float *dwc, *dwg;         // [dm, H]
  float* partial;           // workspace: per-chunk dW partials
};

size_t cg_partial_bytes(int64_t T, int dm);
hipError_t cg_fwd_dispatch(int dtype, const CgArgs& a, hipStream_t st);
hipError_t cg_bwd_dispatch(int dtype, const CgBwdArgs& a, hipStream_t st);

}  // namespace ldc
