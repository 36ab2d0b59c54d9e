// Internal interface between the C ABI (ldc_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

struct FwdArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v;
  const float *c, *g;
  const int32_t* doc;
  float* o;
};

struct BwdArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v, *dO;
  const float *c, *g;
  const int32_t* doc;
  float *dq, *dk, *dv, *dc, *dg;
  float2* stats;  // [T,H] (scaled row max, 1/row sum) of each head's softmax
};

hipError_t fwd_dispatch(int dtype, int d, const FwdArgs& a, hipStream_t st);
// parts: bit 0 = query-side kernel, bit 1 = key-side kernel
hipError_t bwd_dispatch(int dtype, int d, const BwdArgs& a, int parts, hipStream_t st);

}  // namespace ldc
