// Internal interface between the fused-block C ABI (fused_api.cpp) and its kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

struct FusedArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v;
  const float *c, *g;  // Lightweight DC weights [T,H] (unused by the main attention alone)
  const int32_t* doc;
  float* o;
};

// ldc = false: the main attention alone.
hipError_t fused_fwd_dispatch(int d, const FusedArgs& a, bool ldc, hipStream_t st);

}  // namespace ldc
