// Internal interface between the MUDD C ABI (mudd_api.cpp) and its kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mudd {

constexpr int kMaxJ = 16;  // streams
constexpr int kMaxW = 4;   // ways

struct FwdArgs {
  const void* x[kMaxJ];  // J streams [T, dm], storage dtype
  float* y[kMaxW];       // W outputs [T, dm] float32
  const float* a;        // [T, W, J]
  int64_t T;
  int dm, W, J;
};

struct BwdArgs {
  const void* x[kMaxJ];   // J streams [T, dm]
  const void* dy[kMaxW];  // W upstream gradients [T, dm], storage dtype
  float* dx[kMaxJ];       // J outputs [T, dm] float32
  const float* a;         // [T, W, J]
  float* da;              // [T, W, J] float32 out
  int64_t T;
  int dm, W, J;
};

// dtype: 0 = bf16, 1 = float32 (the ldc_dtype values)
hipError_t fwd_dispatch(int dtype, const FwdArgs& a, hipStream_t st);
hipError_t bwd_dispatch(int dtype, const BwdArgs& a, hipStream_t st);

}  // namespace mudd
