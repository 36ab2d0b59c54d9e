// Internal interface between the fused-block C ABI (fused_api.cpp) and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

struct AttnArgs {
  int T, H;
  float scale;
  const void *q, *k, *v;
  const float* g;         // Lightweight DC scale G [T,H] (with the band)
  const uint32_t* band;   // composed-map band of the Lightweight DC score pass, or null
  const int32_t* rs;      // run start of every token
  float* o;
};

// 1024-token blocks of the run-start pass (one int of workspace each).
size_t run_blocks(int64_t T);
// rs[t] = first token of the run of equal ids holding t (`last`: run_blocks(T) ints).
hipError_t run_starts_dispatch(const int32_t* doc, int T, int* last, int* rs, hipStream_t st);
// ldc = false: the main attention alone (a.band, a.g unused).
hipError_t attn_fwd_dispatch(int d, const AttnArgs& a, bool ldc, hipStream_t st);

}  // namespace ldc
