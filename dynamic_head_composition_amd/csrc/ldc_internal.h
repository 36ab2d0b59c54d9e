// Internal interface between the C ABI (ldc_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

// Key blocks per band: 8 for windows up to 113 keys, 10 up to 128.
inline int band_key_blocks(int window) { return window > 113 ? 10 : 8; }

struct FwdArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v;
  const float *c, *g;
  const int32_t* doc;
  float* o;
  uint32_t* band;  // saved shared-map band, or null (nothing saved)
  float2* stats;   // saved [T,H] softmax statistics (with band)
};

struct BwdArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v, *dO;
  const float *c, *g;
  const int32_t* doc;
  float *dq, *dk, *dv, *dc, *dg;
  const uint32_t* band;  // shared-map band saved by the forward pass
  const float2* stats;   // [T,H] (scaled row max, 1/row sum), saved by the forward pass
  float* dband;          // workspace: dPbar band, written by bwd_q, read by bwd_kv
};

// Sizes of the saved state and of the backward workspace: one band block of
// 256 words per key block and 16-query block.
inline size_t band_blocks(int64_t T) { return (size_t)((T + 15) / 16); }
inline size_t saved_band_bytes(int64_t T, int window) {
  return band_blocks(T) * (size_t)band_key_blocks(window) * 256 * 4;
}

// value = false: only the saved state (band and statistics), no O.
hipError_t fwd_dispatch(int dtype, int d, const FwdArgs& a, bool value, hipStream_t st);
// parts: bit 0 = query-side kernel, bit 1 = key-side kernel
hipError_t bwd_dispatch(int dtype, int d, const BwdArgs& a, int parts, hipStream_t st);

// Static device workspace of ldc_bwd_noalloc (bytes per GPU) and the device
// address of one GPU's copy (looked up on first use, then cached).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(int device, void** ptr);

}  // namespace ldc
