// Internal interface between the DCMHA C ABI (dcmha_api.cpp) and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

constexpr int kDcMaxHeads = 6;  // a wave holds every head's band in registers

struct DcFwdArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v;
  const float *cs, *cw;  // [T,H,H] score and weight compositions
  const int32_t* doc;
  float* o;
  uint32_t* pband;  // saved softmax maps P_h (one band per head), or null
  uint32_t* rband;  // saved composed maps R_h, or null (with pband)
};

struct DcBwdArgs {
  int T, H, window;
  float scale;
  const void *q, *k, *v, *dO;
  const float *cs, *cw;
  const int32_t* doc;
  float *dq, *dk, *dv, *dcs, *dcw;
  const uint32_t* pband;  // P_h bands saved by the forward pass
  const uint32_t* rband;  // R_h bands saved by the forward pass
  uint32_t* dsband;       // workspace: dS_h bands, written by bwd_q, read by bwd_kv
};

// Bytes of one set of per-head bands (16-query blocks x H x 2,048 words).
inline size_t dc_bands_bytes(int64_t T, int H) {
  return (size_t)((T + 15) / 16) * (size_t)H * 2048 * 4;
}

// out = false: P and R bands only (no O).
hipError_t dcmha_fwd_dispatch(int dtype, int d, const DcFwdArgs& a, bool out, hipStream_t st);
// parts: bit 0 = query-side kernel, bit 1 = key-side kernel
hipError_t dcmha_bwd_dispatch(int dtype, int d, const DcBwdArgs& a, int parts, hipStream_t st);

}  // namespace ldc
