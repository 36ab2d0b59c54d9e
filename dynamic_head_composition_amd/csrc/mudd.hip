// MUDD layer mixing for gfx950: per token, W weighted sums of J layer streams
// (forward) and their gradients (backward).
//
// The mix (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
// section "第一刀—砍层间"): Y_w[t] = sum_j A[t,w,j] X_j[t]; weights of any
// sign, no normalisation.  Backward: dX_j[t] = sum_w A[t,w,j] dY_w[t] and
// dA[t,w,j] = <dY_w[t], X_j[t]>.
//
// The work is HBM-bound streaming: every stored element is read once and
// every output element written once, with nothing to reuse, so there is no
// LDS staging and no MFMA.  Each wave owns whole token rows (grid-stride over
// rows): the row's W x J weights arrive in one coalesced load (lane i holds
// weight i) and are broadcast with readlane, and lane l covers elements
// [256 s + 4 l, 256 s + 4 l + 4) of slot s, so every load instruction reads
// 512 (bf16) or 1024 (fp32) contiguous bytes and every store writes 1024
// contiguous bytes of a float32 row.  Loads are unconditional (lanes past the
// row end read column 0 of the row and are masked afterwards) so a batch of
// them is in flight before the first use.  Rows are processed in groups of SG
// slots (SG x 256 columns) to bound registers.  Every load and store is
// non-temporal: no element is touched twice, and keeping the streams out of
// the caches measured 4-10% faster than ordinary accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mudd_internal.h"

namespace mudd {
namespace {

constexpr int kWaves = 4;  // waves per workgroup

typedef uint16_t bf16_t;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Four consecutive stored elements, kept in their storage form until used so
// that a batch of loads is in flight before any conversion.
template <typename T>
struct Raw;
template <>
struct Raw<bf16_t> {
  u32x2 u;
  __device__ __forceinline__ void load(const bf16_t* p) {
    u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  __device__ __forceinline__ float4 f() const {
    return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  }
};
template <>
struct Raw<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ float4 f() const { return float4{v.x, v.y, v.z, v.w}; }
};

__device__ __forceinline__ void store_nt(float* p, const float4& v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ void fma4(float4& acc, float s, const float4& x) {
  acc.x = fmaf(s, x.x, acc.x);
  acc.y = fmaf(s, x.y, acc.y);
  acc.z = fmaf(s, x.z, acc.z);
  acc.w = fmaf(s, x.w, acc.w);
}

// weight i of the row, held by lane i of `wl` (i wave-uniform)
__device__ __forceinline__ float weight(float wl, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, int SG>
__global__ __launch_bounds__(kWaves * 64) void fwd_kernel(const FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = a.W, J = a.J, dm = a.dm;
  const int nslot = (dm + 255) >> 8;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wv; t < a.T; t += stride) {
    const float wl = lane < W * J ? a.a[t * (W * J) + lane] : 0.f;
    const size_t row = (size_t)t * dm;
    for (int s0 = 0; s0 < nslot; s0 += SG) {
      int colc[SG];  // this lane's columns, clamped into the row
#pragma unroll
      for (int s = 0; s < SG; ++s) {
        const int col = 256 * (s0 + s) + 4 * lane;
        colc[s] = col < dm ? col : 0;
      }
      float4 acc[kMaxW][SG];
#pragma unroll
      for (int w = 0; w < kMaxW; ++w)
#pragma unroll
        for (int s = 0; s < SG; ++s) acc[w][s] = float4{0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < J; j0 += 4) {
        Raw<T> xv[4][SG];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (j0 + jj >= J) break;  // wave-uniform
          const T* xj = static_cast<const T*>(a.x[j0 + jj]) + row;
#pragma unroll
          for (int s = 0; s < SG; ++s) xv[jj][s].load(xj + colc[s]);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (j0 + jj >= J) break;
#pragma unroll
          for (int w = 0; w < kMaxW; ++w) {
            if (w >= W) break;
            const float aw = weight(wl, w * J + j0 + jj);
#pragma unroll
            for (int s = 0; s < SG; ++s) fma4(acc[w][s], aw, xv[jj][s].f());
          }
        }
      }
#pragma unroll
      for (int w = 0; w < kMaxW; ++w) {
        if (w >= W) break;
        float* yw = a.y[w] + row;
#pragma unroll
        for (int s = 0; s < SG; ++s) {
          const int col = 256 * (s0 + s) + 4 * lane;
          if (col < dm) store_nt(yw + col, acc[w][s]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// One halving step of a sum over lanes of N values at once: lanes that differ
// in bit M pair up; each keeps the half of the values selected by that bit
// and adds its partner's copy of that half.
template <int N, int M>
__device__ __forceinline__ void reduce_step(float (&v)[16], int lane) {
  constexpr int H = N / 2;
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float send = up ? v[i] : v[i + H];
    const float keep = up ? v[i + H] : v[i];
    v[i] = keep + __shfl_xor(send, M);
  }
}

// Sum of v[i] over the 64 lanes for all 16 indices: four halving steps on
// lane bits 5..2 (index bits 3..0) and two plain steps on bits 1..0, so lane
// l ends with the total of index (l >> 2) & 15 (17 shuffles instead of 96).
__device__ __forceinline__ float transpose_reduce16(float (&v)[16], int lane) {
  reduce_step<16, 32>(v, lane);
  reduce_step<8, 16>(v, lane);
  reduce_step<4, 8>(v, lane);
  reduce_step<2, 4>(v, lane);
  float x = v[0];
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

template <typename T, int SG>
__global__ __launch_bounds__(kWaves * 64) void bwd_kernel(const BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = a.W, J = a.J, dm = a.dm;
  const int nslot = (dm + 255) >> 8;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wv; t < a.T; t += stride) {
    const float wl = lane < W * J ? a.a[t * (W * J) + lane] : 0.f;
    const size_t row = (size_t)t * dm;
    // dA of the streams of batch b (4b .. 4b+3), summed over the wave: lane l
    // holds (w, j) = ((l >> 4) & 3, 4b + ((l >> 2) & 3))
    float red[kMaxJ / 4];
#pragma unroll
    for (int b = 0; b < kMaxJ / 4; ++b) red[b] = 0.f;
    for (int s0 = 0; s0 < nslot; s0 += SG) {
      int colc[SG];  // this lane's columns, clamped into the row
#pragma unroll
      for (int s = 0; s < SG; ++s) {
        const int col = 256 * (s0 + s) + 4 * lane;
        colc[s] = col < dm ? col : 0;
      }
      // dY of the ways; zero in lanes past the row end, so they add nothing to dA
      float4 dyv[kMaxW][SG];
      {
        Raw<T> r[kMaxW][SG];
#pragma unroll
        for (int w = 0; w < kMaxW; ++w) {
          if (w >= W) break;  // wave-uniform
          const T* dyw = static_cast<const T*>(a.dy[w]) + row;
#pragma unroll
          for (int s = 0; s < SG; ++s) r[w][s].load(dyw + colc[s]);
        }
#pragma unroll
        for (int w = 0; w < kMaxW; ++w)
#pragma unroll
          for (int s = 0; s < SG; ++s) {
            const bool on = w < W && 256 * (s0 + s) + 4 * lane < dm;
            dyv[w][s] = on ? r[w][s].f() : float4{0.f, 0.f, 0.f, 0.f};
          }
      }
#pragma unroll
      for (int j0 = 0; j0 < kMaxJ; j0 += 4) {
        if (j0 >= J) break;
        Raw<T> xv[4][SG];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (j0 + jj >= J) break;  // wave-uniform
          const T* xj = static_cast<const T*>(a.x[j0 + jj]) + row;
#pragma unroll
          for (int s = 0; s < SG; ++s) xv[jj][s].load(xj + colc[s]);
        }
        float p[16];  // this lane's part of dA, index w * 4 + jj
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = j0 + jj;
          if (j >= J) break;
          float* dxj = a.dx[j] + row;
#pragma unroll
          for (int s = 0; s < SG; ++s) {
            const int col = 256 * (s0 + s) + 4 * lane;
            const float4 x = xv[jj][s].f();
            float4 d = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kMaxW; ++w) {
              if (w >= W) break;
              fma4(d, weight(wl, w * J + j), dyv[w][s]);
              p[w * 4 + jj] = dot4(dyv[w][s], x, p[w * 4 + jj]);
            }
            if (col < dm) store_nt(dxj + col, d);
          }
        }
        red[j0 / 4] += transpose_reduce16(p, lane);
      }
    }
    const int w = (lane >> 4) & 3, jj = (lane >> 2) & 3;
#pragma unroll
    for (int b = 0; b < kMaxJ / 4; ++b) {
      const int j = 4 * b + jj;
      if ((lane & 3) == 0 && w < W && j < J) a.da[t * (W * J) + w * J + j] = red[b];
    }
  }
}

template <typename T, int SG>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + kWaves - 1) / kWaves;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL((fwd_kernel<T, SG>), dim3(grid), dim3(kWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int SG>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  const int64_t blocks = (a.T + kWaves - 1) / kWaves;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL((bwd_kernel<T, SG>), dim3(grid), dim3(kWaves * 64), 0, st, a);
  return hipGetLastError();
}

// slots per group: a whole row when it has at most 4 slots (1,024 columns)
inline int slot_group(int dm) {
  const int nslot = (dm + 255) / 256;
  return nslot < 4 ? nslot : 4;
}

}  // namespace

hipError_t fwd_dispatch(int dtype, const FwdArgs& a, hipStream_t st) {
  const int sg = slot_group(a.dm);
  if (dtype == 0) {
    switch (sg) {
      case 1: return launch_fwd<bf16_t, 1>(a, st);
      case 2: return launch_fwd<bf16_t, 2>(a, st);
      case 3: return launch_fwd<bf16_t, 3>(a, st);
      default: return launch_fwd<bf16_t, 4>(a, st);
    }
  }
  switch (sg) {
    case 1: return launch_fwd<float, 1>(a, st);
    case 2: return launch_fwd<float, 2>(a, st);
    case 3: return launch_fwd<float, 3>(a, st);
    default: return launch_fwd<float, 4>(a, st);
  }
}

hipError_t bwd_dispatch(int dtype, const BwdArgs& a, hipStream_t st) {
  const int sg = slot_group(a.dm);
  if (dtype == 0) {
    switch (sg) {
      case 1: return launch_bwd<bf16_t, 1>(a, st);
      case 2: return launch_bwd<bf16_t, 2>(a, st);
      case 3: return launch_bwd<bf16_t, 3>(a, st);
      default: return launch_bwd<bf16_t, 4>(a, st);
    }
  }
  switch (sg) {
    case 1: return launch_bwd<float, 1>(a, st);
    case 2: return launch_bwd<float, 2>(a, st);
    case 3: return launch_bwd<float, 3>(a, st);
    default: return launch_bwd<float, 4>(a, st);
  }
}

}  // namespace mudd
