// Lightweight DC backward pass for gfx950.
//
// Gradients of the layer defined on the AITNT page "一个国产AI小透明，连续两次
// 刷新NanoGPT Speedrun世界纪录" (section "第二刀-砍层内", Lightweight DC
// paragraph), by the chain rule through: per-head window softmax P_h,
// shared map Pbar = sum_h C_h P_h, O_h = G_h Pbar V_h.  With B_h = dO_h V_h^T:
//   dG_h = rowsum(Pbar o B_h)          dPbar = sum_h G_h B_h
//   dC_h = rowsum(P_h o dPbar)         dS_h  = C_h P_h o (dPbar - dC_h)
//   dQ_h = scale dS_h K_h              dK_h  = scale dS_h^T Q_h
//   dV_h = (G_h o Pbar)^T dO_h
//
// Two deterministic kernels, no atomics and no zero-fill:
//  * bwd_q  (query-centric, like the forward): each wave owns 16 queries and
//    computes their dQ, dC, dG, plus each head's softmax statistics, which it
//    hands to the second kernel through the workspace.
//  * bwd_kv (key-centric): each wave owns 16 keys and the 128 queries whose
//    windows can hold them; it recomputes P_h from the statistics and makes
//    three passes over the heads: Pbar (Q_h staged); dV_h and dPbar (dO_h
//    staged); dS_h and dK_h (Q_h staged).
// Neither writes a T x window map to HBM: the per-pair quantities live in
// registers of the wave that needs them.
#include "ldc_device.hpp"
#include "ldc_internal.h"

namespace ldc {

// ---------------------------------------------------------------------------
// bwd_q: per query.  Transposed orientation as in the forward: lane = query
// column n, 32 band entries (key rows 4g+i of block b) in registers.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void bwd_q_kernel(const BwdArgs a) {
  constexpr int BQ = 16 * NW;
  constexpr int R = BQ + kHalo;
  constexpr int NT = NW * kWave;
  constexpr int S = lds_stride<T, D>();
  __shared__ __attribute__((aligned(16))) T s_x[R * S];
  __shared__ int s_doc[R];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ dO = static_cast<const T*>(a.dO);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int q0 = tile * BQ;
  const int span0 = q0 - kHalo;
  const int brow = 16 * w;
  const int t = q0 + 16 * w + n;
  const bool tval = t < a.T;
  const int H = a.H;

  for (int r = threadIdx.x; r < R; r += NT) {
    const int s = span0 + r;
    s_doc[r] = (s >= 0 && s < a.T) ? a.doc[s] : 0;
  }
  __syncthreads();
  uint32_t mbits = 0;
  if (tval) {
    const int dt = s_doc[brow + kHalo + n];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int s = span0 + r;
        const bool ok = s >= 0 && s <= t && t - s < a.window && s_doc[r] == dt;
        mbits |= (ok ? 1u : 0u) << (4 * b + i);
      }
  }
  uint32_t live = 0;
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b) live |= (__any((mbits >> (4 * b)) & 15u) ? 1u : 0u) << b;

  const float sl2 = a.scale * kLog2e;
  f32x4 pb[kKeyBlocks], dpb[kKeyBlocks];
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b) pb[b] = dpb[b] = zero4();

  // Scores of head h for this lane's query, softmax-normalised in place.
  auto softmax_head = [&](f32x4 (&sc)[kKeyBlocks], const RowFrag<T, D>& qf, float& mx_out,
                          float& inv_out) {
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      sc[b] = zero4();
      if ((live >> b) & 1u) sc[b] = mma_dcontract<T, D>(sc[b], s_x + (brow + 16 * b + n) * S, qf, g);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[b][i] *= sl2;
        if ((mbits >> (4 * b + i)) & 1u) mx = fmaxf(mx, sc[b][i]);
      }
    mx = wave_max4(mx);
    float sum = 0.f;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = ((mbits >> (4 * b + i)) & 1u) ? fast_exp2(sc[b][i] - mx) : 0.f;
        sc[b][i] = e;
        sum += e;
      }
    sum = wave_sum4(sum);
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[b][i] *= inv;
    mx_out = mx;
    inv_out = inv;
  };

  // ---- phase A: P_h, Pbar, softmax statistics ----
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    stage_rows<T, D, R, NT>(s_x, k, span0, a.T, H, h);
    RowFrag<T, D> qf;
    load_row_frag<T, D>(qf, q + ((size_t)t * H + h) * D, g, tval);
    const float ch = tval ? a.c[(size_t)t * H + h] : 0.f;
    __syncthreads();
    f32x4 sc[kKeyBlocks];
    float mx, inv;
    softmax_head(sc, qf, mx, inv);
    if (tval && g == 0) a.stats[(size_t)t * H + h] = float2{mx, inv};
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[b][i] += ch * sc[b][i];
  }

  // ---- phase B: B_h = dO_h V_h^T, dPbar, dG ----
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    stage_rows<T, D, R, NT>(s_x, v, span0, a.T, H, h);
    RowFrag<T, D> df;
    load_row_frag<T, D>(df, dO + ((size_t)t * H + h) * D, g, tval);
    const float gh = tval ? a.g[(size_t)t * H + h] : 0.f;
    __syncthreads();
    float dgs = 0.f;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      if (!((live >> b) & 1u)) continue;
      f32x4 bt = mma_dcontract<T, D>(zero4(), s_x + (brow + 16 * b + n) * S, df, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // masked entries of pb are exactly 0; bt there is finite (zero-filled rows)
        dgs += pb[b][i] * bt[i];
        dpb[b][i] += gh * bt[i];
      }
    }
    dgs = wave_sum4(dgs);
    if (tval && g == 0) a.dg[(size_t)t * H + h] = dgs;
  }

  // ---- phase C: recompute P_h, dC, dS, dQ ----
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    stage_rows<T, D, R, NT>(s_x, k, span0, a.T, H, h);
    RowFrag<T, D> qf;
    load_row_frag<T, D>(qf, q + ((size_t)t * H + h) * D, g, tval);
    const float ch = tval ? a.c[(size_t)t * H + h] : 0.f;
    __syncthreads();
    f32x4 sc[kKeyBlocks];
    float mx, inv;
    softmax_head(sc, qf, mx, inv);
    float dcs = 0.f;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dcs += sc[b][i] * dpb[b][i];
    dcs = wave_sum4(dcs);
    if (tval && g == 0) a.dc[(size_t)t * H + h] = dcs;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[b][i] = ch * sc[b][i] * (dpb[b][i] - dcs);
    BandOperand<T> dso;
    dso.set(sc);
    f32x4 acc[D / 16];
    mma_tcontract<T, D>(acc, s_x, brow, dso, live, g, n);
    if (tval) store_row_f32<T, D>(a.dq + ((size_t)t * H + h) * D, acc, a.scale, g);
  }
}

// ---------------------------------------------------------------------------
// bwd_kv: per key.  Normal orientation S = Q K^T: lane = key column n, rows
// 4g+i of query block b in registers; the wave's queries are the 128 tokens
// [kw, kw+128) that can hold its keys in their windows.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void bwd_kv_kernel(const BwdArgs a) {
  constexpr int BK = 16 * NW;
  constexpr int R = BK + kHalo;  // query rows [k0, k0 + BK + 112)
  constexpr int NT = NW * kWave;
  constexpr int S = lds_stride<T, D>();
  __shared__ __attribute__((aligned(16))) T s_x[R * S];
  __shared__ int s_doc[R];
  __shared__ __attribute__((aligned(16))) float s_c[R];
  __shared__ __attribute__((aligned(16))) float s_g[R];
  __shared__ __attribute__((aligned(16))) float s_dc[R];
  __shared__ __attribute__((aligned(16))) float s_mx[R];
  __shared__ __attribute__((aligned(16))) float s_inv[R];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ dO = static_cast<const T*>(a.dO);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int k0 = tile * BK;
  const int span0 = k0;
  const int brow = 16 * w;        // LDS row of this wave's first query (token kw)
  const int s = k0 + 16 * w + n;  // this lane's key
  const bool sval = s < a.T;
  const int H = a.H;

  for (int r = threadIdx.x; r < R; r += NT) {
    const int t = span0 + r;
    s_doc[r] = (t < a.T) ? a.doc[t] : 0;
  }
  __syncthreads();
  uint32_t mbits = 0;  // bit 4b+i <-> query row brow + 16b + 4g + i
  if (sval) {
    const int ds = s_doc[brow + n];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int t = span0 + r;
        const bool ok = t < a.T && t >= s && t - s < a.window && s_doc[r] == ds;
        mbits |= (ok ? 1u : 0u) << (4 * b + i);
      }
  }
  uint32_t live = 0;
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b) live |= (__any((mbits >> (4 * b)) & 15u) ? 1u : 0u) << b;

  auto stage_scalars = [&](int h) {
    for (int r = threadIdx.x; r < R; r += NT) {
      const int t = span0 + r;
      float c = 0.f, gg = 0.f, dc = 0.f, mx = 0.f, inv = 0.f;
      if (t < a.T) {
        const size_t i = (size_t)t * H + h;
        c = a.c[i];
        gg = a.g[i];
        dc = a.dc[i];
        const float2 st = a.stats[i];
        mx = st.x;
        inv = st.y;
      }
      s_c[r] = c;
      s_g[r] = gg;
      s_dc[r] = dc;
      s_mx[r] = mx;
      s_inv[r] = inv;
    }
  };
  auto rows4 = [&](const float* arr, int b) {
    return *reinterpret_cast<const float4*>(arr + brow + 16 * b + 4 * g);
  };

  const float sl2 = a.scale * kLog2e;
  // P_h of head h on this lane's band (rows = queries), from the statistics.
  auto probs = [&](f32x4 (&sc)[kKeyBlocks], const RowFrag<T, D>& kf) {
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      sc[b] = zero4();
      if ((live >> b) & 1u) sc[b] = mma_dcontract<T, D>(sc[b], s_x + (brow + 16 * b + n) * S, kf, g);
      const float4 mx = rows4(s_mx, b), inv = rows4(s_inv, b);
      const float mxv[4] = {mx.x, mx.y, mx.z, mx.w}, invv[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[b][i] = ((mbits >> (4 * b + i)) & 1u) ? fast_exp2(sc[b][i] * sl2 - mxv[i]) * invv[i] : 0.f;
    }
  };

  // ---- pass 1: Pbar on the band (Q_h staged) ----
  f32x4 pb[kKeyBlocks];
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b) pb[b] = zero4();
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    stage_rows<T, D, R, NT>(s_x, q, span0, a.T, H, h);
    stage_scalars(h);
    RowFrag<T, D> kf;
    load_row_frag<T, D>(kf, k + ((size_t)s * H + h) * D, g, sval);
    __syncthreads();
    f32x4 sc[kKeyBlocks];
    probs(sc, kf);
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      const float4 c4 = rows4(s_c, b);
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[b][i] += cv[i] * sc[b][i];
    }
  }

  // ---- pass 2 (dO_h staged): dV_h = (G_h o Pbar)^T dO_h, and dPbar ----
  f32x4 dpb[kKeyBlocks];
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b) dpb[b] = zero4();
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    stage_rows<T, D, R, NT>(s_x, dO, span0, a.T, H, h);
    stage_scalars(h);
    RowFrag<T, D> vf;
    load_row_frag<T, D>(vf, v + ((size_t)s * H + h) * D, g, sval);
    __syncthreads();
    {
      f32x4 gp[kKeyBlocks];
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b) {
        const float4 g4 = rows4(s_g, b);
        gp[b] = f32x4{g4.x * pb[b][0], g4.y * pb[b][1], g4.z * pb[b][2], g4.w * pb[b][3]};
      }
      BandOperand<T> op;
      op.set(gp);
      f32x4 acc[D / 16];
      mma_tcontract<T, D>(acc, s_x, brow, op, live, g, n);
      if (sval) store_row_f32<T, D>(a.dv + ((size_t)s * H + h) * D, acc, 1.f, g);
    }
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      if (!((live >> b) & 1u)) continue;
      const f32x4 bt = mma_dcontract<T, D>(zero4(), s_x + (brow + 16 * b + n) * S, vf, g);
      const float4 g4 = rows4(s_g, b);
      const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) dpb[b][i] += gv[i] * bt[i];
    }
  }

  // ---- pass 3 (Q_h staged): P_h, dS_h, dK_h = scale dS_h^T Q_h ----
  for (int h = 0; h < H; ++h) {
    __syncthreads();
    stage_rows<T, D, R, NT>(s_x, q, span0, a.T, H, h);
    stage_scalars(h);
    RowFrag<T, D> kf;
    load_row_frag<T, D>(kf, k + ((size_t)s * H + h) * D, g, sval);
    __syncthreads();
    f32x4 sc[kKeyBlocks];
    probs(sc, kf);
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      const float4 c4 = rows4(s_c, b), dc4 = rows4(s_dc, b);
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, dcv[4] = {dc4.x, dc4.y, dc4.z, dc4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[b][i] = cv[i] * sc[b][i] * (dpb[b][i] - dcv[i]);
    }
    BandOperand<T> dso;
    dso.set(sc);
    f32x4 acc[D / 16];
    mma_tcontract<T, D>(acc, s_x, brow, dso, live, g, n);
    if (sval) store_row_f32<T, D>(a.dk + ((size_t)s * H + h) * D, acc, a.scale, g);
  }
}

template <typename T, int D, int NW>
static hipError_t launch_bwd(const BwdArgs& a, int parts, hipStream_t st) {
  constexpr int B = 16 * NW;
  const int nblk = (int)((a.T + B - 1) / B);
  if (parts & 1) {
    hipLaunchKernelGGL((bwd_q_kernel<T, D, NW>), dim3(nblk), dim3(NW * kWave), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (parts & 2) {
    hipLaunchKernelGGL((bwd_kv_kernel<T, D, NW>), dim3(nblk), dim3(NW * kWave), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t bwd_dispatch(int dtype, int d, const BwdArgs& a, int parts, hipStream_t st) {
  if (dtype == 0) {
    if (d == 128) return launch_bwd<bf16_t, 128, 8>(a, parts, st);
    if (d == 64) return launch_bwd<bf16_t, 64, 8>(a, parts, st);
  } else {
    if (d == 128) return launch_bwd<float, 128, 4>(a, parts, st);
    if (d == 64) return launch_bwd<float, 64, 4>(a, parts, st);
    if (d == 16) return launch_bwd<float, 16, 4>(a, parts, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ldc
