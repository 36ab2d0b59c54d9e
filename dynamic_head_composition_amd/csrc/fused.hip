// The Lightweight DC layer fused with the attention block's main attention,
// forward, for gfx950.
//
// Layer (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
// section "第二刀-砍层内", Lightweight DC paragraph: the branch reuses the
// block's Q and K over a short local window, with a dedicated kernel), read as
//   O[t,h] = M[t,h] + G[t,h] sum_{s in A(t)} Pbar[t,s] V[s,h]
// M: causal softmax attention of head h over the query's own run of equal
// document ids (keys run_start(t) .. t); the second term: the Lightweight DC
// layer (its window and document cut, Pbar = sum_h C[t,h] P_h).
//
// One workgroup per 64-query tile (4 waves, one per SIMD) walks every head.
//  * Lightweight DC phase, per head: the window tile of K (keys q0-128 ..
//    q0+63) gives each wave its 8-block band of scores; the band's softmax
//    (window and document masks) is composed into Pbar with C[t,h]
//    (registers, all heads).
//  * Main pass, per head: 192-key tiles of K, then of V, from the run start of
//    the tile's first query up to q0-129, then the window tile: flash-style
//    online softmax (running max and sum per query, an fp32 accumulator of the
//    wave's 16 rows x d).  The window tile's V contraction takes one band
//    operand: the main weights plus l G[t,h] Pbar on the wave's band blocks
//    (l the final running sum), so O = acc / l carries both terms and is
//    written once.
// The window tile's K is read twice per head (once per phase); its V once.
// Tiles stream into LDS by DMA, double-buffered.  Deterministic.
#include "fused_internal.h"
#include "ldc_device.hpp"
#include "ldc_pipeline.hpp"

namespace ldc {

constexpr int kFNW = 4;                 // waves per workgroup
constexpr int kFBQ = 16 * kFNW;         // queries per workgroup
constexpr int kFBlocks = 12;            // 16-row blocks per staged tile
constexpr int kFRows = 16 * kFBlocks;   // 192 rows per staged tile
constexpr int kFWin = 128;              // the window tile starts 128 keys before the tile's first query

// acc += X^T P over a staged tile's NB blocks (X the tile's rows, P a band
// operand in accumulator layout): mma_tcontract_pipe's order (the LDS reads of
// column group p+1 ahead of the MFMAs of group p, the two chains of a group
// alternating) with the chains started from acc instead of zero.
template <typename T, int D, int NB>
__device__ __forceinline__ void tcontract_acc(f32x4 (&acc)[D / 16], const T* tile, int row16,
                                              const LaneOffsets<T, D>& lo, const BandOperand<T, NB>& P) {
  using TL = Tile<T, D>;
  typedef __attribute__((address_space(3))) bf16x4 lds_v4;
  constexpr int NP = D / 32;
  const char* base = reinterpret_cast<const char*>(tile) + row16 * TL::row_bytes;
  bf16x8 a[NP][NB / 2][2];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int ks = 0; ks < NB / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const char* a1 = base + (lo.tr[p] ^ (8 * e)) + 32 * ks * TL::row_bytes;
        const bf16x4 l4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a1));
        const bf16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a1 + 16 * TL::row_bytes));
        a[p][ks][e] = __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    f32x4 c0 = acc[2 * p], c1 = acc[2 * p + 1];
#pragma unroll
    for (int ks = 0; ks < NB / 2; ++ks) {
      c0 = mma(a[p][ks][0], P.hi[ks], c0);
      c1 = mma(a[p][ks][1], P.hi[ks], c1);
      c0 = mma(a[p][ks][0], P.lo[ks], c0);
      c1 = mma(a[p][ks][1], P.lo[ks], c1);
    }
    acc[2 * p] = c0;
    acc[2 * p + 1] = c1;
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * NB, 0);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p + 1 < NP) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NB, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NB, 0);
  }
}

// The stage list of a workgroup: kind, head, first tile row.
//   0: Lightweight DC phase, window tile of K      (heads 0..H-1)
//   1: main pass, K tile before the window          2: main pass, its V tile
//   3: main pass, window tile of K                  4: main pass, window tile of V
//  -1: past the end (no DMA)
struct FStage {
  int kind, h, row0;
};

template <typename T, int D, bool LDC>
__global__ __launch_bounds__(kFNW * kWave, 1) void fused_fwd_kernel(const FusedArgs a) {
  constexpr int NW = kFNW, BQ = kFBQ, R = kFRows, NBT = kFBlocks;
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(16))) int s_doc[(R + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_xp[NW * 512];
  __shared__ int s_red[NW];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int q0 = tile * BQ;
  const int w0 = q0 - kFWin;  // first key of the window tile
  const int t = q0 + 16 * w + n;
  const bool tval = t < a.T;
  const int tc = tval ? t : a.T - 1;
  const int H = a.H;
  const float sl2 = a.scale * kLog2e;
  float* xp = s_xp + w * 512;
  const LaneOffsets<T, D> lo(g, n);

  // ks0: first token of the run holding q0 (the earliest key of the tile's
  // main attention), found by scanning back 256 ids at a time
  int ks0 = 0;
  {
    const int d0 = a.doc[q0];
    for (int base = q0 - 1; base >= 0; base -= 256) {  // workgroup-uniform
      const int s = base - (int)threadIdx.x;
      const int ds = a.doc[s >= 0 ? s : 0];
      const uint64_t mm = __ballot(s >= 0 && ds != d0);
      if (lane == 0) s_red[w] = mm ? base - (64 * w + __builtin_ctzll(mm)) : -1;
      __syncthreads();
      int best = -1;
#pragma unroll
      for (int i = 0; i < NW; ++i) best = s_red[i] > best ? s_red[i] : best;
      __syncthreads();
      if (best >= 0) {
        ks0 = best + 1;
        break;
      }
    }
  }
  const int span = w0 - ks0;  // run keys before the window tile
  const int nc = span > 0 ? (span + R - 1) / R : 0;
  const int per = 2 * (nc + 1);
  const int npre = LDC ? H : 0;
  const int nstages = npre + H * per;
  auto desc = [&](int G) -> FStage {
    if (G < npre) return {0, G, w0};
    G -= npre;
    if (G >= H * per) return {-1, 0, w0};
    const int h = G / per, r = G - h * per, c = r >> 1;
    if (c < nc) return {(r & 1) ? 2 : 1, h, w0 - R * (nc - c)};
    return {(r & 1) ? 4 : 3, h, w0};
  };
  auto buffer = [&](auto bc) -> T* { return decltype(bc)::value == 0 ? s_x0 : s_x1; };
  auto issue_stage = [&](int G, auto bc) {
    const FStage st = desc(G);
    const bool on = st.kind >= 0;
    issue_tile<T, D, R, NW>(buffer(bc), (st.kind == 2 || st.kind == 4) ? v : k, st.row0, a.T, H, on ? st.h : 0,
                            on);
  };
  // a stage's per-head operands, loaded one stage ahead (unconditionally)
  RowFrag<T, D> qf[2];
  float cc[2] = {0.f, 0.f}, gg[2] = {0.f, 0.f};
  auto load_ops = [&](int G, auto sc) {
    constexpr int S = decltype(sc)::value;
    const FStage st = desc(G);
    const int hh = st.kind >= 0 ? st.h : 0;
    load_row_frag<T, D, true>(qf[S], q + ((size_t)tc * H + hh) * D, g);
    if constexpr (LDC) {  // (no C or G without the Lightweight DC terms)
      cc[S] = a.c[(size_t)tc * H + hh];
      gg[S] = a.g[(size_t)tc * H + hh];
    }
  };

  issue_stage(0, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, w0, a.T);
  load_ops(0, Buf<0>{});
  wait_dma();

  // per-query run start: ks0, or the last run boundary in (q0, t]
  int kslo = ks0;
  for (int s = q0 + 1; s <= t && s < a.T; ++s)
    if (s_doc[s - w0] != s_doc[s - 1 - w0]) kslo = s;
  // admission bits of the Lightweight DC band (bit 4b+i: key q0-112+16w+16b+4g+i)
  uint32_t mbits = 0;
  if constexpr (LDC) {
    const int dt = s_doc[t - w0];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 + 16 * w + 16 * b + 4 * g + i;
        const int s = w0 + r;
        const bool ok = tval & (s >= 0) & (s <= t) & (t - s < a.window) & (s_doc[r] == dt);
        mbits |= (ok ? 1u : 0u) << (4 * b + i);
      }
  }

  f32x4 pbar[kKeyBlocks], pw[NBT], acc[D / 16];
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b) pbar[b] = zero4();
#pragma unroll
  for (int b = 0; b < NBT; ++b) pw[b] = zero4();
#pragma unroll
  for (int r = 0; r < D / 16; ++r) acc[r] = zero4();
  float m = -1e30f, l = 0.f;  // running max (log2 units; finite start) and sum

  // online softmax over a scored tile (key of entry (b, i): row0 + 16b + 4g + i)
  auto online = [&](const f32x4 (&s)[NBT], int row0, bool window) {
    float z[NBT][4];
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NBT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = row0 + 16 * b + 4 * g + i;
        const bool ok = (key >= kslo) & (!window | (key <= t));
        z[b][i] = ok ? s[b][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, z[b][i]);
      }
    mx = wave_max4(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int r = 0; r < D / 16; ++r) acc[r] *= alpha;
    float sum = 0.f;
#pragma unroll
    for (int b = 0; b < NBT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(z[b][i] - mn);
        pw[b][i] = p;
        sum += p;
      }
    l = l * alpha + wave_sum4(sum);
    m = mn;
  };

  auto body = [&](int G, auto bc) {
    constexpr int B = decltype(bc)::value;
    if (G >= nstages) return;  // workgroup-uniform
    wait_dma();
    issue_stage(G + 1, Buf<1 - B>{});
    load_ops(G + 1, Buf<1 - B>{});
    const FStage st = desc(G);
    const T* cur = buffer(bc);
    if (st.kind == 0) {
      // Lightweight DC: the band's softmax, composed into Pbar
      f32x4 sb[kKeyBlocks];
      __builtin_amdgcn_s_setprio(2);
      mma_dcontract_band<T, D, kKeyBlocks>(sb, cur, 16 * (w + 1), lo, qf[B]);
      __builtin_amdgcn_s_setprio(0);
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sb[b][i] = ((mbits >> (4 * b + i)) & 1u) ? sb[b][i] * sl2 : -INFINITY;
          mx = fmaxf(mx, sb[b][i]);
        }
      mx = wave_max4(mx);
      const float mxs = mx == -INFINITY ? 0.f : mx;  // (a query past T: no key)
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sb[b][i] = __builtin_amdgcn_exp2f(sb[b][i] - mxs);
          sum += sb[b][i];
        }
      sum = wave_sum4(sum);
      const float f = sum > 0.f ? cc[B] / sum : 0.f;
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) pbar[b][i] = fmaf(f, sb[b][i], pbar[b][i]);
    } else if (st.kind == 1 || st.kind == 3) {
      f32x4 s[NBT];
      __builtin_amdgcn_s_setprio(2);
      mma_dcontract_band<T, D, NBT>(s, cur, 0, lo, qf[B]);
      __builtin_amdgcn_s_setprio(0);
      online(s, st.row0, st.kind == 3);
    } else if (st.kind == 2) {
      BandOperand<T, NBT> op;
      op.set(pw);
      __builtin_amdgcn_s_setprio(2);
      tcontract_acc<T, D, NBT>(acc, cur, 0, lo, op);
      __builtin_amdgcn_s_setprio(0);
    } else if (st.kind == 4) {
      if constexpr (LDC) {
        // the Lightweight DC term joins the main weights on the wave's band
        // blocks (tile blocks w+1 .. w+8): l G Pbar
        const float f = l * gg[B];
#pragma unroll
        for (int b = 0; b < NBT; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
              const int bb = b - 1 - ww;
              if (bb >= 0 && bb < kKeyBlocks && ww == w) x = pbar[bb][i];
            }
            pw[b][i] = fmaf(f, x, pw[b][i]);
          }
      }
      BandOperand<T, NBT> op;
      op.set(pw);
      __builtin_amdgcn_s_setprio(2);
      tcontract_acc<T, D, NBT>(acc, cur, 0, lo, op);
      __builtin_amdgcn_s_setprio(0);
      const float inv = 1.f / l;  // l >= the diagonal key's weight, > 0
#pragma unroll
      for (int r = 0; r < D / 16; ++r) acc[r] *= inv;
      store_row<T, D>(pending_rows<D>(a.o, q0 + 16 * w, n, a.T, H, st.h, true, 1.f, xp), acc, g, n);
#pragma unroll
      for (int r = 0; r < D / 16; ++r) acc[r] = zero4();
      m = -1e30f;
      l = 0.f;
    }
  };
  for (int G = 0; G < nstages; G += 2) {
    body(G, Buf<0>{});
    body(G + 1, Buf<1>{});
  }
  wait_dma();  // no DMA may land in LDS after the workgroup ends
}

template <typename T, int D>
static hipError_t launch_fused(const FusedArgs& a, bool ldc, hipStream_t st) {
  const int nblk = (a.T + kFBQ - 1) / kFBQ;
  if (ldc)
    hipLaunchKernelGGL((fused_fwd_kernel<T, D, true>), dim3(nblk), dim3(kFNW * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((fused_fwd_kernel<T, D, false>), dim3(nblk), dim3(kFNW * kWave), 0, st, a);
  return hipGetLastError();
}

hipError_t fused_fwd_dispatch(int d, const FusedArgs& a, bool ldc, hipStream_t st) {
  if (d == 128) return launch_fused<bf16_t, 128>(a, ldc, st);
  return launch_fused<bf16_t, 64>(a, ldc, st);
}

}  // namespace ldc
