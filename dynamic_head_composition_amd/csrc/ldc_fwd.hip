// Lightweight DC forward pass for gfx950.
//
// Computation (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
// section "第二刀-砍层内", Lightweight DC paragraph): per head a causal softmax
// over a short local window, the heads' maps composed after the softmax into
// one shared map, and the shared map applied to every head's values with a
// per-head scale.
//
// Work split: one workgroup of NW waves owns BQ = 16*NW consecutive queries;
// wave w owns 16 of them and the 128-token key band [q-112, q+16) that covers
// their windows.  The workgroup streams the key span [q0-112, q0+BQ) of one
// head at a time into LDS by DMA, double-buffered: all heads' K (score
// phase), then all heads' V (value phase); the next head's tile is in flight
// while the current one is used.
//
// Scores are computed transposed, S^T = K Q^T, so each lane owns one query
// column and 32 of its band entries: the softmax row reductions are in-lane
// plus two cross-lane steps, and the composed map Pbar^T stays in registers
// where it is directly the B operand of O^T = V^T Pbar^T (V^T read with LDS
// transpose loads).  When the caller asks for the saved state, each wave also
// writes its 16 x 128 block of Pbar and each head's softmax statistics for the
// backward pass.
#include "ldc_device.hpp"
#include "ldc_internal.h"
#include "ldc_pipeline.hpp"

namespace ldc {

// At d = 64 (bf16) a workgroup's LDS (77 KB) leaves room for a second one per
// CU; asking for four waves per SIMD keeps the kernel within 128 VGPRs without
// spills, and two workgroups per CU measured 4% faster there.
// VAL = false: the score phase only, writing the saved state (shared-map band
// and softmax statistics) and no O: the backward pass's recomputation when the
// caller kept no saved state.
// NB: key blocks per band (8 for windows up to 113 keys, 10 up to 128).
template <typename T, int D, int NW, int NB, bool VAL = true>
__global__ __launch_bounds__(NW * kWave, (D == 64 && Elem<T>::bf16 && NB == 8) ? 4 : 1) void fwd_kernel(
    const FwdArgs a) {
  constexpr int BQ = 16 * NW;
  constexpr int kHalo = halo_rows<NB>();
  // tile rows: the span, rounded up to whole DMA instructions (32-byte rows
  // fill 32 rows per instruction)
  constexpr int R = (BQ + kHalo + Tile<T, D>::rows_per_inst - 1) / Tile<T, D>::rows_per_inst *
                    Tile<T, D>::rows_per_inst;
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(16))) int s_doc[(R + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_xp[Elem<T>::bf16 ? NW * 512 : 4];  // row stores

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  float* __restrict__ o = a.o;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int q0 = tile * BQ;
  const int span0 = q0 - kHalo;  // token of LDS row 0
  const int brow = 16 * w;       // LDS row of this wave's band start (token qw - kHalo)
  const int t = q0 + 16 * w + n; // this lane's query
  const bool tval = t < a.T;
  const int tc = tval ? t : a.T - 1;  // a valid row for unconditional loads
  const int H = a.H;
  const int Hp = (H + 1) & ~1;
  const LaneOffsets<T, D> lo(g, n);

  auto issue = [&](int phase, int h, bool on, auto bc) {
    T* buf = decltype(bc)::value == 0 ? s_x0 : s_x1;
    issue_tile<T, D, R, NW>(buf, phase == 0 ? k : v, span0, a.T, H, h, on);
  };
  auto issue_next = [&](int phase, int j, auto bc) {
    const NextStage ns = next_stage(phase, j, H, Hp, VAL ? 2 : 1);
    issue(ns.phase == 0 ? 0 : 1, ns.head >= 0 ? ns.head : 0, ns.head >= 0,
          Buf<1 - decltype(bc)::value>{});
  };
  // Prologue: the first tile, the document ids and the first head's register
  // operands are all in flight before the one wait.
  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  // Per-head register operands are loaded one stage ahead (slot j%2 holds
  // head j), so their latency overlaps the previous stage's compute.  Each Q
  // row is read once here, so its loads are non-temporal (measured 1% faster
  // over the forward and backward together; the backward kernels' register
  // operands measured slower that way and load normally).
  RowFrag<T, D> qfb[2];
  float chb[2];  // rows t >= T are fully masked (coef 0), their loads use row T-1
  load_row_frag<T, D, true>(qfb[0], q + (size_t)tc * H * D, g);
  chb[0] = a.c[(size_t)tc * H];
  wait_dma();

  // Admission mask of this lane's 4NB band entries: bit 4b+i <-> key row brow+16b+4g+i.
  MaskT<NB> mbits = 0;
  {
    const int dt = s_doc[brow + kHalo + n];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int s = span0 + r;
        const bool ok = tval & (s >= 0) & (s <= t) & (t - s < a.window) & (s_doc[r] == dt);
        mbits |= (MaskT<NB>)(ok ? 1u : 0u) << (4 * b + i);
      }
  }
  const uint32_t full = full_blocks<NB>(mbits);  // wave-uniform

  const float sl2 = a.scale * kLog2e;
  f32x4 pb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) pb[b] = zero4();

  // Softmax statistics of each head go to the saved state for the backward
  // pass; the store is deferred past the next stage's barrier.
  float st_mx = 0.f, st_inv = 0.f;
  int st_h = -1;
  auto flush_stats = [&]() {
    if (st_h >= 0 && a.band && tval && g == 0)
      a.stats[(size_t)t * H + st_h] = float2{st_mx, st_inv};
    st_h = -1;
  };

  // ---- phase 0 (K_h staged): scores, softmax, composition into Pbar^T ----
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    const int hn = j + 1 < H ? j + 1 : 0;
    load_row_frag<T, D, true>(qfb[1 - B], q + ((size_t)tc * H + hn) * D, g);
    chb[1 - B] = a.c[(size_t)tc * H + hn];
    __builtin_amdgcn_sched_barrier(0);
    issue_next(0, j, bc);
    __builtin_amdgcn_s_setprio(2);
    if (!real) return;
    const RowFrag<T, D>& qf = qfb[B];
    const float ch = chb[B];
    flush_stats();

    f32x4 sc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) sc[b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, qf);
    // Raw scores; entries outside the window or document become -inf (only
    // in blocks not fully admitted), so max and exp need no further masking.
    // The scale is positive, so rounding(s * scale*log2e) is monotonic in s
    // and the row max of the scaled scores is the scaled raw max: the max
    // entry gets exp2(0) = 1 exactly (a one-key window gives P = 1).
    mask_band(sc, mbits, full, -INFINITY);
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[b][i]);
    __builtin_amdgcn_s_setprio(0);
    mx = wave_max4(mx);
    const float mxs = mx == -INFINITY ? 0.f : mx * sl2;  // a row with no key: all terms 0
    float sum = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2_scaled(sc[b][i], sl2, mxs);
        sc[b][i] = e;
        sum += e;
      }
    sum = wave_sum4(sum);
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    const float coef = ch * inv;
    st_mx = mxs;
    st_inv = inv;
    st_h = j;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[b][i] += coef * sc[b][i];
  });

  flush_stats();
  BandOperand<T, NB> pop;
  pop.set(pb);
  if (a.band && q0 + 16 * w < a.T) {
    // the wave's 16 x 16NB shared map, for the backward pass
    uint32_t* blk = a.band + (size_t)((q0 >> 4) + w) * band_words<NB>();
    if constexpr (Elem<T>::bf16) {
      uint32_t wv[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[b][i] = band_encode<T>(pb[b][i]);
      store_band_block(blk, wv, s_xp + w * 512, g, n);
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) blk[b * 256 + (4 * g + i) * 16 + n] = band_encode<T>(pb[b][i]);
    }
  }

  if constexpr (!VAL) {
    wait_dma();  // no DMA may land in LDS after the workgroup ends
    return;
  }

  // ---- phase 1 (V_h staged): O^T_h = V_h^T Pbar^T, scaled by G ----
  // A stage's output row is stored during the next stage, spread over its
  // contraction, after that stage's DMA has been issued.
  float ghb[2];
  ghb[0] = a.g[(size_t)tc * H];
  f32x4 pend[D / 16];
  int pend_h = -1;
  auto pending = [&]() {
    return pending_rows<D>(o, q0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0, 1.f,
                           s_xp + (Elem<T>::bf16 ? w * 512 : 0));
  };
  auto flush = [&]() {
    store_row<T, D>(pending(), pend, g, n);
    pend_h = -1;
  };
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    ghb[1 - B] = a.g[(size_t)tc * H + (j + 1 < H ? j + 1 : 0)];
    __builtin_amdgcn_sched_barrier(0);
    issue_next(1, j, bc);
    __builtin_amdgcn_s_setprio(2);
    if (!real) {
      flush();
      return;
    }
    const float gh = ghb[B];
    mma_tcontract<T, D, NB>(pend, cur, brow, lo, pop, g, n, pending());
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int r = 0; r < D / 16; ++r) pend[r] *= gh;
    pend_h = j;
  });
  flush();
  wait_dma();  // no DMA may land in LDS after the workgroup ends
}

template <typename T, int D, int NW, int NB>
static hipError_t launch_fwd(const FwdArgs& a, bool value, hipStream_t st) {
  constexpr int BQ = 16 * NW;
  const int nblk = (int)((a.T + BQ - 1) / BQ);
  if (value)
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, NB, true>), dim3(nblk), dim3(NW * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, NB, false>), dim3(nblk), dim3(NW * kWave), 0, st, a);
  return hipGetLastError();
}

// Windows up to 113 keys: 8-block bands.  Wider windows (up to 128): 10-block
// bands in 4-wave workgroups, one wave per SIMD (the larger band arrays need
// more than 256 registers; the longer halo needs the LDS of the 8-wave tiles).
hipError_t fwd_dispatch(int dtype, int d, const FwdArgs& a, bool value, hipStream_t st) {
  const bool wide = a.window > kMaxWindow;
  if (dtype == 0) {
    if (d == 128) return wide ? launch_fwd<bf16_t, 128, 4, 10>(a, value, st) : launch_fwd<bf16_t, 128, 8, 8>(a, value, st);
    if (d == 64) return wide ? launch_fwd<bf16_t, 64, 4, 10>(a, value, st) : launch_fwd<bf16_t, 64, 8, 8>(a, value, st);
    if (d == 16) return wide ? launch_fwd<bf16_t, 16, 4, 10>(a, value, st) : launch_fwd<bf16_t, 16, 8, 8>(a, value, st);
  } else {
    if (d == 128 && !wide) return launch_fwd<float, 128, 2, 8>(a, value, st);
    if (d == 64) return wide ? launch_fwd<float, 64, 4, 10>(a, value, st) : launch_fwd<float, 64, 4, 8>(a, value, st);
    if (d == 16) return wide ? launch_fwd<float, 16, 4, 10>(a, value, st) : launch_fwd<float, 16, 4, 8>(a, value, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ldc
