// Full DCMHA composition (scores and weights composed across heads) on the
// Lightweight DC window, forward and backward, for gfx950.
//
// Layer (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
// section "第二刀-砍层内", DCMHA paragraph: a Compose module transforms the
// attention scores and the attention weights across heads, dynamically), read
// as per-query H x H compositions CS[t] (scores, before the softmax) and CW[t]
// (weights, after it):
//   S_h = scale Q_h K_h^T   Z_h = sum_h' CS[t,h,h'] S_h'   P_h = softmax(Z_h)
//   R_h = sum_h' CW[t,h,h'] P_h'                            O_h = R_h V_h
// Backward:
//   dR_h = dO_h V_h^T        dV_h = R_h^T dO_h       dCW[t,h,h'] = <dR_h, P_h'>_t
//   dP_h' = sum_h CW[t,h,h'] dR_h                    dZ_h = P_h (dP_h - <dP_h, P_h>_t)
//   dCS[t,h,h'] = <dZ_h, S_h'>_t    dS_h' = sum_h CS[t,h,h'] dZ_h
//   dQ_h = scale dS_h K_h           dK_h = scale dS_h^T Q_h
//
// Composition couples every head at each (query, key) pair, so a wave keeps
// all heads' 16 x 128 bands of its queries in registers (HM x 32 per lane):
// the query-side kernels run one wave per SIMD (4 waves, 64 queries per
// workgroup) with up to 512 registers per lane.  Tiles of one head at a time
// stream into LDS by DMA, double-buffered, as in the Lightweight DC kernels.
//  * fwd    (query-centric): K phase (raw scores of each source head composed
//           into every target's Z), softmax of every target in registers, V
//           phase (R_h from all heads' P, then O_h).  Saves P and R bands.
//  * bwd_q  (query-centric): V phase (dR of every head, unrolled so each
//           head's band has its own registers), VALU mixing (dCW, dP, dZ with
//           the saved P), K phase (raw scores for dCS; dS, dQ; dS bands saved
//           for the key side).
//  * bwd_kv (key-centric): dV_h = R_h^T dO_h and dK_h = scale dS_h^T Q_h from
//           the bands: token contractions only.
// Bands: one 2,048-word block per 16-query block qb and head h, at word
// (qb*H + h) * kBandWords.  The R and dS bands, read by the key-centric
// kernel, use the Lightweight DC layout ([key block][key 16][query 16]: a
// key-centric lane reads its 4 queries as one 16-byte word group).  The P
// band is read only by query-centric waves and is stored query-major
// ([key block][query 16][key 16]): lane (g, n) holds keys 4g..4g+3 of block
// b, one 16-byte piece at word b*256 + n*16 + 4g, so it is written and read
// as whole 1 KB lines per block.  Deterministic: no atomics, every output
// element written once.
#include "dcmha_internal.h"
#include "ldc_device.hpp"
#include "ldc_pipeline.hpp"

namespace ldc {

// per-lane scalars of this lane's query t: x[(t*H + row)*H + col]
__device__ __forceinline__ float comp_at(const float* x, int t, int H, int row, int col) {
  return x[((size_t)t * H + row) * H + col];
}

// Write one wave's 16 x 128 band block (accumulator layout, lane (g, n) holds
// words (4g+i)*16 + n of key block b) as 4-byte words.
template <typename T, bool ENCODE>
__device__ __forceinline__ void write_band(uint32_t* blk, const f32x4 (&x)[kKeyBlocks], float* xp,
                                           int g, int n) {
  uint32_t wv[kKeyBlocks][4];
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[b][i] = ENCODE ? band_encode<T>(x[b][i]) : __float_as_uint(x[b][i]);
  if constexpr (Elem<T>::bf16) {
    store_band_block(blk, wv, xp, g, n);
  } else {
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) blk[b * 256 + (4 * g + i) * 16 + n] = wv[b][i];
  }
}

// ---------------------------------------------------------------------------
// forward
// OUT = false: P and R bands only (the backward's recomputation), no O and no
// V traffic.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int HM, bool OUT>
__global__ __launch_bounds__(NW * kWave, 1) void dcmha_fwd_kernel(const DcFwdArgs a) {
  constexpr int BQ = 16 * NW;
  constexpr int R = BQ + kHalo;
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(16))) int s_doc[(R + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_xp[Elem<T>::bf16 ? NW * 512 : 4];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int q0 = tile * BQ;
  const int span0 = q0 - kHalo;
  const int brow = 16 * w;
  const int t = q0 + 16 * w + n;
  const bool tval = t < a.T;
  const int tc = tval ? t : a.T - 1;
  const int H = a.H;
  const int Hp = (H + 1) & ~1;
  const int qb = (q0 >> 4) + w;
  const bool wval = q0 + 16 * w < a.T;
  const bool save = a.pband != nullptr;
  float* xp = s_xp + (Elem<T>::bf16 ? w * 512 : 0);
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = K (scores), 1 = V (values; nothing loaded when !OUT)
  auto issue = [&](int phase, int h, bool on, auto bc) {
    T* buf = decltype(bc)::value == 0 ? s_x0 : s_x1;
    issue_tile<T, D, R, NW>(buf, phase == 0 ? k : v, span0, a.T, H, h, on && (phase == 0 || OUT));
  };
  auto issue_next = [&](int phase, int j, auto bc) {
    const NextStage ns = next_stage(phase, j, H, Hp, 2);
    issue(ns.phase, ns.head >= 0 ? ns.head : 0, ns.head >= 0, Buf<1 - decltype(bc)::value>{});
  };
  // column h' of CS[t] (every target h), pre-scaled by the softmax scale
  auto load_cs = [&](float (&dst)[HM], int hs) {
#pragma unroll
    for (int h = 0; h < HM; ++h) dst[h] = h < H ? a.scale * comp_at(a.cs, tc, H, h, hs) : 0.f;
  };
  // row h of CW[t] (every source h')
  auto load_cw = [&](float (&dst)[HM], int ht) {
#pragma unroll
    for (int h = 0; h < HM; ++h) dst[h] = h < H ? comp_at(a.cw, tc, H, ht, h) : 0.f;
  };

  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  RowFrag<T, D> qfb[2];
  float csb[2][HM];
  load_row_frag<T, D, true>(qfb[0], q + (size_t)tc * H * D, g);
  load_cs(csb[0], 0);
  wait_dma();

  uint32_t mbits = 0;
  {
    const int dt = s_doc[brow + kHalo + n];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int s = span0 + r;
        const bool ok = tval & (s >= 0) & (s <= t) & (t - s < a.window) & (s_doc[r] == dt);
        mbits |= (ok ? 1u : 0u) << (4 * b + i);
      }
  }
  const uint32_t full = full_blocks(mbits);

  // composed scores Z_h of every target head (then P_h in place)
  f32x4 z[HM][kKeyBlocks];
#pragma unroll
  for (int h = 0; h < HM; ++h)
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) z[h][b] = zero4();

  // ---- phase 0 (K_h' staged): Z_h += scale CS[t,h,h'] Q_h' K_h'^T ----
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    const int hn = j + 1 < H ? j + 1 : 0;
    load_row_frag<T, D, true>(qfb[1 - B], q + ((size_t)tc * H + hn) * D, g);
    load_cs(csb[1 - B], hn);
    __builtin_amdgcn_sched_barrier(0);
    issue_next(0, j, bc);
    if (!real) return;
    __builtin_amdgcn_s_setprio(2);
    f32x4 s[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) s[b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, qfb[B]);
    __builtin_amdgcn_s_setprio(0);
    static_for<0, HM>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if (h < H) {
        const float c = csb[B][h];
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[h][b][i] = fmaf(c, s[b][i], z[h][b][i]);
      }
    });
  });

  // ---- softmax of every target head over the window ----
  static_for<0, HM>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    if (h < H) {
      mask_band(z[h], mbits, full, -INFINITY);
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[h][b][i]);
      mx = wave_max4(mx);
      const float mxs = mx == -INFINITY ? 0.f : mx * kLog2e;  // a row with no key: all terms 0
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2_scaled(z[h][b][i], kLog2e, mxs);
          z[h][b][i] = e;
          sum += e;
        }
      sum = wave_sum4(sum);
      const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b) z[h][b] *= inv;
      if (save && wval) {  // query-major P band: 16 bytes per lane and key block
        uint32_t* blk = a.pband + ((size_t)qb * H + h) * kBandWords;
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
          __builtin_nontemporal_store(
              u32x4{band_encode<T>(z[h][b][0]), band_encode<T>(z[h][b][1]), band_encode<T>(z[h][b][2]),
                    band_encode<T>(z[h][b][3])},
              reinterpret_cast<u32x4*>(blk + b * 256 + n * 16 + 4 * g));
      }
    }
  });

  // ---- phase 1 (V_h staged): R_h = sum_h' CW[t,h,h'] P_h', O_h = R_h V_h ----
  float cwb[2][HM];
  load_cw(cwb[0], 0);
  f32x4 pend[D / 16];
  int pend_h = -1;
  auto pending = [&]() {
    return pending_rows<D>(a.o, q0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0, 1.f, xp);
  };
  auto flush = [&]() {
    if constexpr (OUT) store_row<T, D>(pending(), pend, g, n);
    pend_h = -1;
  };
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    load_cw(cwb[1 - B], j + 1 < H ? j + 1 : 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_next(1, j, bc);
    if (!real) {
      flush();
      return;
    }
    f32x4 r[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) r[b] = zero4();
    static_for<0, HM>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if (h < H) {
        const float c = cwb[B][h];
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) r[b][i] = fmaf(c, z[h][b][i], r[b][i]);
      }
    });
    if (save && wval) write_band<T, true>(a.rband + ((size_t)qb * H + j) * kBandWords, r, xp, g, n);
    if constexpr (OUT) {
      BandOperand<T> op;
      op.set(r);
      __builtin_amdgcn_s_setprio(2);
      mma_tcontract<T, D>(pend, cur, brow, lo, op, g, n, pending());
      __builtin_amdgcn_s_setprio(0);
      pend_h = j;
    }
  });
  flush();
  wait_dma();  // no DMA may land in LDS after the workgroup ends
}

// ---------------------------------------------------------------------------
// bwd_q: per query (lane = query column n, 32 band entries per head)
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int HM>
__global__ __launch_bounds__(NW * kWave, 1) void dcmha_bwd_q_kernel(const DcBwdArgs a) {
  constexpr int BQ = 16 * NW;
  constexpr int R = BQ + kHalo;
  constexpr int HMp = HM;
  static_assert(HM % 2 == 0, "the V phase is unrolled in stage pairs");
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(16))) int s_doc[(R + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_xp[Elem<T>::bf16 ? NW * 512 : 4];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const T* __restrict__ dO = static_cast<const T*>(a.dO);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int q0 = tile * BQ;
  const int span0 = q0 - kHalo;
  const int brow = 16 * w;
  const int t = q0 + 16 * w + n;
  const bool tval = t < a.T;
  const int tc = tval ? t : a.T - 1;
  const int H = a.H;
  const int Hp = (H + 1) & ~1;
  const int qb = (q0 >> 4) + w;
  const bool wval = q0 + 16 * w < a.T;
  float* xp = s_xp + (Elem<T>::bf16 ? w * 512 : 0);
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = V (dR), 1 = K (dCS, dS, dQ)
  auto issue = [&](int phase, int h, bool on, auto bc) {
    T* buf = decltype(bc)::value == 0 ? s_x0 : s_x1;
    issue_tile<T, D, R, NW>(buf, phase == 0 ? v : k, span0, a.T, H, h, on);
  };
  auto issue_next = [&](int phase, int j, auto bc) {
    const NextStage ns = next_stage(phase, j, H, Hp, 2);
    issue(ns.phase, ns.head >= 0 ? ns.head : 0, ns.head >= 0, Buf<1 - decltype(bc)::value>{});
  };

  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  RowFrag<T, D> fb[2];
  load_row_frag<T, D>(fb[0], dO + (size_t)tc * H * D, g);
  // Every head's saved P of this wave's queries (query-major band: one
  // 16-byte piece per head and key block), in flight during the V phase.
  u32x4 pw[HM][kKeyBlocks];
  {
    const uint32_t* pblk = a.pband + (size_t)(wval ? qb : 0) * H * kBandWords;
#pragma unroll
    for (int h = 0; h < HM; ++h)
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
        pw[h][b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            pblk + (size_t)(h < H ? h : 0) * kBandWords + b * 256 + n * 16 + 4 * g));
  }
  wait_dma();

  uint32_t mbits = 0;
  {
    const int dt = s_doc[brow + kHalo + n];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int s = span0 + r;
        const bool ok = tval & (s >= 0) & (s <= t) & (t - s < a.window) & (s_doc[r] == dt);
        mbits |= (ok ? 1u : 0u) << (4 * b + i);
      }
  }

  // dR_h of every head (then dP_h', then dZ_h, in place)
  f32x4 dr[HM][kKeyBlocks];
#pragma unroll
  for (int h = 0; h < HM; ++h)
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) dr[h][b] = zero4();

  // ---- phase 0 (V_h staged): dR_h = dO_h V_h^T, unrolled over the heads ----
  auto vstage = [&](auto jc, auto bc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int B = decltype(bc)::value;
    if (j >= Hp) return;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    if (j + 1 < H) load_row_frag<T, D>(fb[1 - B], dO + ((size_t)tc * H + j + 1) * D, g);
    __builtin_amdgcn_sched_barrier(0);
    issue_next(0, j, bc);
    if (j >= H) return;
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) dr[j][b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, fb[B]);
    __builtin_amdgcn_s_setprio(0);
  };
  static_for<0, HMp / 2>([&](auto pc) {
    constexpr int j0 = 2 * decltype(pc)::value;
    vstage(std::integral_constant<int, j0>{}, Buf<0>{});
    vstage(std::integral_constant<int, j0 + 1>{}, Buf<1>{});
  });

  // K phase operands of the first head, in flight during the mixing
  float csb[2][HM];
  auto load_cs = [&](float (&dst)[HM], int hs) {
#pragma unroll
    for (int h = 0; h < HM; ++h) dst[h] = h < H ? comp_at(a.cs, tc, H, h, hs) : 0.f;
  };
  load_row_frag<T, D>(fb[0], q + (size_t)tc * H * D, g);
  load_cs(csb[0], 0);

  // ---- mixing: dCW = dR P^T, dP = CW^T dR, dZ = P (dP - rowsum(dP P)) ----
  {
    // P of every head, decoded in place (heads past H hold 0)
    f32x4 pv[HM][kKeyBlocks];
#pragma unroll
    for (int h = 0; h < HM; ++h)
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = pw[h][b][i];
          pv[h][b][i] = h < H ? band_decode<T>(u) : 0.f;
        }
    // dCW[t,h,h'] = sum_s dR_h P_h'
#pragma unroll
    for (int h = 0; h < HM; ++h)
#pragma unroll
      for (int h2 = 0; h2 < HM; ++h2) {
        float x = 0.f;
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) x = fmaf(dr[h][b][i], pv[h2][b][i], x);
        x = wave_sum4(x);
        if (tval && g == 0 && h < H && h2 < H) a.dcw[((size_t)t * H + h) * H + h2] = x;
      }
    // dP_h' = sum_h CW[t,h,h'] dR_h (in place), and rowsum(dP_h' P_h')
    float cwr[HM][HM];
#pragma unroll
    for (int h = 0; h < HM; ++h)
#pragma unroll
      for (int h2 = 0; h2 < HM; ++h2) cwr[h][h2] = (h < H && h2 < H) ? comp_at(a.cw, tc, H, h, h2) : 0.f;
    float dlt[HM];
#pragma unroll
    for (int h = 0; h < HM; ++h) dlt[h] = 0.f;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float dp[HM];
#pragma unroll
        for (int h2 = 0; h2 < HM; ++h2) {
          float x = 0.f;
#pragma unroll
          for (int h = 0; h < HM; ++h) x = fmaf(cwr[h][h2], dr[h][b][i], x);
          dp[h2] = x;
        }
#pragma unroll
        for (int h2 = 0; h2 < HM; ++h2) {
          dr[h2][b][i] = dp[h2];
          dlt[h2] = fmaf(dp[h2], pv[h2][b][i], dlt[h2]);
        }
      }
    // dZ_h = P_h (dP_h - rowsum(dP_h P_h))
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      const float dl = wave_sum4(dlt[h]);
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) dr[h][b][i] = pv[h][b][i] * (dr[h][b][i] - dl);
    }
  }

  // ---- phase 1 (K_h' staged): S_h', dCS[.,h'], dS_h', dQ_h' ----
  f32x4 pend[D / 16];
  int pend_h = -1;
  auto pending = [&]() {
    return pending_rows<D>(a.dq, q0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0,
                           a.scale, xp);
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
    const int hn = j + 1 < H ? j + 1 : 0;
    load_row_frag<T, D>(fb[1 - B], q + ((size_t)tc * H + hn) * D, g);
    load_cs(csb[1 - B], hn);
    __builtin_amdgcn_sched_barrier(0);
    issue_next(1, j, bc);
    if (!real) {
      flush();
      return;
    }
    const PendingRow prev = pending();
    __builtin_amdgcn_s_setprio(2);
    f32x4 sv[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) sv[b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, fb[B]);
    __builtin_amdgcn_s_setprio(0);
    // dCS[t,h,j] = sum_s dZ_h S_j (S_j = scale x the contraction)
    static_for<0, HM>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if (h < H) {
        float x = 0.f;
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) x = fmaf(dr[h][b][i], sv[b][i], x);
        x = wave_sum4(x) * a.scale;
        if (tval && g == 0) a.dcs[((size_t)t * H + h) * H + j] = x;
      }
    });
    // dS_j = sum_h CS[t,h,j] dZ_h (0 where masked: dZ is)
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.f;
#pragma unroll
        for (int h = 0; h < HM; ++h) x = fmaf(csb[B][h], dr[h][b][i], x);
        sv[b][i] = x;
      }
    if (wval) write_band<T, false>(a.dsband + ((size_t)qb * H + j) * kBandWords, sv, xp, g, n);
    BandOperand<T> dso;
    dso.set(sv);
    __builtin_amdgcn_s_setprio(2);
    mma_tcontract<T, D>(pend, cur, brow, lo, dso, g, n, prev);
    __builtin_amdgcn_s_setprio(0);
    pend_h = j;
  });
  flush();
  wait_dma();
}

// ---------------------------------------------------------------------------
// bwd_kv: per key (lane = key column n; rows 4g+i of query block b)
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * kWave) void dcmha_bwd_kv_kernel(const DcBwdArgs a) {
  constexpr int BK = 16 * NW;
  constexpr int R = BK + kHalo;  // query rows [k0, k0 + BK + 112)
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(16))) int s_doc[(R + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_xp[Elem<T>::bf16 ? NW * 512 : 4];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ dO = static_cast<const T*>(a.dO);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int k0 = tile * BK;
  const int span0 = k0;
  const int brow = 16 * w;
  const int s = k0 + 16 * w + n;
  const bool sval = s < a.T;
  const int H = a.H;
  const int Hp = (H + 1) & ~1;
  float* xp = s_xp + (Elem<T>::bf16 ? w * 512 : 0);
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = dO (dV from the R bands), 1 = Q (dK from the dS bands)
  auto issue = [&](int phase, int h, bool on, auto bc) {
    T* buf = decltype(bc)::value == 0 ? s_x0 : s_x1;
    issue_tile<T, D, R, NW>(buf, phase == 0 ? dO : q, span0, a.T, H, h, on);
  };
  auto issue_next = [&](int phase, int j, auto bc) {
    const NextStage ns = next_stage(phase, j, H, Hp, 2);
    issue(ns.phase, ns.head >= 0 ? ns.head : 0, ns.head >= 0, Buf<1 - decltype(bc)::value>{});
  };
  // This lane's (key, 4 queries) entries of head h's band: query block kq + b,
  // key block 7 - b, 16 bytes per block (blocks past the stream clamp to the
  // last one and are masked below).
  const int kq = (k0 >> 4) + w;
  const int nqb = (a.T + 15) >> 4;
  auto load_band = [&](u32x4 (&dst)[kKeyBlocks], const uint32_t* band, int h) {
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) {
      const int qbk = kq + b < nqb ? kq + b : nqb - 1;
      dst[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          band + ((size_t)qbk * H + h) * kBandWords + (7 - b) * 256 + n * 16 + 4 * g));
    }
  };

  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  u32x4 rb[2][kKeyBlocks];
  load_band(rb[0], a.rband, 0);
  wait_dma();

  uint32_t mbits = 0;  // bit 4b+i <-> query row brow + 16b + 4g + i
  {
    const int ds = s_doc[brow + n];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int tq = span0 + r;
        const bool ok = sval & (tq < a.T) & (tq >= s) & (tq - s < a.window) & (s_doc[r] == ds);
        mbits |= (ok ? 1u : 0u) << (4 * b + i);
      }
  }

  f32x4 pend[D / 16];
  int pend_h = -1;
  auto pending = [&](float* dst, float scale) {
    return pending_rows<D>(dst, k0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0, scale, xp);
  };
  // the band operand of a stage: decoded, 0 outside the window
  auto operand = [&](const u32x4 (&u)[kKeyBlocks], bool enc, BandOperand<T>& op) {
    f32x4 x[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[b][i] = keep_admitted(mbits, b, i, enc ? band_decode<T>(u[b][i]) : __uint_as_float(u[b][i]), 0.f);
    op.set(x);
  };

  // ---- phase 0 (dO_h staged): dV_h = R_h^T dO_h ----
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    if (j + 1 < H)
      load_band(rb[1 - B], a.rband, j + 1);
    else if (j == Hp - 1)
      load_band(rb[1 - B], a.dsband, 0);  // the Q phase's first band
    __builtin_amdgcn_sched_barrier(0);
    issue_next(0, j, bc);
    if (!real) {
      store_row<T, D>(pending(a.dv, 1.f), pend, g, n);
      pend_h = -1;
      return;
    }
    BandOperand<T> op;
    operand(rb[B], true, op);
    __builtin_amdgcn_s_setprio(2);
    mma_tcontract<T, D>(pend, cur, brow, lo, op, g, n, pending(a.dv, 1.f));
    __builtin_amdgcn_s_setprio(0);
    pend_h = j;
  });

  // ---- phase 1 (Q_h staged): dK_h = scale dS_h^T Q_h ----
  bool first = true;
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    const PendingRow prev = pending(first ? a.dv : a.dk, first ? 1.f : a.scale);
    first = false;
    if (j + 1 < H) load_band(rb[1 - B], a.dsband, j + 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_next(1, j, bc);
    if (!real) {
      store_row<T, D>(prev, pend, g, n);
      pend_h = -1;
      return;
    }
    BandOperand<T> op;
    operand(rb[B], false, op);
    __builtin_amdgcn_s_setprio(2);
    mma_tcontract<T, D>(pend, cur, brow, lo, op, g, n, prev);
    __builtin_amdgcn_s_setprio(0);
    pend_h = j;
  });
  store_row<T, D>(pending(a.dk, a.scale), pend, g, n);
  wait_dma();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int HM>
static hipError_t launch_dc_fwd(const DcFwdArgs& a, bool out, hipStream_t st) {
  constexpr int BQ = 16 * NW;
  const int nblk = (int)((a.T + BQ - 1) / BQ);
  if (out)
    hipLaunchKernelGGL((dcmha_fwd_kernel<T, D, NW, HM, true>), dim3(nblk), dim3(NW * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((dcmha_fwd_kernel<T, D, NW, HM, false>), dim3(nblk), dim3(NW * kWave), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D, int NW, int NWK, int HM>
static hipError_t launch_dc_bwd(const DcBwdArgs& a, int parts, hipStream_t st) {
  if (parts & 1) {
    const int nblk = (int)((a.T + 16 * NW - 1) / (16 * NW));
    hipLaunchKernelGGL((dcmha_bwd_q_kernel<T, D, NW, HM>), dim3(nblk), dim3(NW * kWave), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (parts & 2) {
    const int nblk = (int)((a.T + 16 * NWK - 1) / (16 * NWK));
    hipLaunchKernelGGL((dcmha_bwd_kv_kernel<T, D, NWK>), dim3(nblk), dim3(NWK * kWave), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t dcmha_fwd_dispatch(int dtype, int d, const DcFwdArgs& a, bool out, hipStream_t st) {
  const bool small = a.H <= 2;
  if (dtype == 0) {
    if (d == 128) return small ? launch_dc_fwd<bf16_t, 128, 4, 2>(a, out, st) : launch_dc_fwd<bf16_t, 128, 4, 6>(a, out, st);
    if (d == 64) return small ? launch_dc_fwd<bf16_t, 64, 4, 2>(a, out, st) : launch_dc_fwd<bf16_t, 64, 4, 6>(a, out, st);
  } else {
    if (d == 64) return small ? launch_dc_fwd<float, 64, 4, 2>(a, out, st) : launch_dc_fwd<float, 64, 4, 6>(a, out, st);
  }
  return hipErrorInvalidValue;
}

hipError_t dcmha_bwd_dispatch(int dtype, int d, const DcBwdArgs& a, int parts, hipStream_t st) {
  const bool small = a.H <= 2;
  if (dtype == 0) {
    if (d == 128)
      return small ? launch_dc_bwd<bf16_t, 128, 4, 8, 2>(a, parts, st) : launch_dc_bwd<bf16_t, 128, 4, 8, 6>(a, parts, st);
    if (d == 64)
      return small ? launch_dc_bwd<bf16_t, 64, 4, 8, 2>(a, parts, st) : launch_dc_bwd<bf16_t, 64, 4, 8, 6>(a, parts, st);
  } else {
    if (d == 64)
      return small ? launch_dc_bwd<float, 64, 4, 4, 2>(a, parts, st) : launch_dc_bwd<float, 64, 4, 4, 6>(a, parts, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ldc
