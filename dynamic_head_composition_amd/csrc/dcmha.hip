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
// stream into LDS by DMA: through three buffers in the query-side kernels
// (one workgroup per CU, so each tile's DMA gets two stages of lead), two in
// the key-side one.
//  * fwd    (query-centric): K phase (raw scores of each source head composed
//           into every target's Z), softmax of every target in registers, V
//           phase (R_h from all heads' P, then O_h).  Saves P and R bands.
//  * bwd_q  (query-centric): V phase (dR of each head, mixed as soon as it
//           is complete into dCW and the running dP of every head, with the
//           saved P), dZ, K phase (raw scores for dCS; dS, dQ; dS bands saved
//           for the key side).
//  * bwd_kv (key-centric): dV_h = R_h^T dO_h and dK_h = scale dS_h^T Q_h from
//           the bands: token contractions only.
// Bands: one 2,048-word block per 16-query block qb and head h, at word
// (qb*H + h) * kBandWords, of plain fp32 words (a band that feeds an MFMA is
// split into bf16 high and low parts where it is loaded).  The R and dS
// bands, read by the key-centric kernel, use the Lightweight DC layout ([key
// block][key 16][query 16]: a key-centric lane reads its 4 queries as one
// 16-byte word group).  The P band is read only by query-centric waves and is
// stored query-major ([key block][query 16][key 16]): lane (g, n) holds keys
// 4g..4g+3 of block b, one 16-byte piece at word b*256 + n*16 + 4g, so it is
// written and read as whole 1 KB lines per block.  Deterministic: no atomics,
// every output element written once.
#include "dcmha_internal.h"
#include "ldc_device.hpp"
#include "ldc_pipeline.hpp"

namespace ldc {

// per-lane scalars of this lane's query t: x[(t*H + row)*H + col]
__device__ __forceinline__ float comp_at(const float* x, int t, int H, int row, int col) {
  return x[((size_t)t * H + row) * H + col];
}

// comp_at when ok, else 0, with the load itself unconditional (from entry
// (0, 0) when !ok): a load under a branch is waited for inside the branch,
// which serialises a row of such loads on the memory latency.
__device__ __forceinline__ float comp_or0(const float* x, int t, int H, int row, int col, bool ok) {
  const float v = comp_at(x, t, H, ok ? row : 0, ok ? col : 0);
  return ok ? v : 0.f;
}

// Write one wave's 16 x 128 band block (accumulator layout, lane (g, n) holds
// words (4g+i)*16 + n of key block b) as 4-byte words.
template <typename T>
__device__ __forceinline__ void write_band(uint32_t* blk, const f32x4 (&x)[kKeyBlocks], float* xp,
                                           int g, int n) {
  uint32_t wv[kKeyBlocks][4];
#pragma unroll
  for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[b][i] = __float_as_uint(x[b][i]);
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
  __shared__ __attribute__((aligned(1024))) T s_x2[R * D];
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
  const int Hp = (H + 2) / 3 * 3;
  constexpr int NIW = tile_insts_per_wave<T, D, R, NW>();
  const int qb = (q0 >> 4) + w;
  const bool wval = q0 + 16 * w < a.T;
  const bool save = a.pband != nullptr;
  float* xp = s_xp + (Elem<T>::bf16 ? w * 512 : 0);
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = K (scores), 1 = V (values; nothing loaded when !OUT).
  // Three LDS buffers: stage j reads buffer j%3 and issues the DMA of stage
  // j+2 into buffer (j+2)%3, which stage j-1 has finished reading.
  auto buffer = [&](auto bc) -> T* {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? s_x0 : (B == 1 ? s_x1 : s_x2);
  };
  auto issue = [&](int phase, int h, bool on, auto bc) {
    issue_tile<T, D, R, NW>(buffer(bc), phase == 0 ? k : v, span0, a.T, H, h, on && (phase == 0 || OUT));
  };
  auto issue_ahead = [&](int phase, int j, auto bc) {
    const NextStage ns = stage_after_next(phase, j, H, Hp, 2);
    issue(ns.phase, ns.head >= 0 ? ns.head : 0, ns.head >= 0, Buf<(decltype(bc)::value + 2) % 3>{});
  };
  // column h' of CS[t] (every target h), pre-scaled by the softmax scale
  auto load_cs = [&](float (&dst)[HM], int hs) {
#pragma unroll
    for (int h = 0; h < HM; ++h) dst[h] = a.scale * comp_or0(a.cs, tc, H, h, hs, h < H);
  };
  // row h of CW[t] (every source h')
  auto load_cw = [&](float (&dst)[HM], int ht) {
#pragma unroll
    for (int h = 0; h < HM; ++h) dst[h] = comp_or0(a.cw, tc, H, ht, h, h < H);
  };

  // Register operands rotate with the buffers: stage j uses slot j%3 and
  // loads slot (j+1)%3 before it issues its DMA.  The V phase's first CW row
  // is loaded here, so that no load is issued between the DMAs of the last
  // K stages and the first V stage.
  RowFrag<T, D> qfb[3];
  float csb[3][HM], cwb[3][HM];
  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  load_row_frag<T, D, true>(qfb[0], q + (size_t)tc * H * D, g);
  load_cs(csb[0], 0);
  load_cw(cwb[0], 0);
  issue(0, 1, 1 < H, Buf<1>{});
  wait_dma_except<NIW>();

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
  // composed scores Z_h of every target head (then P_h in place), started
  // at 0 where the key is admitted and at -inf where it is not: the finite
  // score terms leave -inf in place, so Z is masked without a separate pass
  f32x4 z[HM][kKeyBlocks];
  {
    f32x4 z0[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) z0[b][i] = ((mbits >> (4 * b + i)) & 1u) ? 0.f : -INFINITY;
#pragma unroll
    for (int h = 0; h < HM; ++h)
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b) z[h][b] = z0[b];
  }

  // ---- phase 0 (K_h' staged): Z_h += scale CS[t,h,h'] Q_h' K_h'^T ----
  for_stage_triples(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    constexpr int B1 = (B + 1) % 3;
    const T* cur = buffer(bc);
    wait_dma_except<NIW>();
    const bool real = j < H;
    const int hn = j + 1 < H ? j + 1 : 0;
    load_row_frag<T, D, true>(qfb[B1], q + ((size_t)tc * H + hn) * D, g);
    load_cs(csb[B1], hn);
    __builtin_amdgcn_sched_barrier(0);
    issue_ahead(0, j, bc);
    if (!real) return;
    __builtin_amdgcn_s_setprio(2);
    f32x4 s[kKeyBlocks];
    mma_dcontract_band<T, D, kKeyBlocks>(s, cur, brow, lo, qfb[B]);
    __builtin_amdgcn_s_setprio(0);
    // every slot h < HM, with no branch on H: past H the coefficient is 0
    static_for<0, HM>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float c = csb[B][h];
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[h][b][i] = fmaf(c, s[b][i], z[h][b][i]);
    });
  });

  // ---- softmax of every target head over the window (every slot h < HM,
  // with no branch on H, so the heads' reductions can overlap; slots past H
  // hold finite values and are not stored) ----
  static_for<0, HM>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    {
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
      if (save && wval && h < H) {  // query-major P band: 16 bytes per lane and key block
        uint32_t* blk = a.pband + ((size_t)qb * H + h) * kBandWords;
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, z[h][b]),
                                      reinterpret_cast<u32x4*>(blk + b * 256 + n * 16 + 4 * g));
      }
    }
  });

  // ---- phase 1 (V_h staged): R_h = sum_h' CW[t,h,h'] P_h', O_h = R_h V_h ----
  f32x4 pend[D / 16];
  int pend_h = -1;
  auto pending = [&]() {
    return pending_rows<D>(a.o, q0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0, 1.f, xp);
  };
  auto flush = [&]() {
    if constexpr (OUT) store_row<T, D>(pending(), pend, g, n);
    pend_h = -1;
  };
  for_stage_triples(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = buffer(bc);
    wait_dma_except<NIW>();
    const bool real = j < H;
    load_cw(cwb[(B + 1) % 3], j + 1 < H ? j + 1 : 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_ahead(1, j, bc);
    if (!real) {
      flush();
      return;
    }
    f32x4 r[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b) r[b] = zero4();
    static_for<0, HM>([&](auto hc) {  // (past H the coefficient is 0)
      constexpr int h = decltype(hc)::value;
      const float c = cwb[B][h];
#pragma unroll
      for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) r[b][i] = fmaf(c, z[h][b][i], r[b][i]);
    });
    if (save && wval) write_band<T>(a.rband + ((size_t)qb * H + j) * kBandWords, r, xp, g, n);
    if constexpr (OUT) {
      BandOperand<T> op;
      op.set(r);
      __builtin_amdgcn_s_setprio(2);
      mma_tcontract_pipe<T, D>(pend, cur, brow, lo, op, g, n, pending());
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
  constexpr int HM3 = (HM + 2) / 3 * 3;
  constexpr int NIW = tile_insts_per_wave<T, D, R, NW>();
  constexpr int kCompFloats = BQ * HM * HM;  // the CS or CW rows of the tile's queries
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x2[R * D];
  __shared__ __attribute__((aligned(16))) float s_cw[(kCompFloats + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_cs[(kCompFloats + 63) / 64 * 64];
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
  const int Hp = (H + 2) / 3 * 3;
  const int qb = (q0 >> 4) + w;
  const bool wval = q0 + 16 * w < a.T;
  float* xp = s_xp + (Elem<T>::bf16 ? w * 512 : 0);
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = V (dR), 1 = K (dCS, dS, dQ).  Three LDS buffers: stage j
  // reads buffer j%3 and issues the DMA of stage j+2 into buffer (j+2)%3.
  auto buffer = [&](auto bc) -> T* {
    constexpr int B = decltype(bc)::value;
    return B == 0 ? s_x0 : (B == 1 ? s_x1 : s_x2);
  };
  auto issue = [&](int phase, int h, bool on, auto bc) {
    issue_tile<T, D, R, NW>(buffer(bc), phase == 0 ? v : k, span0, a.T, H, h, on);
  };
  auto issue_ahead = [&](int phase, int j, auto bc) {
    const NextStage ns = stage_after_next(phase, j, H, Hp, 2);
    issue(ns.phase, ns.head >= 0 ? ns.head : 0, ns.head >= 0, Buf<(decltype(bc)::value + 2) % 3>{});
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
  // CW[t] and CS[t] of the tile's queries (rows past T read as zero)
  issue_scalars<kCompFloats, NW>(s_cw, a.cw, 1, 0, q0 * H * H, a.T * H * H, 1, 0);
  issue_scalars<kCompFloats, NW>(s_cs, a.cs, 1, 0, q0 * H * H, a.T * H * H, 1, 0);
  issue(0, 1, 1 < H, Buf<1>{});
  wait_dma_except<NIW>();

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

  // P of every head (heads past H hold 0), and dP_h' = sum_h CW[t,h,h'] dR_h
  // accumulated head by head over the V phase (then dZ_h' in place)
  f32x4 pv[HM][kKeyBlocks], dp[HM][kKeyBlocks];
#pragma unroll
  for (int h = 0; h < HM; ++h)
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[h][b][i] = h < H ? __uint_as_float(pw[h][b][i]) : 0.f;
        dp[h][b][i] = 0.f;
      }
  const float* cw_row = s_cw + (16 * w + n) * H * H;

  // ---- phase 0 (V_h staged): dR_h = dO_h V_h^T, unrolled over the heads;
  // each dR_h is mixed as soon as it is complete, while the next tiles stream
  // in: dCW[t,h,h'] = <dR_h, P_h'>_t and dP_h' += CW[t,h,h'] dR_h ----
  static_for<0, HM3>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int F = j % 2;  // dO fragment slot
    if (j >= Hp) return;
    const T* cur = buffer(Buf<j % 3>{});
    wait_dma_except<NIW>();
    if (j + 1 < H) load_row_frag<T, D>(fb[1 - F], dO + ((size_t)tc * H + j + 1) * D, g);
    __builtin_amdgcn_sched_barrier(0);
    issue_ahead(0, j, Buf<j % 3>{});
    if constexpr (j < HM) {  // (stages past HM are padding)
      if (j >= H) return;
      f32x4 dr[kKeyBlocks];
      __builtin_amdgcn_s_setprio(2);
      mma_dcontract_band<T, D, kKeyBlocks, 1>(dr, cur, brow, lo, fb[F]);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int h2 = 0; h2 < HM; ++h2) {
        float x = 0.f;
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) x = fmaf(dr[b][i], pv[h2][b][i], x);
        x = wave_sum4(x);
        if (tval && g == 0 && h2 < H) a.dcw[((size_t)t * H + j) * H + h2] = x;
      }
#pragma unroll
      for (int h2 = 0; h2 < HM; ++h2) {
        const float c = cw_row[j * H + (h2 < H ? h2 : 0)];
        const float cj = h2 < H ? c : 0.f;
#pragma unroll
        for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) dp[h2][b][i] = fmaf(cj, dr[b][i], dp[h2][b][i]);
      }
    }
  });

  // K phase operands: stage j of the K phase uses slot j%3 and loads slot
  // (j+1)%3.  Column hs of CS[t] comes from LDS.
  RowFrag<T, D> qf[3];
  float csb[3][HM];
  const float* cs_row = s_cs + (16 * w + n) * H * H;
  auto load_cs = [&](float (&dst)[HM], int hs) {
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      const float x = cs_row[(h < H ? h : 0) * H + hs];
      dst[h] = h < H ? x : 0.f;
    }
  };
  load_row_frag<T, D>(qf[0], q + (size_t)tc * H * D, g);
  load_cs(csb[0], 0);

  // ---- dZ_h = P_h (dP_h - rowsum(dP_h P_h)), in place of dP ----
  f32x4 (&dr)[HM][kKeyBlocks] = dp;
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    float dl = 0.f;
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dl = fmaf(dp[h][b][i], pv[h][b][i], dl);
    dl = wave_sum4(dl);
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[h][b][i] = pv[h][b][i] * (dp[h][b][i] - dl);
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
  for_stage_triples(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    constexpr int B1 = (B + 1) % 3;
    const T* cur = buffer(bc);
    wait_dma_except<NIW>();
    const bool real = j < H;
    const int hn = j + 1 < H ? j + 1 : 0;
    load_row_frag<T, D>(qf[B1], q + ((size_t)tc * H + hn) * D, g);
    load_cs(csb[B1], hn);
    __builtin_amdgcn_sched_barrier(0);
    issue_ahead(1, j, bc);
    if (!real) {
      flush();
      return;
    }
    const PendingRow prev = pending();
    __builtin_amdgcn_s_setprio(2);
    f32x4 sv[kKeyBlocks];
    mma_dcontract_band<T, D, kKeyBlocks>(sv, cur, brow, lo, qf[B]);
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
    if (wval) write_band<T>(a.dsband + ((size_t)qb * H + j) * kBandWords, sv, xp, g, n);
    BandOperand<T> dso;
    dso.set(sv);
    __builtin_amdgcn_s_setprio(2);
    mma_tcontract_pipe<T, D>(pend, cur, brow, lo, dso, g, n, prev);
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
  // the band operand of a stage: fp32 words, 0 outside the window
  auto operand = [&](const u32x4 (&u)[kKeyBlocks], BandOperand<T>& op) {
    f32x4 x[kKeyBlocks];
#pragma unroll
    for (int b = 0; b < kKeyBlocks; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[b][i] = keep_admitted(mbits, b, i, __uint_as_float(u[b][i]), 0.f);
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
    operand(rb[B], op);
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
    operand(rb[B], op);
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
