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
// The forward pass saves the shared map (as a band of 16x16 blocks) and each
// head's softmax statistics, so neither backward kernel recomputes Pbar.
// Two deterministic kernels, no atomics and no zero-fill:
//  * bwd_q  (query-centric, like the forward): each wave owns 16 queries.
//    Phases over the heads: V_h staged (B_h, dPbar, dG); then, with dPbar
//    complete and written to the workspace band, K_h staged (P_h from the
//    scores and the saved statistics, dC, dS, dQ).
//  * bwd_kv (key-centric): each wave owns 16 keys and the 16*NB queries whose
//    windows can hold them; Pbar and dPbar come from the two bands.  Phases:
//    dO_h staged (dV_h), then Q_h staged (P_h, dS_h, dK_h).
// Neither writes a T x window x H map: per-head quantities live in registers
// of the wave that needs them.  Tiles stream into LDS by DMA, double-buffered,
// as in the forward pass.
#include "ldc_device.hpp"
#include "ldc_internal.h"
#include "ldc_pipeline.hpp"

#include <mutex>

namespace ldc {

// ---------------------------------------------------------------------------
// bwd_q: per query.  Transposed orientation as in the forward: lane = query
// column n, 32 band entries (key rows 4g+i of block b) in registers.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int NB>
__global__ __launch_bounds__(NW * kWave) void bwd_q_kernel(const BwdArgs a) {
  constexpr int BQ = 16 * NW;
  constexpr int kHalo = halo_rows<NB>();
  constexpr int kBandWords = band_words<NB>();
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
  const T* __restrict__ dO = static_cast<const T*>(a.dO);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  // Tiles in reverse order: the first workgroups then work on the tiles the
  // forward pass touched last, whose inputs are still in the memory-side
  // cache; the key-side kernel runs forward and so starts where this one ends.
  const int tile = gridDim.x - 1 - xcd_tile(blockIdx.x, gridDim.x);
  const int q0 = tile * BQ;
  const int span0 = q0 - kHalo;
  const int brow = 16 * w;
  const int t = q0 + 16 * w + n;
  const bool tval = t < a.T;
  const int tc = tval ? t : a.T - 1;
  const int H = a.H;
  const int Hp = (H + 1) & ~1;
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = V (dPbar, dG), 1 = K (dC, dS, dQ)
  auto issue = [&](int phase, int h, bool on, auto bc) {
    T* buf = decltype(bc)::value == 0 ? s_x0 : s_x1;
    issue_tile<T, D, R, NW>(buf, phase == 0 ? v : k, span0, a.T, H, h, on);
  };
  // part pp of the DMA of the stage after stage j of `phase`
  auto issue_part = [&](int phase, int j, auto bc, auto pp) {
    constexpr int NIW = tile_insts_per_wave<T, D, R, NW>(), P = decltype(pp)::value;
    const NextStage ns = next_stage(phase, j, H, Hp, 2);
    T* buf = decltype(bc)::value == 0 ? s_x1 : s_x0;
    __builtin_amdgcn_sched_barrier(0);
    issue_tile<T, D, R, NW, P * NIW / kIssueParts, (P + 1) * NIW / kIssueParts>(
        buf, ns.phase == 0 ? v : k, span0, a.T, H, ns.head >= 0 ? ns.head : 0, ns.head >= 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue_rest = [&](int phase, int j, auto bc, auto from) {
    static_for<decltype(from)::value, kIssueParts>([&](auto pp) { issue_part(phase, j, bc, pp); });
  };
  // Prologue: the first tile, the document ids, the saved shared map and the
  // first head's register operands are all in flight before the one wait.
  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  const float sl2 = a.scale * kLog2e;
  const int qb = (q0 >> 4) + w;         // this wave's 16-query block
  const bool wval = q0 + 16 * w < a.T;  // the block holds at least one query
  const size_t bandb = (size_t)(wval ? qb : 0) * kBandWords;  // this wave's band block
  // The shared map saved by the forward pass (masked entries are stored as 0).
  // Each band word is read once here: non-temporal loads (bwd_q -1%).
  uint32_t bandv[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bandv[b][i] = __builtin_nontemporal_load(a.band + bandb + b * 256 + (4 * g + i) * 16 + n);

  // Per-head register operands are loaded one stage ahead (slot j%2 holds head j).
  RowFrag<T, D> fb[2];
  float sb[2];
  float2 stb[2];
  auto preload = [&](const T* src, const float* scal, bool st) {
    load_row_frag<T, D>(fb[0], src + (size_t)tc * H * D, g);
    sb[0] = scal[(size_t)tc * H];
    if (st) stb[0] = a.stats[(size_t)tc * H];
  };
  auto prefetch = [&](int j, auto bc, const T* src, const float* scal, bool st) {
    constexpr int B = decltype(bc)::value;
    const int hn = j + 1 < H ? j + 1 : 0;
    load_row_frag<T, D>(fb[1 - B], src + ((size_t)tc * H + hn) * D, g);
    sb[1 - B] = scal[(size_t)tc * H + hn];
    if (st) stb[1 - B] = a.stats[(size_t)tc * H + hn];
  };
  preload(dO, a.g, false);
  wait_dma();

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
  f32x4 pb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[b][i] = band_decode<T>(bandv[b][i]);

  // ---- phase 0 (V_h staged): B_h = dO_h V_h^T, dPbar, dG ----
  // Small results are stored at the start of the next stage, after its
  // barrier, so the stage wait (vmcnt 0) never waits for fresh stores.
  f32x4 dpb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dpb[b] = zero4();
  float dg_val = 0.f;
  int dg_h = -1;
  auto flush_dg = [&]() {
    if (dg_h >= 0 && tval && g == 0) a.dg[(size_t)t * H + dg_h] = dg_val;
    dg_h = -1;
  };
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    // the last stage of this phase prefetches the first head of the next one
    const bool last = j + 1 >= H;
    flush_dg();
    issue_part(0, j, bc, Part<0>{});
    __builtin_amdgcn_s_setprio(2);
    if (!real) {
      prefetch(j, bc, last ? q : dO, last ? a.c : a.g, last);
      issue_rest(0, j, bc, Part<1>{});
      return;
    }
    const RowFrag<T, D>& df = fb[B];
    const float gh = sb[B];
    float dgs = 0.f;
    f32x4 bt[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      bt[b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, df);
      if (b == 1) issue_part(0, j, bc, Part<1>{});
      if (b == 3) issue_part(0, j, bc, Part<2>{});
      if (b == 5) issue_part(0, j, bc, Part<3>{});
    }
    // next stage's register operands, issued after this stage's DMA and
    // contraction (right after the barrier every wave's issue would contend)
    prefetch(j, bc, last ? q : dO, last ? a.c : a.g, last);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // masked entries of pb are exactly 0; bt there is finite (zero-filled rows)
        dgs += pb[b][i] * bt[b][i];
        dpb[b][i] += gh * bt[b][i];
      }
    __builtin_amdgcn_s_setprio(0);
    dg_val = wave_sum4(dgs);
    dg_h = j;
  });
  flush_dg();
  if (wval) {
    // dPbar of this wave's block, for the key-centric kernel
    uint32_t* blk = reinterpret_cast<uint32_t*>(a.dband) + bandb;
    if constexpr (Elem<T>::bf16) {
      uint32_t wv[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[b][i] = __float_as_uint(dpb[b][i]);
      store_band_block(blk, wv, s_xp + w * 512, g, n);
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) blk[b * 256 + (4 * g + i) * 16 + n] = __float_as_uint(dpb[b][i]);
    }
  }

  // ---- phase 1 (K_h staged): P_h, dC, dS, dQ ----
  f32x4 pend[D / 16];
  float dc_val = 0.f;
  int pend_h = -1;
  // The previous head's dQ row is stored during this stage's token
  // contraction (see mma_tcontract), late in the stage: stores issued early
  // would queue ahead of the other waves' DMA of the next tile.
  auto pending = [&]() {
    return pending_rows<D>(a.dq, q0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0,
                           a.scale, s_xp + (Elem<T>::bf16 ? w * 512 : 0));
  };
  auto flush_dc = [&]() {
    if (pend_h >= 0 && tval && g == 0) a.dc[(size_t)t * H + pend_h] = dc_val;
  };
  auto flush_dq = [&]() {
    flush_dc();
    store_row<T, D>(pending(), pend, g, n);
    pend_h = -1;
  };
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    wait_dma();
    const bool real = j < H;
    flush_dc();
    issue_part(1, j, bc, Part<0>{});
    __builtin_amdgcn_s_setprio(2);
    if (!real) {
      issue_rest(1, j, bc, Part<1>{});
      flush_dq();
      return;
    }
    const PendingRow prev = pending();
    const RowFrag<T, D>& qf = fb[B];
    const float ch = sb[B];
    const float2 st = stb[B];  // (row max in log2 units, 1/row sum) saved by the forward pass
    // e = exp2(s*scale*log2e - max) = P_h / inv; masked entries 0
    f32x4 p[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      p[b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, qf);
      if (b == 1) issue_part(1, j, bc, Part<1>{});
      if (b == 3) issue_part(1, j, bc, Part<2>{});
      if (b == 5) issue_part(1, j, bc, Part<3>{});
    }
    prefetch(j, bc, q, a.c, true);  // next stage's operands (see the V phase)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[b][i] = exp2_scaled(p[b][i], sl2, st.x);  // as in the forward pass
    mask_band(p, mbits, full, 0.f);
    float dcs = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) dcs = fmaf(p[b][i], dpb[b][i], dcs);
    dcs = wave_sum4(dcs) * st.y;  // dC = sum_s P_h dPbar
    dc_val = dcs;
    const float cs = ch * st.y;   // dS = C P (dPbar - dC) = (C inv) e (dPbar - dC)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[b][i] = cs * p[b][i] * (dpb[b][i] - dcs);
    BandOperand<T, NB> dso;
    dso.set(p);
    __builtin_amdgcn_s_setprio(0);
    mma_tcontract<T, D, NB>(pend, cur, brow, lo, dso, g, n, prev);
    pend_h = j;
  });
  flush_dq();
  wait_dma();
}

// ---------------------------------------------------------------------------
// bwd_kv: per key.  Normal orientation S = Q K^T: lane = key column n, rows
// 4g+i of query block b in registers; the wave's queries are the 16*NB tokens
// [kw, kw+16*NB) that can hold its keys in their windows.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int NB>
__global__ __launch_bounds__(NW * kWave) void bwd_kv_kernel(const BwdArgs a) {
  constexpr int BK = 16 * NW;
  constexpr int kHalo = halo_rows<NB>();
  constexpr int kBandWords = band_words<NB>();
  // query rows [k0, k0 + BK + kHalo), rounded up to whole DMA instructions
  constexpr int R = (BK + kHalo + Tile<T, D>::rows_per_inst - 1) / Tile<T, D>::rows_per_inst *
                    Tile<T, D>::rows_per_inst;
  constexpr int RP = (R + 63) / 64 * 64;
  // per-row scalars of the staged head: C, G, dC, row max, 1/row sum
  enum { SC_C = 0, SC_G = 1, SC_DC = 2, SC_MX = 3, SC_INV = 4, NSC = 5 };
  __shared__ __attribute__((aligned(1024))) T s_x0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_x1[R * D];
  __shared__ __attribute__((aligned(16))) float s_sc0[NSC * RP];
  __shared__ __attribute__((aligned(16))) float s_sc1[NSC * RP];
  __shared__ __attribute__((aligned(16))) int s_doc[(R + 63) / 64 * 64];
  __shared__ __attribute__((aligned(16))) float s_xp[Elem<T>::bf16 ? NW * 512 : 4];  // row stores

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ dO = static_cast<const T*>(a.dO);
  const float* __restrict__ stats = reinterpret_cast<const float*>(a.stats);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int k0 = tile * BK;
  const int span0 = k0;
  const int brow = 16 * w;        // LDS row of this wave's first query (token kw)
  const int s = k0 + 16 * w + n;  // this lane's key
  const bool sval = s < a.T;
  const int sc_ = sval ? s : a.T - 1;
  const int H = a.H;
  const int Hp = (H + 1) & ~1;
  const LaneOffsets<T, D> lo(g, n);

  // phases: 0 = dO (dV), 1 = Q (dS, dK)
  auto issue = [&](int phase, int h, bool on, auto bc) {
    constexpr int B = decltype(bc)::value;
    T* buf = B == 0 ? s_x0 : s_x1;
    float* sc = B == 0 ? s_sc0 : s_sc1;
    issue_tile<T, D, R, NW>(buf, phase == 0 ? dO : q, span0, a.T, H, h, on);
    issue_scalars<R, NW>(sc + SC_C * RP, a.c, 1, 0, span0, a.T, H, h, on);
    issue_scalars<R, NW>(sc + SC_G * RP, a.g, 1, 0, span0, a.T, H, h, on);
    issue_scalars<R, NW>(sc + SC_DC * RP, a.dc, 1, 0, span0, a.T, H, h, on);
    issue_scalars<R, NW>(sc + SC_MX * RP, stats, 2, 0, span0, a.T, H, h, on);
    issue_scalars<R, NW>(sc + SC_INV * RP, stats, 2, 1, span0, a.T, H, h, on);
  };
  // part pp of the DMA of the stage after stage j of `phase` (part 0 also
  // issues the per-row scalars)
  auto issue_part = [&](int phase, int j, auto bc, auto pp) {
    constexpr int NIW = tile_insts_per_wave<T, D, R, NW>(), P = decltype(pp)::value;
    const NextStage ns = next_stage(phase, j, H, Hp, 2);
    const int h = ns.head >= 0 ? ns.head : 0;
    const bool on = ns.head >= 0;
    T* buf = decltype(bc)::value == 0 ? s_x1 : s_x0;
    float* sc = decltype(bc)::value == 0 ? s_sc1 : s_sc0;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (P == 0) {
      issue_scalars<R, NW>(sc + SC_C * RP, a.c, 1, 0, span0, a.T, H, h, on);
      issue_scalars<R, NW>(sc + SC_G * RP, a.g, 1, 0, span0, a.T, H, h, on);
      issue_scalars<R, NW>(sc + SC_DC * RP, a.dc, 1, 0, span0, a.T, H, h, on);
      issue_scalars<R, NW>(sc + SC_MX * RP, stats, 2, 0, span0, a.T, H, h, on);
      issue_scalars<R, NW>(sc + SC_INV * RP, stats, 2, 1, span0, a.T, H, h, on);
    }
    issue_tile<T, D, R, NW, P * NIW / kIssueParts, (P + 1) * NIW / kIssueParts>(
        buf, ns.phase == 0 ? dO : q, span0, a.T, H, h, on);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue_rest = [&](int phase, int j, auto bc, auto from) {
    static_for<decltype(from)::value, kIssueParts>([&](auto pp) { issue_part(phase, j, bc, pp); });
  };
  // Prologue: the first tile, the document ids and the saved shared map are
  // all in flight before the one wait.
  issue(0, 0, true, Buf<0>{});
  issue_doc<R, NW>(s_doc, a.doc, span0, a.T);
  // Pbar (phase 0) and dPbar (phase 1) of this lane's (key, 4 queries)
  // entries, from the bands: query block kq + b, key block NB-1-b, 16 bytes
  // per block; entries beyond the stream or outside the window read as 0.
  // Loaded non-temporally, like every band read (bwd_kv -3%).
  const int kq = (k0 >> 4) + w;
  const int nqb = (a.T + 15) >> 4;
  auto band_word = [&](int b) {
    const int qbk = kq + b < nqb ? kq + b : nqb - 1;
    return (size_t)qbk * kBandWords + (NB - 1 - b) * 256 + n * 16 + 4 * g;
  };
  uint4 bandv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    bandv[b] = __builtin_bit_cast(
        uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.band + band_word(b))));
  wait_dma();

  MaskT<NB> mbits = 0;  // bit 4b+i <-> query row brow + 16b + 4g + i
  {
    const int ds = s_doc[brow + n];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = brow + 16 * b + 4 * g + i;
        const int t = span0 + r;
        const bool ok = sval & (t < a.T) & (t >= s) & (t - s < a.window) & (s_doc[r] == ds);
        mbits |= (MaskT<NB>)(ok ? 1u : 0u) << (4 * b + i);
      }
  }
  const uint32_t full = full_blocks<NB>(mbits);  // wave-uniform
  f32x4 pb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t uu[4] = {bandv[b].x, bandv[b].y, bandv[b].z, bandv[b].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[b][i] = keep_admitted(mbits, b, i, band_decode<T>(uu[i]), 0.f);
  }

  auto rows4 = [&](const float* sc, int field, int b) {
    return *reinterpret_cast<const float4*>(sc + field * RP + brow + 16 * b + 4 * g);
  };
  const float sl2 = a.scale * kLog2e;

  // A stage's output row is stored during the next stage, after that stage's
  // DMA has been issued, spread over its contractions (see mma_tcontract).
  f32x4 pend[D / 16];
  int pend_h = -1;
  auto pending = [&](float* dst, float scale) {
    return pending_rows<D>(dst, k0 + 16 * w, n, a.T, H, pend_h >= 0 ? pend_h : 0, pend_h >= 0, scale,
                           s_xp + (Elem<T>::bf16 ? w * 512 : 0));
  };
  auto flush = [&](float* dst, float scale) {
    store_row<T, D>(pending(dst, scale), pend, g, n);
    pend_h = -1;
  };

  // Q phase operands loaded during the last dO stage: dPbar of this lane's
  // (key, 4 queries) entries and the first head's K fragment.
  f32x4 dpb[NB];
  RowFrag<T, D> kfb[2];
  auto load_q_phase = [&]() {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4 d4 =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.dband + band_word(b)));
      dpb[b] = d4;  // only multiplied by P_h, which is 0 where masked
    }
    load_row_frag<T, D>(kfb[0], k + (size_t)sc_ * H * D, g);
  };

  // ---- phase 0 (dO_h staged): dV_h = (G_h o Pbar)^T dO_h ----
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    const float* sc = B == 0 ? s_sc0 : s_sc1;
    wait_dma();
    const bool real = j < H;
    issue_part(0, j, bc, Part<0>{});
    if (j + 1 >= H) load_q_phase();
    __builtin_amdgcn_s_setprio(2);
    if (!real) {
      issue_rest(0, j, bc, Part<1>{});
      flush(a.dv, 1.f);
      return;
    }
    f32x4 gp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4 g4 = rows4(sc, SC_G, b);
      gp[b] = f32x4{g4.x * pb[b][0], g4.y * pb[b][1], g4.z * pb[b][2], g4.w * pb[b][3]};
    }
    BandOperand<T, NB> op;
    op.set(gp);
    __builtin_amdgcn_s_setprio(1);
    mma_tcontract<T, D, NB>(pend, cur, brow, lo, op, g, n, pending(a.dv, 1.f), [&](auto pp) {
      if constexpr (decltype(pp)::value < kIssueParts) issue_part(0, j, bc, pp);
    });
    issue_rest(0, j, bc, Part<tcontract_groups<T, D>()>{});
    __builtin_amdgcn_s_setprio(0);
    pend_h = j;
  });

  // ---- phase 1 (Q_h staged): P_h, dS_h, dK_h = scale dS_h^T Q_h ----
  bool first = true;
  for_stage_pairs(Hp, [&](int j, auto bc) {
    constexpr int B = decltype(bc)::value;
    const T* cur = B == 0 ? s_x0 : s_x1;
    const float* sc = B == 0 ? s_sc0 : s_sc1;
    wait_dma();
    const bool real = j < H;
    // the first stage of this phase stores the last dV row (during its token
    // contraction, late in the stage: see the query-side kernel)
    const PendingRow prev = pending(first ? a.dv : a.dk, first ? 1.f : a.scale);
    first = false;
    issue_part(1, j, bc, Part<0>{});
    __builtin_amdgcn_s_setprio(2);
    if (!real) {
      issue_rest(1, j, bc, Part<1>{});
      store_row<T, D>(prev, pend, g, n);
      pend_h = -1;
      return;
    }
    const RowFrag<T, D>& kf = kfb[B];
    f32x4 p[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      p[b] = mma_dcontract<T, D>(zero4(), cur, brow + 16 * b, lo, kf);
      if (b == 1) issue_part(1, j, bc, Part<1>{});
      if (b == 3) issue_part(1, j, bc, Part<2>{});
      if (b == 5) issue_part(1, j, bc, Part<3>{});
    }
    // next head's K row, issued after this stage's DMA and score contraction
    load_row_frag<T, D>(kfb[1 - B], k + ((size_t)sc_ * H + (j + 1 < H ? j + 1 : 0)) * D, g);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4 mx = rows4(sc, SC_MX, b), inv = rows4(sc, SC_INV, b);
      const float4 c4 = rows4(sc, SC_C, b), dc4 = rows4(sc, SC_DC, b);
      const float mxv[4] = {mx.x, mx.y, mx.z, mx.w}, invv[4] = {inv.x, inv.y, inv.z, inv.w};
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, dcv[4] = {dc4.x, dc4.y, dc4.z, dc4.w};
      // dS_h = C P_h (dPbar - dC) with P_h = exp2(s*scale*log2e - max) / sum
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[b][i] = (cv[i] * invv[i]) * exp2_scaled(p[b][i], sl2, mxv[i]) * (dpb[b][i] - dcv[i]);
    }
    mask_band(p, mbits, full, 0.f);
    BandOperand<T, NB> dso;
    dso.set(p);
    __builtin_amdgcn_s_setprio(0);
    mma_tcontract<T, D, NB>(pend, cur, brow, lo, dso, g, n, prev);
    pend_h = j;
  });
  flush(a.dk, a.scale);
  wait_dma();
}

template <typename T, int D, int NW, int NB>
static hipError_t launch_bwd(const BwdArgs& a, int parts, hipStream_t st) {
  constexpr int B = 16 * NW;
  const int nblk = (int)((a.T + B - 1) / B);
  if (parts & 1) {
    hipLaunchKernelGGL((bwd_q_kernel<T, D, NW, NB>), dim3(nblk), dim3(NW * kWave), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (parts & 2) {
    hipLaunchKernelGGL((bwd_kv_kernel<T, D, NW, NB>), dim3(nblk), dim3(NW * kWave), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Windows up to 113 keys: 8-block bands; wider (up to 128): 10-block bands in
// 4-wave workgroups (one wave per SIMD, up to 512 registers).
hipError_t bwd_dispatch(int dtype, int d, const BwdArgs& a, int parts, hipStream_t st) {
  const bool wide = a.window > kMaxWindow;
  if (dtype == 0) {
    if (d == 128) return wide ? launch_bwd<bf16_t, 128, 4, 10>(a, parts, st) : launch_bwd<bf16_t, 128, 8, 8>(a, parts, st);
    if (d == 64) return wide ? launch_bwd<bf16_t, 64, 4, 10>(a, parts, st) : launch_bwd<bf16_t, 64, 8, 8>(a, parts, st);
    if (d == 16) return wide ? launch_bwd<bf16_t, 16, 4, 10>(a, parts, st) : launch_bwd<bf16_t, 16, 8, 8>(a, parts, st);
  } else {
    if (d == 128 && !wide) return launch_bwd<float, 128, 2, 8>(a, parts, st);
    if (d == 64) return wide ? launch_bwd<float, 64, 4, 10>(a, parts, st) : launch_bwd<float, 64, 4, 8>(a, parts, st);
    if (d == 16) return wide ? launch_bwd<float, 16, 4, 10>(a, parts, st) : launch_bwd<float, 16, 4, 8>(a, parts, st);
  }
  return hipErrorInvalidValue;
}

// Workspace of the allocation-free backward entry point: one array per GPU,
// held by the loaded code object until the process ends.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(int device, void** ptr) {
  // The host-side name of `scratch` is not a device address: the device
  // address is asked for once per device, with that device current.
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

}  // namespace ldc
