// The attention block's main attention with the Lightweight DC layer fused
// in, forward, for gfx950.
//
// Layer (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
// section "第二刀-砍层内", Lightweight DC paragraph: the branch reuses the
// block's Q and K over a short local window, with a dedicated kernel), read as
//   O[t,h] = M[t,h] + G[t,h] sum_{s in A(t)} Pbar[t,s] V[s,h]
// M: causal softmax attention of head h over the query's own run of equal
// document ids (keys run_start(t) .. t); the second term: the Lightweight DC
// layer (its window and document cut, Pbar = sum_h C[t,h] P_h).
//
// Launches (one stream, in order):
//  1. run_marks / run_starts: run_start(t) of every token (a two-level
//     prefix maximum of the run boundaries over 1024-token blocks).
//  2. (fused only) the Lightweight DC score pass: the composed map Pbar of
//     every 16-query block over its 128-key band, in the layout of the
//     layer's saved state (it is that state, usable by the backward pass).
//  3. attn_fwd_kernel: one workgroup of 8 waves per (128-query tile, head),
//     flash-style: 128-key stages of K then V stream through a four-slot LDS
//     ring by DMA (three half-stages in flight), scores on MFMA, online
//     softmax in registers, P V on MFMA into an fp32 accumulator per wave
//     (16 queries x d).  Stages run from the tile's earliest run start to the
//     tile's last query; the last two (the keys q0-128 .. q0+127) hold every
//     key of the tile's Lightweight DC bands, so after the last stage the
//     band's value contraction l G Pbar V joins the accumulator (l the final
//     softmax sum) and O = acc / l is written once.
// Work items are (tile, head) pairs, so a long document's tiles spread over
// the whole chip; every launch is deterministic.
#include "fused_internal.h"
#include "ldc_device.hpp"

namespace ldc {

// ---------------------------------------------------------------------------
// Run starts
// ---------------------------------------------------------------------------
constexpr int kRunBlock = 1024;  // tokens per run-start block (256 threads x 4)
constexpr int kTileQ = 128;      // queries per main-attention tile
constexpr int kStageK = 64;      // keys per main-attention stage
constexpr int kOrderBins = 1024;  // stage-count classes of the item order

// Stages of a tile before its four window stages: chunks of kStageK keys from
// its earliest run start up to q0 - 2 kStageK.
__device__ __forceinline__ int tile_chunks(int q0, int rs0) {
  const int span = (q0 - 2 * kStageK) - rs0;
  return span > 0 ? (span + kStageK - 1) / kStageK : 0;
}
// Order class of a tile: most chunks first (the last class holds every tile
// with kOrderBins - 1 or more).
__device__ __forceinline__ int order_bin(int q0, int rs0) {
  const int c = tile_chunks(q0, rs0);
  return kOrderBins - 1 - (c < kOrderBins - 1 ? c : kOrderBins - 1);
}

__device__ __forceinline__ int block_max_256(int x, int* red) {
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  const int r = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  return r;
}

// is t the first token of its run (t == 0 or its id differs from t-1's)?
__device__ __forceinline__ bool run_boundary(const int32_t* __restrict__ doc, int t) {
  return t == 0 || doc[t] != doc[t - 1];
}

// last[b]: the last run boundary in tokens [1024 b, 1024 b + 1024), or -1.
__global__ __launch_bounds__(256) void run_marks_kernel(const int32_t* __restrict__ doc, int T,
                                                        int* __restrict__ last, int* __restrict__ order) {
  __shared__ int red[4];
  if (blockIdx.x == 0)  // the order histogram and cursors start at zero
    for (int i = threadIdx.x; i < 2 * kOrderBins; i += 256) order[i] = 0;
  const int t0 = blockIdx.x * kRunBlock + 4 * threadIdx.x;
  int best = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < T && run_boundary(doc, t0 + j)) best = t0 + j;
  best = block_max_256(best, red);
  if (threadIdx.x == 0) last[blockIdx.x] = best;
}

// rs[t] = run_start(t): the larger of the last boundary before the block
// (from the block summaries, looked back 256 blocks at a time; block 0 always
// holds token 0's boundary) and the block's own prefix maximum up to t.
__global__ __launch_bounds__(256) void run_starts_kernel(const int32_t* __restrict__ doc, int T,
                                                         const int* __restrict__ last,
                                                         int* __restrict__ rs, int* __restrict__ order) {
  __shared__ int red[4];
  __shared__ int wtot[4];
  const int b = blockIdx.x;
  int carry = -1;
  for (int base = b - 1; base >= 0 && carry < 0; base -= 256) {  // workgroup-uniform
    const int j = base - (int)threadIdx.x;
    carry = block_max_256(j >= 0 ? last[j] : -1, red);
  }
  const int t0 = b * kRunBlock + 4 * threadIdx.x;
  int r[4];
  int run = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j < T && run_boundary(doc, t0 + j)) run = t0 + j;
    r[j] = run;
  }
  // exclusive prefix maximum of the threads' last values
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = run;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x = max(x, y);
  }
  if (lane == 63) wtot[w] = x;
  int before = __shfl_up(x, 1);
  if (lane == 0) before = -1;
  __syncthreads();
  for (int i = 0; i < w; ++i) before = max(before, wtot[i]);
  before = max(before, carry);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < T) {
      const int rsv = max(before, r[j]);
      rs[t0 + j] = rsv;
      // a tile's first query: count the tile in its order class
      if (((t0 + j) & (kTileQ - 1)) == 0) atomicAdd(&order[order_bin(t0 + j, rsv)], 1);
    }
}

// The tiles' order: tile list position = the classes before the tile's own
// (an exclusive scan of the histogram, redone by every workgroup) + a slot
// claimed in its class.  Tiles of one class land in any order (the order
// only schedules work; every tile computes the same result wherever it
// runs).
__global__ __launch_bounds__(256) void tile_order_kernel(const int* __restrict__ rs, int T,
                                                         int* __restrict__ order) {
  __shared__ int base[kOrderBins];
  __shared__ int wtot[4];
  const int* hist = order;
  int* cursor = order + kOrderBins;
  int* list = order + 2 * kOrderBins;
  int cnt[4];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cnt[i] = hist[4 * threadIdx.x + i];
    tot += cnt[i];
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = tot;  // inclusive scan over the wave
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  int excl = x - tot;
  for (int i = 0; i < w; ++i) excl += wtot[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    base[4 * threadIdx.x + i] = excl;
    excl += cnt[i];
  }
  __syncthreads();
  const int tile = blockIdx.x * 256 + threadIdx.x;
  const int ntile = (T + kTileQ - 1) / kTileQ;
  if (tile < ntile) {
    const int b = order_bin(tile * kTileQ, rs[tile * kTileQ]);
    list[base[b] + atomicAdd(&cursor[b], 1)] = tile;
  }
}

// ---------------------------------------------------------------------------
// Main attention
// ---------------------------------------------------------------------------
constexpr int kANW = 8;                // waves per workgroup
constexpr int kABQ = 16 * kANW;        // 128 queries per tile
constexpr int kARows = kStageK;        // keys per stage
static_assert(kABQ == kTileQ, "the item order counts the kernel's tiles");
constexpr int kABlocks = kARows / 16;  // 4 key blocks per stage

template <int I>
using IC = std::integral_constant<int, I>;

// The 32-bit LDS address of a pointer into a __shared__ array.
template <typename T>
__device__ __forceinline__ uint32_t lds_offset(const T* p) {
  typedef const __attribute__((address_space(3))) char* lds_cptr;
  return (uint32_t)(uintptr_t)(lds_cptr)(const void*)p;
}

// s[b] = (16 keys of block b of a staged tile) x (this lane's query row),
// contracted over the head dimension: the transposed score block, lane (g, n)
// holding keys 4g..4g+3 of query n.  Each block's K fragments are read just
// before its MFMAs.
template <typename T, int D, int NB>
__device__ __forceinline__ void score_band(f32x4 (&s)[NB], const T* tile, const LaneOffsets<T, D>& lo,
                                           const RowFrag<T, D>& f) {
  using TL = Tile<T, D>;
  constexpr int KK = D / 32;
  const char* base = reinterpret_cast<const char*>(tile);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    bf16x8 u[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      u[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(base + 16 * b * TL::row_bytes + lo.dk[kk]));
    f32x4 c = zero4();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) c = mma(u[kk], f.v[kk], c);
    s[b] = c;
  }
}

// acc += X^T P over NB 16-row blocks of staged tiles, block b starting at
// LDS byte address blk[b] (X the rows, P a band operand in accumulator
// layout; HILO: P carried as hi + lo bf16 parts, else hi only), one column
// group of the output at a time: its transposed reads, then its MFMAs.
template <typename T, int D, int NB, bool HILO>
__device__ __forceinline__ void pv_stream(f32x4 (&acc)[D / 16], const char* const (&blk)[NB],
                                          const LaneOffsets<T, D>& lo, const BandOperand<T, NB>& P) {
  typedef __attribute__((address_space(3))) bf16x4 lds_v4;
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    bf16x8 a[NB / 2][2];
#pragma unroll
    for (int ks = 0; ks < NB / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int off = lo.tr[p] ^ (8 * e);
        const bf16x4 l4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(blk[2 * ks] + off));
        const bf16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(blk[2 * ks + 1] + off));
        a[ks][e] = __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    f32x4 c0 = acc[2 * p], c1 = acc[2 * p + 1];
#pragma unroll
    for (int ks = 0; ks < NB / 2; ++ks) {
      c0 = mma(a[ks][0], P.hi[ks], c0);
      c1 = mma(a[ks][1], P.hi[ks], c1);
      if constexpr (HILO) {
        c0 = mma(a[ks][0], P.lo[ks], c0);
        c1 = mma(a[ks][1], P.lo[ks], c1);
      }
    }
    acc[2 * p] = c0;
    acc[2 * p + 1] = c1;
  }
}

// One workgroup per (128-query tile, head).  Two workgroups share a CU: the
// ring (four 64-key slots) is 64 KB at d = 128 and the kernel keeps to 128
// VGPRs, so each SIMD holds four waves.  NBB: key blocks of the Lightweight
// DC band (8 for windows up to 113 keys, 10 up to 128).
template <typename T, int D, bool LDC, int NBB = kKeyBlocks>
__global__ __launch_bounds__(kANW * kWave, 4) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NW = kANW, BQ = kABQ, R = kARows, NB = kABlocks;
  constexpr int NIW = tile_insts_per_wave<T, D, R, NW>();  // DMA instructions per wave per half-stage
  using TL = Tile<T, D>;
  // the ring: slot i holds half-stage j with j % 4 == i (K of stage s is
  // half-stage 2s, V of stage s is 2s + 1).  Four separate arrays, always
  // chosen at compile time, so that the compiler sees which LDS object a
  // pending DMA writes and does not wait for it before reading another.
  __shared__ __attribute__((aligned(1024))) T s_r0[R * D];
  __shared__ __attribute__((aligned(1024))) T s_r1[R * D];
  __shared__ __attribute__((aligned(1024))) T s_r2[R * D];
  __shared__ __attribute__((aligned(1024))) T s_r3[R * D];
  // row-store scratch (2 KB per wave): slot 0 once the ring is done where a
  // slot holds it (d = 128), else an array of its own
  constexpr bool kXpInRing = R * D * (int)sizeof(T) >= NW * 512 * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) float s_xp[kXpInRing ? 4 : NW * 512];
  // a 10-block band reaches 16 rows below the window stages: those V rows
  constexpr int kExRows = NBB > kKeyBlocks ? 16 * (NBB - kKeyBlocks) / 2 : 1;
  __shared__ __attribute__((aligned(1024))) T s_ex[kExRows * D];

  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ k = static_cast<const T*>(a.k);
  const T* __restrict__ v = static_cast<const T*>(a.v);
  const int H = a.H;
  // work items (tile, head), tiles with the most stages first
  const int item = blockIdx.x;
  const int slot_i = item / H, h = item - slot_i * H;
  const int ntile = (a.T + BQ - 1) / BQ;
  int tile = __builtin_amdgcn_readfirstlane(a.order[slot_i]);
  tile = tile < 0 ? 0 : tile < ntile ? tile : ntile - 1;  // the list is a permutation; kept in range regardless
  const int q0 = tile * BQ;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int t = q0 + 16 * w + n;
  const int tc = t < a.T ? t : a.T - 1;
  const int tw = q0 + 16 * w;  // the wave's first query
  const float sl2 = a.scale * kLog2e;
  const LaneOffsets<T, D> lo(g, n);

  // operands of the whole item (older than every DMA below)
  RowFrag<T, D> qf;
  load_row_frag<T, D, true>(qf, q + ((size_t)tc * H + h) * D, g);
  const int kslo = a.rs[tc];
  const int ks0 = __builtin_amdgcn_readfirstlane(a.rs[q0]);  // earliest key of the tile
  float gh = 0.f;
  if constexpr (LDC) gh = a.g[(size_t)tc * H + h];

  // stages: chunks of R keys from (at or before) ks0 up to q0-129, then the
  // four window stages [q0-128, q0+128)
  const int w1 = q0 - 2 * R;
  const int nc = tile_chunks(q0, ks0);
  const int NS = nc + 4;
  auto stage_row = [&](int s) __attribute__((always_inline)) { return w1 - R * (nc - s); };
  auto slot = [&](auto c) __attribute__((always_inline)) -> T* {
    constexpr int I = decltype(c)::value & 3;
    return I == 0 ? s_r0 : I == 1 ? s_r1 : I == 2 ? s_r2 : s_r3;
  };
  // DMA of R rows of `src` from row0 into a slot.  The lane offsets of an
  // in-range tile are fixed for the item; only the buffer resource and, for
  // a tile with rows outside [lim0, lim1) (those read as zero), the offsets
  // change.  The DMA instructions are the same straight-line sequence either
  // way, so the number in flight is always NIW per call.
  constexpr int RPI = TL::rows_per_inst, NI = R / RPI;
  const uint32_t rstride = (uint32_t)H * D * sizeof(T);
  uint32_t voff[NIW];
#pragma unroll
  for (int u = 0; u < NIW; ++u) {
    const int jj = (w + u * NW < NI) ? w + u * NW : NI - 1;
    const int rl = jj * RPI + lane / TL::chunks;
    voff[u] = (uint32_t)rl * rstride + (uint32_t)TL::pos(rl, lane % TL::chunks) * 16u;
  }
  auto issue_rows = [&](auto c, const T* src, int row0, int lim1) __attribute__((always_inline)) {
    i32x4 rsrc;
    uint32_t vo[NIW];
    if (row0 >= 0 && row0 + R <= lim1) {  // workgroup-uniform
      rsrc = make_rsrc(src + ((size_t)row0 * H + h) * D, (uint32_t)(R - 1) * rstride + D * sizeof(T));
#pragma unroll
      for (int u = 0; u < NIW; ++u) vo[u] = voff[u];
    } else {
      const int lo_r = row0 > 0 ? row0 : 0;
      const int hi_r = row0 + R < lim1 ? row0 + R : lim1;
      const uint32_t bytes = hi_r > lo_r ? (uint32_t)(hi_r - 1 - lo_r) * rstride + D * sizeof(T) : 0u;
      rsrc = make_rsrc(src + ((size_t)(hi_r > lo_r ? lo_r : 0) * H + h) * D, bytes);
#pragma unroll
      for (int u = 0; u < NIW; ++u) {
        const int jj = (w + u * NW < NI) ? w + u * NW : NI - 1;
        const int sr = row0 + jj * RPI + lane / TL::chunks;
        // out of range: an offset at the end of the (possibly empty) buffer reads zero
        vo[u] = (sr >= lo_r && sr < hi_r) ? voff[u] - (uint32_t)(lo_r - row0) * rstride : bytes;
      }
    }
    char* base = reinterpret_cast<char*>(slot(c));
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
      const int jj = (w + u * NW < NI) ? w + u * NW : NI - 1;
      ldc_buffer_load_lds(rsrc, (lds_u32_ptr)(base + jj * 1024), 16, (int)vo[u], 0, 0, 0);
    }
  };
  // half-stage j of the loop; past the last stage it reads nothing (zeros)
  const int lim_loop = q0 + BQ < a.T ? q0 + BQ : a.T;
  auto issue_half = [&](auto c, int j) __attribute__((always_inline)) {
    const T* src = (decltype(c)::value & 1) ? v : k;
    issue_rows(c, src, stage_row(j >> 1), j < 2 * NS ? lim_loop : -(1 << 30));
  };
  // a stage needs masking when it holds keys below the wave's latest run
  // start (run starts never decrease, so that of its last query) or past
  // the wave's first query
  const int kmax = __builtin_amdgcn_readfirstlane(a.rs[tw + 15 < a.T ? tw + 15 : a.T - 1]);
  issue_half(IC<0>{}, 0);
  issue_half(IC<1>{}, 1);
  issue_half(IC<2>{}, 2);
  // the item's operand loads (older) are complete, the DMA still in flight;
  // said here, the compiler need not drain the DMA before the stage loop
  __builtin_amdgcn_s_waitcnt(((3 * NIW) & 15) | (((3 * NIW) >> 4) << 14) | (7 << 4) | (15 << 8));

  f32x4 acc[D / 16];
#pragma unroll
  for (int r = 0; r < D / 16; ++r) acc[r] = zero4();
  float m = -1e30f, l = 0.f;  // running max (log2 units; finite start) and sum
  BandOperand<T, NB> pop;     // the current stage's P (its hi part is used)

  // scores of a K stage and the online-softmax update; leaves P in pop
  auto k_stage = [&](const T* kt, int row0) __attribute__((always_inline)) {
    f32x4 s[NB];
    __builtin_amdgcn_s_setprio(1);
    score_band<T, D, NB>(s, kt, lo, qf);
    __builtin_amdgcn_s_setprio(0);
    if (row0 < kmax || row0 + R - 1 > tw) {  // wave-uniform
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = row0 + 16 * b + 4 * g + i;
          s[b][i] = (key >= kslo && key <= t) ? s[b][i] : -INFINITY;
        }
    }
    // the scale is positive: the max of the raw scores gives the max of the
    // scaled ones, and the scaling joins the exponent's FMA
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b) mx = fmaxf(mx, fmaxf(fmaxf(s[b][0], s[b][1]), fmaxf(s[b][2], s[b][3])));
    mx = wave_max4(mx);
    const float mn = fmaxf(m, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // wave-uniform
#pragma unroll
      for (int r = 0; r < D / 16; ++r) acc[r] *= alpha;
    }
    float sum = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[b][i] = __builtin_amdgcn_exp2f(fmaf(s[b][i], sl2, -mn));
        sum += s[b][i];
      }
    l = l * alpha + wave_sum4(sum);
    m = mn;
    pop.set(s);
  };
  auto v_stage = [&](const T* vt) __attribute__((always_inline)) {
    const char* blk[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) blk[b] = reinterpret_cast<const char*>(vt) + 16 * b * TL::row_bytes;
    __builtin_amdgcn_s_setprio(1);
    pv_stream<T, D, NB, false>(acc, blk, lo, pop);
    __builtin_amdgcn_s_setprio(0);
  };

  // Stage s with its K in slot P = 2s % 4; three half-stages in flight, so
  // each wait leaves the two younger ones pending.  Every call issues the
  // same DMA instructions (past the last stage they read nothing), so the
  // counts hold to the end.
  auto chunk = [&](auto pc, int s) __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    wait_dma_except<2 * NIW>();
    issue_half(IC<P + 3>{}, 2 * s + 3);
    k_stage(slot(IC<P>{}), stage_row(s));
    wait_dma_except<2 * NIW>();
    issue_half(IC<P + 4>{}, 2 * s + 4);
    v_stage(slot(IC<P + 1>{}));
  };
  int s = 0;
  for (; s + 2 <= NS; s += 2) {  // workgroup-uniform
    chunk(IC<0>{}, s);
    chunk(IC<2>{}, s + 1);
  }
  if (NS & 1) chunk(IC<0>{}, s);
  wait_dma_except<0>();  // the two empty half-stages; every wave is past the loop

  if constexpr (LDC) {
    // l G Pbar V over the wave's band: the window's V rows [q0-128, q0+128)
    // are staged again, 64 to a slot (the L2 still holds them), and for a
    // 10-block band the 16 rows below them into s_ex; band block b of wave w
    // holds keys q0 + 16w - 16 (NBB - 1) + 16b, row r = 16w + 16b + 16 (9 -
    // NBB) of the window (r = -16: s_ex)
    static_assert(NBB == kKeyBlocks || NBB == kKeyBlocks + 2, "8- or 10-block bands");
    const int lim_v = q0 + BQ < a.T ? q0 + BQ : a.T;
    issue_rows(IC<0>{}, v, w1, lim_v);
    issue_rows(IC<1>{}, v, w1 + R, lim_v);
    issue_rows(IC<2>{}, v, w1 + 2 * R, lim_v);
    issue_rows(IC<3>{}, v, w1 + 3 * R, lim_v);
    if constexpr (NBB > kKeyBlocks) {
      // rows [q0-144, q0-128): RPI rows per DMA instruction, one instruction
      // for each of the first 16 / RPI waves (rows below 0 read as zero)
      constexpr int NI16 = 16 / RPI;
      if (w < NI16) {  // wave-uniform
        const int row0 = w1 - 16;
        const int sr = row0 + w * RPI + lane / TL::chunks;
        const int lo_r = row0 > 0 ? row0 : 0;
        const int hi_r = row0 + 16 < lim_v ? row0 + 16 : lim_v;
        const uint32_t bytes = hi_r > lo_r ? (uint32_t)(hi_r - 1 - lo_r) * rstride + D * sizeof(T) : 0u;
        const i32x4 rsrc = make_rsrc(v + ((size_t)(hi_r > lo_r ? lo_r : 0) * H + h) * D, bytes);
        const int rl = w * RPI + lane / TL::chunks;  // row within the 16
        const uint32_t vo = (sr >= lo_r && sr < hi_r)
                                ? (uint32_t)(sr - lo_r) * rstride + (uint32_t)TL::pos(rl, lane % TL::chunks) * 16u
                                : bytes;
        ldc_buffer_load_lds(rsrc, (lds_u32_ptr)(reinterpret_cast<char*>(s_ex) + w * 1024), 16, (int)vo, 0, 0, 0);
      }
    }
    uint32_t bw[NBB][4];
    {
      // word (b, 4g+i, n) of the wave's 16 x 16NBB band block
      const int qb = (q0 >> 4) + w, nqb = (a.T + 15) >> 4;
      const uint32_t* blk = a.band + (size_t)(qb < nqb ? qb : nqb - 1) * band_words<NBB>();
#pragma unroll
      for (int b = 0; b < NBB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) bw[b][i] = blk[b * 256 + (4 * g + i) * 16 + n];
    }
    wait_dma_except<0>();
    const float f = l * gh;
    f32x4 pb[NBB];
#pragma unroll
    for (int b = 0; b < NBB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[b][i] = f * band_decode<T>(bw[b][i]);
    BandOperand<T, NBB> bop;
    bop.set(pb);
    const char* blk[NBB];
#pragma unroll
    for (int b = 0; b < NBB; ++b) {
      const int r = 16 * w + 16 * b + 16 * (9 - NBB);  // wave-uniform, -16 .. 239
      const char* sl = reinterpret_cast<const char*>(r < 0 ? s_ex : r < R ? slot(IC<0>{}) : r < 2 * R ? slot(IC<1>{})
                                                     : r < 3 * R ? slot(IC<2>{}) : slot(IC<3>{}));
      blk[b] = sl + (r < 0 ? 0 : r % R) * TL::row_bytes;
    }
    __builtin_amdgcn_s_setprio(1);
    pv_stream<T, D, NBB, true>(acc, blk, lo, bop);
    __builtin_amdgcn_s_setprio(0);
  }
  const float inv = 1.f / l;  // l >= the diagonal key's weight, > 0
#pragma unroll
  for (int r = 0; r < D / 16; ++r) acc[r] *= inv;
  float* xp;
  if constexpr (kXpInRing) {
    __syncthreads();  // every wave is done reading the ring
    xp = reinterpret_cast<float*>(s_r0) + w * 512;
  } else {
    xp = s_xp + w * 512;
  }
  store_row<T, D>(pending_rows<D>(a.o, tw, n, a.T, H, h, true, 1.f, xp), acc, g, n);
}

template <typename T, int D>
static hipError_t launch_attn(const AttnArgs& a, bool ldc, hipStream_t st) {
  const int ntile = (a.T + kABQ - 1) / kABQ;
  const dim3 grid(ntile * a.H), block(kANW * kWave);
  if (ldc && a.window > kMaxWindow)
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, true, kKeyBlocks + 2>), grid, block, 0, st, a);
  else if (ldc)
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

size_t run_blocks(int64_t T) { return (size_t)((T + kRunBlock - 1) / kRunBlock); }

size_t order_ints(int64_t T) { return 2 * kOrderBins + (size_t)((T + kTileQ - 1) / kTileQ); }
int order_list_offset() { return 2 * kOrderBins; }

hipError_t run_starts_dispatch(const int32_t* doc, int T, int* last, int* rs, int* order, hipStream_t st) {
  const int nb = (int)run_blocks(T);
  hipLaunchKernelGGL(run_marks_kernel, dim3(nb), dim3(256), 0, st, doc, T, last, order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(run_starts_kernel, dim3(nb), dim3(256), 0, st, doc, T, last, rs, order);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntile = (T + kTileQ - 1) / kTileQ;
  hipLaunchKernelGGL(tile_order_kernel, dim3((ntile + 255) / 256), dim3(256), 0, st, rs, T, order);
  return hipGetLastError();
}

hipError_t attn_fwd_dispatch(int d, const AttnArgs& a, bool ldc, hipStream_t st) {
  if (d == 128) return launch_attn<bf16_t, 128>(a, ldc, st);
  return launch_attn<bf16_t, 64>(a, ldc, st);
}

}  // namespace ldc
