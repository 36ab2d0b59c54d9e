// Device-side building blocks of the Lightweight DC kernels for gfx950 (CDNA4).
//
// Fragment conventions (verified on gfx950 for v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32; lane l, group g = l/16, column n = l%16):
//   A operand   lane holds A[m = n][k-slots of group g]
//   B operand   lane holds B[k-slots of group g][n]
//   accumulator lane holds D[4g + i][n], i = 0..3
// bf16: group g owns k-slots 8g..8g+7; fp32: group g owns the single slot g.
//
// ds_read_tr16_b64 (gfx950 LDS transpose read), per 16-lane group: lane
// 4r+b supplies the address of 4 consecutive 16-bit elements; lane q
// receives element q%4 of the addresses supplied by lanes 4e + q/4, e = 0..3.
// Rows of a token-major LDS tile therefore land as the k-slots of an MFMA
// operand whose m index runs along the head dimension.
//
// buffer_load_dwordx4 ... lds (verified on gfx950): lane i's 16 bytes land at
// LDS address M0 + 16*i; offsets outside the buffer's range read as zero.
//
// LDS tiles are token-major rows of D elements with no padding; the 16-byte
// chunk c of row r is stored at chunk position c ^ swz(r).  The swizzle makes
// both read patterns conflict-free: 16 consecutive rows at one chunk per lane
// group (score operands, 16-byte reads) and 4 consecutive rows x 4
// consecutive chunks (transpose reads, 8-byte halves: the lanes reading
// chunks 4p and 4p+2 take one half, those reading 4p+1 and 4p+3 the other).
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT of single-pattern probes): a 16-byte
// read is served to two lane groups (32 lanes) at a time over 64 banks of 8
// bytes, so the two groups together must cover 64 distinct banks.  The row
// bit -> chunk bit maps below do that for both patterns; the plain
// (r & 3) << 2 | r >> 2 map of 16-chunk rows leaves every score read 2-way
// conflicted (~3.8 extra LDS cycles per instruction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ldc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage of one bfloat16
typedef __attribute__((address_space(3))) uint32_t* lds_u32_ptr;

constexpr int kWave = 64;
constexpr int kKeyBlocks = 8;                 // 16-token blocks in one wave's band
constexpr int kBand = 16 * kKeyBlocks;        // 128 tokens
constexpr int kHalo = kBand - 16;             // 112 rows before a 16-row block
constexpr int kMaxWindow = kHalo + 1;         // 113: widest window the band holds
constexpr float kLog2e = 1.4426950408889634f;

// Bands of NB key blocks (NB even: the bf16 token contraction takes key
// blocks in pairs).  NB = 8 holds windows up to 113 keys; NB = 10 up to 145
// (the widest window accepted is 128).  A lane holds 4 entries per block:
// its admission bits fit 32 bits for NB <= 8, 64 bits beyond.
template <int NB>
constexpr int halo_rows() {
  return 16 * (NB - 1);
}
template <int NB>
constexpr int band_words() {
  return NB * 256;
}
template <int NB>
using MaskT = typename std::conditional<(NB * 4 <= 32), uint32_t, uint64_t>::type;

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Direct global -> LDS load through a buffer resource (llvm.amdgcn.raw.buffer.load.lds).
extern "C" __device__ void ldc_buffer_load_lds(i32x4 rsrc, lds_u32_ptr lds, int size, int voffset,
                                               int soffset, int offset,
                                               int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr bool bf16 = true;
};
template <>
struct Elem<float> {
  static constexpr bool bf16 = false;
};

template <typename T, int D>
struct Tile {
  static constexpr int row_bytes = D * (int)sizeof(T);
  static constexpr int chunks = row_bytes / 16;      // 16-byte chunks per row
  static constexpr int rows_per_inst = 64 / chunks;  // rows one wave-wide DMA fills
  // chunk position of logical chunk c in row r
  static __device__ __forceinline__ int pos(int r, int c) {
    if constexpr (Elem<T>::bf16 && D == 16) {
      // 32-byte rows: a 16-row block is one contiguous 512-byte region, read
      // conflict-free by both patterns without a swizzle
      return c;
    } else if constexpr (Elem<T>::bf16 && D == 128) {
      // row bits 0, 1, 2, 3 -> chunk bits 0, 2, 3, 1
      return c ^ ((r & 1) | ((r & 6) << 1) | ((r >> 2) & 2));
    } else if constexpr (Elem<T>::bf16 && D == 64) {
      // row bits 1, 2, 3 -> chunk bits 0, 2, 1
      return c ^ (((r >> 1) & 1) | (r & 4) | ((r >> 2) & 2));
    } else if constexpr (D == 16) {
      return c ^ ((r >> 2) & 3);
    } else {
      return c ^ (r & 15);
    }
  }
  // byte offset of element `col` (16-byte aligned group start) in row r
  static __device__ __forceinline__ int off(int r, int col) {
    constexpr int epc = 16 / (int)sizeof(T);
    return r * row_bytes + pos(r, col / epc) * 16 + (col % epc) * (int)sizeof(T);
  }
};

// bf16 rows of 16 elements contract on v_mfma_f32_16x16x16_bf16 (K = 16, four
// bf16 values per lane); wider bf16 rows on the K = 32 instruction.
template <typename T, int D>
constexpr bool kNarrow = Elem<T>::bf16 && D == 16;

// Number of 32-bit registers the lane needs for one row's d-slice.
template <typename T, int D>
struct RowFrag {
  // bf16: D/32 chunks of 8 values (D = 16: one piece of 4); fp32: D/4 values
  // (one per 16x16x4 step)
  static constexpr int n = kNarrow<T, D> ? 1 : Elem<T>::bf16 ? D / 32 : D / 4;
  typename std::conditional<kNarrow<T, D>, bf16x4,
                            typename std::conditional<Elem<T>::bf16, bf16x8, float>::type>::type v[n];
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Index of this wave in the workgroup, as a wave-uniform (scalar) value, so
// that addresses derived from it stay in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                    0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(s * sl2 - m) with the product rounded before the subtraction (no FMA
// contraction): when m is the rounded product of the row max, the max entry
// gets exactly exp2(0) = 1, so a one-key window yields P = 1 exactly.
__device__ __forceinline__ float exp2_scaled(float s, float sl2, float m) {
#pragma clang fp contract(off)
  return __builtin_amdgcn_exp2f(s * sl2 - m);
}

// Reductions over the four 16-lane groups (lanes n, n+16, n+32, n+48) with
// the gfx950 lane-swap instructions (VALU only, no LDS round trip):
// permlane16_swap(x, x) returns {x of this lane or of lane^16} in some order,
// permlane32_swap(x, x) likewise for lane^32, so op(r[0], r[1]) combines the
// pair without a lane-dependent select.
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max4(float x) { return swap32_max(swap16_max(x)); }
__device__ __forceinline__ float wave_sum4(float x) { return swap32_sum(swap16_sum(x)); }

// Wave-uniform bit mask over the NB token blocks of a wave's band, from the
// lane's admission bits (bit 4b+i): bit b set when every entry of block b
// of every lane is admitted (no per-entry masking needed there).
template <int NB = kKeyBlocks>
__device__ __forceinline__ uint32_t full_blocks(MaskT<NB> mbits) {
  uint32_t full = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    full |= (__all(((mbits >> (4 * b)) & 15u) == 15u) ? 1u : 0u) << b;
  // one packed scalar, opaque, rather than 8 lane masks kept live for the tests
  asm volatile("" : "+s"(full));
  return full;
}
// x where entry (b, i) of the lane's band is admitted, else `other`: a bit
// select on the lane's admission bits, two vector ALU operations and no
// per-entry lane masks held in scalar registers.
__device__ __forceinline__ float keep_admitted(uint32_t mbits, int b, int i, float x, float other) {
  const int m = (int)(mbits << (31 - (4 * b + i))) >> 31;  // all ones when admitted
  return __int_as_float((__float_as_int(x) & m) | (__float_as_int(other) & ~m));
}
__device__ __forceinline__ float keep_admitted(uint64_t mbits, int b, int i, float x, float other) {
  const int m = (int)((int64_t)(mbits << (63 - (4 * b + i))) >> 63);
  return __int_as_float((__float_as_int(x) & m) | (__float_as_int(other) & ~m));
}
// The value unchanged, but opaque to the optimizer: used once per stage on
// the admission bits so that the 32 per-entry masks are formed where they are
// used instead of being hoisted out of the stage loop and kept live.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint64_t opaque(uint64_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// The same for a wave-uniform value (the full-block mask): its per-block
// branch conditions are then scalar bit tests at the point of use.
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Replace the entries of a lane's band that are not admitted by `other`.
// In a wave whose band lies inside one document, only the first and the last
// token blocks are partial (the window's far edge and the causal diagonal);
// that case takes a branch of its own, the general case tests every block.
template <int NB = kKeyBlocks>
__device__ __forceinline__ void mask_band(f32x4 (&p)[NB], MaskT<NB> mbits, uint32_t full, float other) {
  constexpr uint32_t kInner = ((1u << NB) - 1) & ~1u & ~(1u << (NB - 1));
  const MaskT<NB> mb = opaque(mbits);
  const uint32_t fl = opaque_s(full);
  if (fl == kInner) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[0][i] = keep_admitted(mb, 0, i, p[0][i], other);
      p[NB - 1][i] = keep_admitted(mb, NB - 1, i, p[NB - 1][i], other);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (!((fl >> b) & 1u))
#pragma unroll
        for (int i = 0; i < 4; ++i) p[b][i] = keep_admitted(mb, b, i, p[b][i], other);
  }
}

// ---------------------------------------------------------------------------
// Buffer resources and DMA staging
// ---------------------------------------------------------------------------
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);  // stride 0
  r[2] = (int)bytes;                            // num_records (bytes)
  r[3] = 0x00020000;                            // gfx9 data format: 32-bit, raw
  return r;
}

// Issue (asynchronously) the DMA of rows [row0, row0+R) of head h of a
// [T,H,D] tensor into an LDS tile; rows outside [0,T) read as zero, and
// nothing but zeros is read when !on.  Every wave issues the same number of
// DMA instructions, unconditionally (a surplus instruction repeats the last
// one: identical bytes to identical LDS addresses), so that the compiler's
// wait counters see one straight-line sequence of vector-memory operations.
// Completion is waited for with s_waitcnt vmcnt + a barrier by the caller.
// Instructions each wave issues for one tile (the issue_tile sequence length).
template <typename T, int D, int R, int NW>
constexpr int tile_insts_per_wave() {
  return (R / Tile<T, D>::rows_per_inst + NW - 1) / NW;
}

// With U0/U1, only instructions [U0, U1) of the wave's sequence are issued
// (for callers that spread the issue over a stage).
template <typename T, int D, int R, int NW, int U0 = 0, int U1 = 1 << 20>
__device__ __forceinline__ void issue_tile(T* tile, const T* __restrict__ src, int row0, int T_,
                                           int H, int h, bool on = true) {
  using TL = Tile<T, D>;
  constexpr int RPI = TL::rows_per_inst;
  static_assert(R % RPI == 0, "tile rows must fill whole DMA instructions");
  constexpr int NI = R / RPI;
  constexpr int NIW = (NI + NW - 1) / NW;  // instructions per wave
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lo = row0 > 0 ? row0 : 0;
  const int hi = (row0 + R < T_) ? row0 + R : T_;
  const uint32_t rstride = (uint32_t)H * D * sizeof(T);
  const uint32_t bytes =
      (on && hi > lo) ? (uint32_t)(hi - 1 - lo) * rstride + (uint32_t)D * sizeof(T) : 0u;
  const i32x4 rsrc = make_rsrc(src + ((size_t)(hi > lo ? lo : 0) * H + h) * D, bytes);
  const int rsub = lane / TL::chunks, pc = lane % TL::chunks;
  char* base = reinterpret_cast<char*>(tile);
#pragma unroll
  for (int u = U0; u < (U1 < NIW ? U1 : NIW); ++u) {
    const int j = (w + u * NW < NI) ? w + u * NW : NI - 1;
    const int rl = j * RPI + rsub;
    const int s = row0 + rl;
    const int lc = TL::pos(rl, pc);  // the swizzle is an involution: pos(pos(c)) = c
    const uint32_t voff = (s >= lo && s < hi) ? (uint32_t)(s - lo) * rstride + (uint32_t)lc * 16u : bytes;
    ldc_buffer_load_lds(rsrc, (lds_u32_ptr)(base + j * 1024), 16, (int)voff, 0, 0, 0);
  }
}

// Issue the DMA of the float scalars x[(t*H + h)*spt + fld] for rows
// [row0, row0+R) into an LDS array of round_up(R, 64) floats; rows outside
// [0,T) (or everything when !on) read as zero.  Same issue discipline as
// issue_tile.
template <int R, int NW>
__device__ __forceinline__ void issue_scalars(float* arr, const float* __restrict__ src, int spt,
                                              int fld, int row0, int T_, int H, int h,
                                              bool on = true) {
  constexpr int NI = (R + 63) / 64;
  constexpr int NIW = (NI + NW - 1) / NW;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lo = row0 > 0 ? row0 : 0;
  const int hi = (row0 + R < T_) ? row0 + R : T_;
  const uint32_t rstride = (uint32_t)H * spt * 4u;
  const uint32_t bytes = (on && hi > lo) ? (uint32_t)(hi - 1 - lo) * rstride + 4u : 0u;
  const i32x4 rsrc = make_rsrc(src + ((size_t)(hi > lo ? lo : 0) * H + h) * spt + fld, bytes);
  char* base = reinterpret_cast<char*>(arr);
#pragma unroll
  for (int u = 0; u < NIW; ++u) {
    const int j = (w + u * NW < NI) ? w + u * NW : NI - 1;
    const int s = row0 + j * 64 + lane;
    const uint32_t voff = (s >= lo && s < hi) ? (uint32_t)(s - lo) * rstride : bytes;
    ldc_buffer_load_lds(rsrc, (lds_u32_ptr)(base + j * 256), 4, (int)voff, 0, 0, 0);
  }
}

// Issue the DMA of the document ids of rows [row0, row0+R) into an LDS array
// of round_up(R, 64) ints; rows outside [0,T) read as 0.
template <int R, int NW>
__device__ __forceinline__ void issue_doc(int* s_doc, const int32_t* __restrict__ doc, int row0,
                                          int T_) {
  issue_scalars<R, NW>(reinterpret_cast<float*>(s_doc), reinterpret_cast<const float*>(doc), 1, 0,
                       row0, T_, 1, 0);
}

__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Wait until at most N of this wave's vector-memory operations are in flight
// and all its LDS operations are done, then barrier.  Loads complete in issue
// order, so when at least N loads were issued after the operations that must
// be complete (the DMA of the following stage, say), those are complete after
// the wait, whatever stores are still in flight.
template <int N>
__device__ __forceinline__ void wait_dma_except() {
  static_assert(N >= 0 && N < 64, "the vector-memory counter holds 6 bits");
  // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] (7: no wait), lgkmcnt[11:8]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// MFMA building blocks over staged tiles
// ---------------------------------------------------------------------------
// The d-slice of one token row that lane group g contributes to a contraction
// over the head dimension (global memory source; the caller passes a valid
// row and ignores the result of lanes it does not need).
// bf16: chunk kk holds d = 32kk + 8g .. +7.  fp32: slot kk holds d = g*D/4 + kk.
// NT: non-temporal loads (the caller reads each such row once).
template <typename T, int D, bool NT = false>
__device__ __forceinline__ void load_row_frag(RowFrag<T, D>& f, const T* __restrict__ row, int g) {
  if constexpr (kNarrow<T, D>) {
    // d = 4g .. 4g+3
    const u32x2* src = reinterpret_cast<const u32x2*>(row + 4 * g);
    f.v[0] = __builtin_bit_cast(bf16x4, NT ? __builtin_nontemporal_load(src) : *src);
  } else if constexpr (Elem<T>::bf16) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const u32x4* src = reinterpret_cast<const u32x4*>(row + 32 * kk + 8 * g);
      f.v[kk] = __builtin_bit_cast(bf16x8, NT ? __builtin_nontemporal_load(src) : *src);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 4; kk += 4) {
      const f32x4* src = reinterpret_cast<const f32x4*>(row + g * (D / 4) + kk);
      const f32x4 u = NT ? __builtin_nontemporal_load(src) : *src;
      f.v[kk] = u[0]; f.v[kk + 1] = u[1]; f.v[kk + 2] = u[2]; f.v[kk + 3] = u[3];
    }
  }
}

// Per-lane byte offsets of the LDS reads, relative to a tile row that is a
// multiple of 16 (every swizzle depends on row & 15 only).  With these, each
// read is tile + uniform row offset + one of a few lane offsets + an
// immediate, which keeps the address registers to a handful.
template <typename T, int D>
struct LaneOffsets {
  using TL = Tile<T, D>;
  static constexpr int ND = kNarrow<T, D> ? 1 : Elem<T>::bf16 ? D / 32 : D / 16;  // score reads per row
  static constexpr int NT = kNarrow<T, D> ? 1 : Elem<T>::bf16 ? D / 32 : 1;       // transpose column groups
  int dk[ND];  // score operand: row n of the block, chunk of k-step kk
  int tr[NT];  // value operand (bf16): row 4g + n/4, chunk 4p + n%4, half (n/4)%2 (for e = 0)
  __device__ __forceinline__ LaneOffsets(int g, int n) {
    if constexpr (kNarrow<T, D>) {
      // score operand: 8 bytes of row n at d = 4g; value operand: lane supplies
      // row 4g + n/4 at d = 4(n%4), so that lane q receives d = q of 4 rows
      dk[0] = n * TL::row_bytes + 8 * g;
      tr[0] = (4 * g + (n >> 2)) * TL::row_bytes + 8 * (n & 3);
    } else if constexpr (Elem<T>::bf16) {
#pragma unroll
      for (int kk = 0; kk < ND; ++kk) dk[kk] = n * TL::row_bytes + TL::pos(n, 4 * kk + g) * 16;
      const int rr = n >> 2, bq = n & 3, row = 4 * g + rr;
#pragma unroll
      for (int p = 0; p < NT; ++p) tr[p] = row * TL::row_bytes + TL::pos(row, 4 * p + bq) * 16 + 8 * (bq & 1);
    } else {
#pragma unroll
      for (int c = 0; c < ND; ++c) dk[c] = n * TL::row_bytes + TL::pos(n, g * (D / 16) + c) * 16;
      tr[0] = 0;
    }
  }
};

// acc += A x B for a contraction over the head dimension, where the A operand
// row (m = this lane's n) is tile row row16 + n (row16 a multiple of 16) and
// B is the fragment f.
template <typename T, int D>
__device__ __forceinline__ f32x4 mma_dcontract(f32x4 acc, const T* tile, int row16,
                                               const LaneOffsets<T, D>& lo, const RowFrag<T, D>& f) {
  using TL = Tile<T, D>;
  const char* base = reinterpret_cast<const char*>(tile) + row16 * TL::row_bytes;
  if constexpr (kNarrow<T, D>) {
    const uint2 u = *reinterpret_cast<const uint2*>(base + lo.dk[0]);
    acc = mma(__builtin_bit_cast(bf16x4, u), f.v[0], acc);
  } else if constexpr (Elem<T>::bf16) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint4 u = *reinterpret_cast<const uint4*>(base + lo.dk[kk]);
      acc = mma(__builtin_bit_cast(bf16x8, u), f.v[kk], acc);
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      float4 u = *reinterpret_cast<const float4*>(base + lo.dk[c]);
      acc = mma(u.x, f.v[4 * c], acc);
      acc = mma(u.y, f.v[4 * c + 1], acc);
      acc = mma(u.z, f.v[4 * c + 2], acc);
      acc = mma(u.w, f.v[4 * c + 3], acc);
    }
  }
  return acc;
}

// All NB key blocks of a band at once: s[b] = A x B with the A operand rows
// row16 + 16b + n.  For bf16 tiles the LDS reads of the next G blocks are
// issued ahead of the MFMAs of the current G (scheduling groups pin that
// order), whose G dependent chains alternate: a wave that is alone on its
// SIMD would otherwise wait out the LDS latency before every MFMA.  G = 2
// keeps up to 4 blocks of operands in registers, G = 1 up to 2.
template <typename T, int D, int NB, int G = 2>
__device__ __forceinline__ void mma_dcontract_band(f32x4 (&s)[NB], const T* tile, int row16,
                                                   const LaneOffsets<T, D>& lo, const RowFrag<T, D>& f) {
  if constexpr (Elem<T>::bf16 && !kNarrow<T, D> && NB % G == 0) {
    using TL = Tile<T, D>;
    constexpr int KK = D / 32;
    const char* base = reinterpret_cast<const char*>(tile) + row16 * TL::row_bytes;
    bf16x8 u[NB][KK];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        u[b][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(base + 16 * b * TL::row_bytes +
                                                                              lo.dk[kk]));
#pragma unroll
    for (int b = 0; b < NB; b += G) {
      f32x4 a[G];
#pragma unroll
      for (int c = 0; c < G; ++c) a[c] = zero4();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int c = 0; c < G; ++c) a[c] = mma(u[b + c][kk], f.v[kk], a[c]);
#pragma unroll
      for (int c = 0; c < G; ++c) s[b + c] = a[c];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, G * KK, 0);  // LDS reads, first G blocks
#pragma unroll
    for (int b = 0; b < NB; b += G) {
      if (b + G < NB) __builtin_amdgcn_sched_group_barrier(0x100, G * KK, 0);  // reads, next G
      __builtin_amdgcn_sched_group_barrier(0x008, G * KK, 0);                  // MFMAs, these G
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b] = mma_dcontract<T, D>(zero4(), tile, row16 + 16 * b, lo, f);
  }
}

// Token-contraction operand: a 16 x 16NB band held in accumulator layout
// (lane: token rows 4g+i of block b, column n) packed as B-operand k-chunks.
// bf16: chunk ks covers blocks 2ks, 2ks+1; slot j <-> block 2ks + j/4, row 4g + j%4.
// The fp32 band is carried as two bf16 operands, hi = bf16(x) and
// lo = bf16(x - hi), so the contraction keeps ~16 mantissa bits of x; the
// other operand (a bf16 input tensor) is exact.
template <typename T, int NB = kKeyBlocks>
struct BandOperand;
template <int NB>
struct BandOperand<bf16_t, NB> {
  bf16x8 hi[NB / 2], lo[NB / 2];
  __device__ __forceinline__ void set(const f32x4 (&p)[NB]) {
#pragma unroll
    for (int ks = 0; ks < NB / 2; ++ks) {
      u32x4 h4, l4;
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) {
        // slots 2jp, 2jp+1: one packed conversion for the pair, the high
        // parts widened back by shifts, one packed conversion of the remainders
        const float x0 = p[2 * ks + (jp >> 1)][2 * (jp & 1)];
        const float x1 = p[2 * ks + (jp >> 1)][2 * (jp & 1) + 1];
        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
        const float r0 = x0 - __uint_as_float(hb << 16);
        const float r1 = x1 - __uint_as_float(hb & 0xffff0000u);
        h4[jp] = hb;
        l4[jp] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
      }
      hi[ks] = __builtin_bit_cast(bf16x8, h4);
      lo[ks] = __builtin_bit_cast(bf16x8, l4);
    }
  }
};
template <int NB>
struct BandOperand<float, NB> {
  f32x4 v[NB];
  __device__ __forceinline__ void set(const f32x4 (&p)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) v[b] = p[b];
  }
};

// Offset (elements) of the 4 consecutive d-values a lane holds in acc[r] of
// mma_tcontract's result (the lane's group g; layout given there).
template <typename T, int D>
__device__ __forceinline__ int tcontract_d(int r, int g) {
  if constexpr (Elem<T>::bf16 && !kNarrow<T, D>)
    return 32 * (r >> 1) + 8 * g + 4 * ((r & 1) ^ (g & 1));
  else
    return 16 * r + 4 * g;
}

// Output rows are written once and never read back by the kernel that writes
// them, so every output store is non-temporal (streaming): it does not take
// cache lines from the input tiles whose halo rows neighbouring workgroups
// share through L2.  Measured at the GPT-2 small layer: forward -13%,
// backward kernels -4 to -7%.
__device__ __forceinline__ void store4(float* dst, f32x4 v, float s) {
  __builtin_nontemporal_store(f32x4{v[0] * s, v[1] * s, v[2] * s, v[3] * s},
                              reinterpret_cast<f32x4*>(dst));
}

// A wave's finished output rows (one per lane column n) still held in
// registers, to be stored while the next result is computed.
struct PendingRow {
  float* row;    // this lane's row (row0 + n * stride)
  float scale;
  bool on;       // this lane's row exists and is pending
  float* row0;   // the wave's first row; rows row0 + i * stride, i = 0..15
  int nrows;     // rows [0, nrows) exist and are pending (0: none); wave-uniform
  int stride;    // floats between consecutive rows
  float* xp;     // the wave's LDS scratch (16 x 32 floats), bf16 path
};

// Rows r0 + i (i = 0..15, r0 >= 0 wave-uniform) of head h of a [T,H,D]
// float32 tensor; `pend` false (or rows at or past T_) stores nothing.
template <int D>
__device__ __forceinline__ PendingRow pending_rows(float* base, int r0, int n, int T_, int H, int h,
                                                   bool pend, float scale, float* xp) {
  const int left = T_ - r0;
  const int nrows = pend ? (left < 0 ? 0 : left > 16 ? 16 : left) : 0;
  float* row0 = base + ((size_t)r0 * H + h) * D;
  return PendingRow{row0 + (size_t)n * H * D, scale, n < nrows, row0, nrows, H * D, xp};
}

// Store columns [32p, 32p+32) of a pending bf16-path row block as whole
// 128-byte lines (8 rows per instruction: measured 12% more write bandwidth
// than 16 rows of four scattered 16-byte pieces).  The slice's two
// accumulator registers go through the wave's LDS scratch: lane (g, n) holds
// chunks 2g + (e ^ g%2) (register e) of row n; 16-byte chunk c of row r sits
// at chunk position c ^ (r % 8), so both the writes (8 rows at one chunk)
// and the reads (one row's 8 chunks) are conflict-free.  Reads of one wave
// follow its writes in LDS order, so no barrier is needed.
__device__ __forceinline__ void store_slice(const PendingRow& pr, const f32x4& a0, const f32x4& a1,
                                            int p, int g, int n) {
  char* xp = reinterpret_cast<char*>(pr.xp);
  const int c0 = 2 * g + (g & 1), c1 = 2 * g + 1 - (g & 1);
  *reinterpret_cast<f32x4*>(xp + n * 128 + ((c0 ^ (n & 7)) << 4)) = a0;
  *reinterpret_cast<f32x4*>(xp + n * 128 + ((c1 ^ (n & 7)) << 4)) = a1;
  const int lane = threadIdx.x & 63, rr = lane >> 3, c = lane & 7;
  const f32x4 v0 = *reinterpret_cast<const f32x4*>(xp + rr * 128 + ((c ^ rr) << 4));
  const f32x4 v1 = *reinterpret_cast<const f32x4*>(xp + (rr + 8) * 128 + ((c ^ rr) << 4));
  float* dst = pr.row0 + 32 * p + 4 * c;
  if (rr < pr.nrows) store4(dst + (size_t)rr * pr.stride, v0, pr.scale);
  if (rr + 8 < pr.nrows) store4(dst + (size_t)(rr + 8) * pr.stride, v1, pr.scale);
}

// Store a whole pending row block (a tcontract result, scaled by pr.scale).
template <typename T, int D>
__device__ __forceinline__ void store_row(const PendingRow& pr, const f32x4 (&acc)[D / 16], int g,
                                          int n) {
  if constexpr (Elem<T>::bf16 && !kNarrow<T, D>) {
    if (pr.nrows > 0)
#pragma unroll
      for (int p = 0; p < D / 32; ++p) store_slice(pr, acc[2 * p], acc[2 * p + 1], p, g, n);
  } else {
    if (pr.on)
#pragma unroll
      for (int r = 0; r < D / 16; ++r) store4(pr.row + tcontract_d<T, D>(r, g), acc[r], pr.scale);
  }
}

// Keep vector-memory writes from being moved across this point by the
// scheduler; every other kind of instruction may still move across it.
__device__ __forceinline__ void store_fence() { __builtin_amdgcn_sched_barrier(0x00A1); }

// Contraction over the 16NB band tokens:  out[d, n] = sum_tok X[tok, d] * P[tok, n]
// with X a staged tile (rows base_row + tok) and P the band operand.
// Result layout (lane: column n; register r = 4*blk + i):
//   bf16: acc[2p+e][i] <-> d = 32p + 8g + 4(e ^ g%2) + i  (8 consecutive d per p, g)
//   fp32: acc[db][i]   <-> d = 16db + 4g + i
// Every token block is contracted (entries outside the band are zero in P):
// no branches, so the LDS reads of all blocks can be in flight together.
// acc holds the previous result rows `prev` on entry; they are stored group
// by group just before the group's registers are reused (bf16: as whole lines,
// see store_slice), so the stores leave spread over the contraction instead
// of in one burst (a burst of stores stalls the wave until the memory
// pipeline has taken them).
// hook(Part<k>) runs before column group k >= 1 (bf16; k < tcontract_groups),
// so that callers can spread other work (the next stage's DMA) over the
// contraction.
template <int P>
using Part = std::integral_constant<int, P>;
template <typename T, int D>
constexpr int tcontract_groups() {
  return (Elem<T>::bf16 && !kNarrow<T, D>) ? D / 32 : 1;
}
struct NoHook {
  template <typename P>
  __device__ __forceinline__ void operator()(P) const {}
};
template <typename T, int D, int NB = kKeyBlocks, typename Hook = NoHook>
__device__ __forceinline__ void mma_tcontract(f32x4 (&acc)[D / 16], const T* tile, int row16,
                                              const LaneOffsets<T, D>& lo, const BandOperand<T, NB>& P,
                                              int g, int n, const PendingRow& prev,
                                              Hook&& hook = Hook{}) {
  using TL = Tile<T, D>;
  const char* base = reinterpret_cast<const char*>(tile) + row16 * TL::row_bytes;
  if constexpr (kNarrow<T, D>) {
    // K = 16 steps: one transpose read per 16-token block (rows 4g..4g+3 of
    // the block for lane group g), contracted with that block's half of the
    // band operand's hi and lo chunks
    typedef __attribute__((address_space(3))) bf16x4 lds_v4;
    if (prev.on) store4(prev.row + tcontract_d<T, D>(0, g), acc[0], prev.scale);
    store_fence();
    acc[0] = zero4();
#pragma unroll
    for (int ks = 0; ks < NB / 2; ++ks) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4*)(base + lo.tr[0] + (32 * ks + 16 * half) * TL::row_bytes));
        const bf16x4 ph = half ? __builtin_shufflevector(P.hi[ks], P.hi[ks], 4, 5, 6, 7)
                               : __builtin_shufflevector(P.hi[ks], P.hi[ks], 0, 1, 2, 3);
        const bf16x4 pl = half ? __builtin_shufflevector(P.lo[ks], P.lo[ks], 4, 5, 6, 7)
                               : __builtin_shufflevector(P.lo[ks], P.lo[ks], 0, 1, 2, 3);
        acc[0] = mma(x, ph, acc[0]);
        acc[0] = mma(x, pl, acc[0]);
      }
    }
  } else if constexpr (Elem<T>::bf16) {
    typedef __attribute__((address_space(3))) bf16x4 lds_v4;
    constexpr int NP = D / 32;  // column groups of 32
    constexpr int PG = 1;       // column groups per store group
    static_for<0, NP / PG>([&](auto gi) {
      constexpr int p0 = decltype(gi)::value * PG;
      if constexpr (p0 > 0) hook(Part<p0 / PG>{});
      if (prev.nrows > 0)
#pragma unroll
        for (int p = p0; p < p0 + PG; ++p) store_slice(prev, acc[2 * p], acc[2 * p + 1], p, g, n);
      store_fence();
#pragma unroll
      for (int r = 2 * p0; r < 2 * (p0 + PG); ++r) acc[r] = zero4();
#pragma unroll
      for (int ks = 0; ks < NB / 2; ++ks) {
#pragma unroll
        for (int p = p0; p < p0 + PG; ++p) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            // rows 32ks + 4g + n/4 and 16 further down: same swizzle, immediate
            // offsets; e flips the 8-byte half the lane reads (recomputed at
            // each use rather than held in registers across the loop)
            int off = lo.tr[p];
            if (e) asm volatile("v_xor_b32 %0, 8, %0" : "+v"(off));
            const char* a1 = base + off + 32 * ks * TL::row_bytes;
            const char* a2 = a1 + 16 * TL::row_bytes;
            bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a1));
            bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a2));
            bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[2 * p + e] = mma(a, P.hi[ks], acc[2 * p + e]);
            acc[2 * p + e] = mma(a, P.lo[ks], acc[2 * p + e]);
          }
        }
      }
    });
  } else {
    if (prev.on)
#pragma unroll
      for (int r = 0; r < D / 16; ++r) store4(prev.row + tcontract_d<T, D>(r, g), acc[r], prev.scale);
    store_fence();
#pragma unroll
    for (int r = 0; r < D / 16; ++r) acc[r] = zero4();
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * b + 4 * g + i;  // relative to row16
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const float x = *reinterpret_cast<const float*>(base + TL::off(r, 16 * db + n));
          acc[db] = mma(x, P.v[b][i], acc[db]);
        }
      }
    }
  }
}

// mma_tcontract for waves that run alone on their SIMD (bf16, D >= 64): the
// pending rows are stored first (all column groups), then the LDS operands of
// column group p+1 are read while the MFMAs of group p run, with the group's
// two chains (e = 0, 1) alternating, so the LDS latency and the MFMA
// dependency are paid once per group rather than once per MFMA.
template <typename T, int D, int NB = kKeyBlocks>
__device__ __forceinline__ void mma_tcontract_pipe(f32x4 (&acc)[D / 16], const T* tile, int row16,
                                                   const LaneOffsets<T, D>& lo, const BandOperand<T, NB>& P,
                                                   int g, int n, const PendingRow& prev) {
  if constexpr (Elem<T>::bf16 && !kNarrow<T, D>) {
    using TL = Tile<T, D>;
    typedef __attribute__((address_space(3))) bf16x4 lds_v4;
    constexpr int NP = D / 32;
    const char* base = reinterpret_cast<const char*>(tile) + row16 * TL::row_bytes;
    if (prev.nrows > 0)
#pragma unroll
      for (int p = 0; p < NP; ++p) store_slice(prev, acc[2 * p], acc[2 * p + 1], p, g, n);
    store_fence();
    bf16x8 a[NP][NB / 2][2];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ks = 0; ks < NB / 2; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // rows 32ks + 4g + n/4 and 16 further down; e flips the lane's 8-byte half
          const char* a1 = base + (lo.tr[p] ^ (8 * e)) + 32 * ks * TL::row_bytes;
          const bf16x4 l4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a1));
          const bf16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(a1 + 16 * TL::row_bytes));
          a[p][ks][e] = __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      f32x4 c0 = zero4(), c1 = zero4();
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
    constexpr int RD = 2 * NB;  // LDS reads per column group
    constexpr int MF = 2 * NB;  // MFMAs per column group
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p + 1 < NP) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    }
  } else {
    mma_tcontract<T, D, NB>(acc, tile, row16, lo, P, g, n, prev);
  }
}

// ---------------------------------------------------------------------------
// Saved shared-map band and dPbar band
// ---------------------------------------------------------------------------
// Per 16-query block qb: NB key blocks kb, each a [key 16][query 16] array of
// 4-byte words; key block kb of query block qb holds keys 16*qb - 16(NB-1) + 16*kb
// + (0..15).  Word of the shared map: bf16 path (hi | lo << 16) with
// hi = bf16(x), lo = bf16(x - hi); fp32 path: the float.  The dPbar band
// (float32) uses the same indexing.  Query-centric waves (lane = query n,
// keys 4g+i of block b) touch word (4g+i)*16 + n; key-centric waves (lane =
// key n, queries 4g+i of query block qb + b) read the 16 bytes at n*16 + 4g.
constexpr int kBandWords = kKeyBlocks * 256;  // words per 16-query block

__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}
template <typename T>
__device__ __forceinline__ uint32_t band_encode(float x) {
  if constexpr (Elem<T>::bf16) {
    const uint32_t h = bf16_bits_rne(x);
    const uint32_t l = bf16_bits_rne(x - bf16_bits_to_float(h));
    return h | (l << 16);
  } else {
    return __float_as_uint(x);
  }
}
template <typename T>
__device__ __forceinline__ float band_decode(uint32_t u) {
  if constexpr (Elem<T>::bf16)
    return bf16_bits_to_float(u & 0xffffu) + bf16_bits_to_float(u >> 16);
  else
    return __uint_as_float(u);
}

// A query-centric wave's band block (lane (g, n) holds words (4g+i)*16 + n
// of key block b, i = 0..3) stored as whole 1 KB lines: through the wave's 2 KB LDS scratch, two key blocks at a time, so
// each instruction covers one contiguous key block (lane l: words 4l..4l+3)
// instead of 32 scattered 4-byte accesses per lane.  `blk` is the block's
// first word (16-byte aligned); one wave's scratch accesses follow each other
// in LDS order, so no barrier is needed.
template <int NB = kKeyBlocks>
__device__ __forceinline__ void store_band_block(uint32_t* blk, const uint32_t (&wv)[NB][4], float* xp,
                                                 int g, int n) {
  uint32_t* xs = reinterpret_cast<uint32_t*>(xp);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < NB / 2; ++r) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[bb * 256 + (4 * g + i) * 16 + n] = wv[2 * r + bb][i];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(xs + bb * 256 + 4 * lane),
                                  reinterpret_cast<u32x4*>(blk + (2 * r + bb) * 256 + 4 * lane));
  }
}
// Workgroup -> tile map that gives each XCD a contiguous run of tiles, so the
// halo rows a tile shares with its neighbour are fetched through the same L2.
// (Workgroups are dispatched to the 8 XCDs round-robin by block index.)
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
  constexpr int X = 8;
  const int xcd = bid % X, idx = bid / X;
  const int q = nblocks / X, rem = nblocks % X;
  return xcd * q + (xcd < rem ? xcd : rem) + idx;
}

}  // namespace ldc
