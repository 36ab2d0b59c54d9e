// Generator of the Lightweight DC weights for gfx950: C = x WC and G = x WG
// from the layer's input hidden state, and their gradients.
//
// Reading (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
// section "第二刀-砍层内", DCMHA and Lightweight DC paragraphs: the
// composition is decided from the current input): both weights are linear
// projections of x[t], no bias, no nonlinearity.  Together they are one
// skinny product x [T, dm] x W [dm, 2H] with 2H <= 16 output columns; the
// work is bound by reading x (forward) and by reading x and writing dx
// (backward).
//  * cg_fwd: MFMA.  Each wave computes 16-token x 16-column tiles, D^T =
//    W^T x^T: the A operand is W^T, staged once per workgroup in LDS (rows
//    padded by 16 bytes, so the 16 lanes of a group read 16 different banks),
//    the B operand is x, 16 bytes per lane per k-step straight from HBM, with
//    two batches of eight k-steps in flight ahead of the one contracted.
//  * cg_bwd: VALU streaming.  A thread owns four feature columns i of W (its
//    4 x 2H weights in registers) and walks a run of tokens: dx[t, i] =
//    sum_j dCG[t, j] W[i, j] is written as it goes and dW[i, j] += x[t, i]
//    dCG[t, j] accumulates in registers; dCG of the chunk is staged in LDS
//    and read as broadcasts.  Each chunk leaves its dW partial in the
//    workspace and cg_reduce sums the partials in a fixed order
//    (deterministic, no atomics).
#include "cg_internal.h"
#include "ldc_device.hpp"

namespace ldc {

constexpr int kCgCols = 16;      // output columns of the MFMA tile (2H <= 16)
constexpr int kCgWaves = 4;      // waves per cg_fwd workgroup
constexpr int kCgBlocks = 4;     // 16-token blocks per wave
constexpr int kCgChunk = 256;    // tokens per cg_bwd workgroup

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// BPB > 0: dm = BPB x 256 (bf16) or BPB x 128 (fp32), every batch of eight
// k-steps whole; waves with all kCgBlocks blocks then run a fully unrolled
// stream of batches with no branch.  BPB = 0: any dm (a multiple of 64).
template <typename T, int BPB>
__global__ __launch_bounds__(kCgWaves * kWave) void cg_fwd_kernel(const CgArgs a) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int KS = 4 * EPC;               // features per k-step (the 4 groups' chunks): 32 bf16, 16 f32
  constexpr int U = 8;                      // k-steps per batch of loads
  extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
  T* s_wt = reinterpret_cast<T*>(s_raw);   // W^T [16][dm + EPC]
  const int dm = a.dm, H = a.H, ld = dm + EPC;
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ wc = static_cast<const T*>(a.wc);
  const T* __restrict__ wg = static_cast<const T*>(a.wg);

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, n = lane & 15;
  const int tb0 = (blockIdx.x * kCgWaves + w) * kCgBlocks;  // the wave's first 16-token block
  const bool full = (tb0 + kCgBlocks) * 16 <= a.T;          // wave-uniform
  constexpr int NB = kCgBlocks * BPB;                       // batches of a full wave (fast path)
  constexpr int BP1 = BPB > 0 ? BPB : 1;
  auto load = [&](u32x4 (&dst)[U], int bi) {
    const int blk = bi / BP1, k0 = (bi % BP1) * U * KS;
    const T* xrow = x + (size_t)((tb0 + blk) * 16 + n) * dm + k0 + g * EPC;
#pragma unroll
    for (int u = 0; u < U; ++u) dst[u] = *reinterpret_cast<const u32x4*>(xrow + u * KS);
  };
  u32x4 xb[3][U];
  if constexpr (BPB > 0) {
    if (full) {  // the first two batches of x arrive while W^T is staged
      load(xb[0], 0);
      load(xb[1], 1);
    }
  }

  // Stage W^T: row j < H from WC, H <= j < 2H from WG, the rest zero.
  if constexpr (BPB > 0 && Elem<T>::bf16) {
    // dm = 256 BPB: thread r stages rows r + 256 q, q < BPB; all its
    // 16 BPB loads (each from a valid address) go out before any write
    T v[BPB][kCgCols];
#pragma unroll
    for (int q = 0; q < BPB; ++q) {
      const int i = (int)threadIdx.x + 256 * q;
#pragma unroll
      for (int j = 0; j < kCgCols; ++j) {
        const T* src = j < H ? wc + (size_t)i * H + j : wg + (size_t)i * H + (j < 2 * H ? j - H : 0);
        v[q][j] = *src;
      }
    }
#pragma unroll
    for (int q = 0; q < BPB; ++q) {
      const int i = (int)threadIdx.x + 256 * q;
#pragma unroll
      for (int j = 0; j < kCgCols; ++j) s_wt[j * ld + i] = j < 2 * H ? v[q][j] : T(0);
    }
  } else {
    // any dm: a thread's eight elements of a round are loaded (each from a
    // valid address) before any is written, so their latencies overlap
    {
      const int ne = kCgCols * dm;
      for (int e0 = threadIdx.x; e0 < ne; e0 += 8 * (int)blockDim.x) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u * (int)blockDim.x;
          const int ec = e < ne ? e : 0;
          const int j = ec / dm, i = ec - j * dm;
          const T* src = j < H ? wc + (size_t)i * H + j : wg + (size_t)i * H + (j < 2 * H ? j - H : 0);
          v[u] = *src;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u * (int)blockDim.x;
          if (e < ne) {
            const int j = e / dm, i = e - j * dm;
            s_wt[j * ld + i] = j < 2 * H ? v[u] : T(0);
          }
        }
      }
    }
  }
  __syncthreads();

  const T* arow = s_wt + n * ld;  // A operand row: output column n
  // lane (g, n) holds columns 4g+i of token t
  auto store_block = [&](const f32x4& acc, int t) {
    if (t < a.T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * g + i;
        if (j < H)
          a.c[(size_t)t * H + j] = acc[i];
        else if (j < 2 * H)
          a.g[(size_t)t * H + (j - H)] = acc[i];
      }
    }
  };
  auto contract = [&](f32x4& acc, const u32x4& wb, const u32x4& xv) {
    if constexpr (Elem<T>::bf16) {
      acc = mma(__builtin_bit_cast(bf16x8, wb), __builtin_bit_cast(bf16x8, xv), acc);
    } else {
      const f32x4 xf = __builtin_bit_cast(f32x4, xv), wf = __builtin_bit_cast(f32x4, wb);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma(wf[e], xf[e], acc);
    }
  };

  if constexpr (BPB > 0) {
    if (full) {
      // The wave's kCgBlocks x BPB batches as one stream, the loads of the
      // next two batches in flight while one is contracted (three register
      // slots, all fixed at compile time).
      f32x4 acc = zero4();
      static_for<0, NB>([&](auto bc) {
        constexpr int bi = decltype(bc)::value;
        if constexpr (bi + 2 < NB) load(xb[(bi + 2) % 3], bi + 2);
        constexpr int k0 = (bi % BPB) * U * KS;
#pragma unroll
        for (int u = 0; u < U; ++u)
          contract(acc, *reinterpret_cast<const u32x4*>(arow + k0 + u * KS + g * EPC), xb[bi % 3][u]);
        if constexpr (bi % BPB == BPB - 1) {
          store_block(acc, (tb0 + bi / BPB) * 16 + n);
          acc = zero4();
        }
      });
      return;
    }
  }
  // any dm, and the last waves of the stream: block by block, eight k-steps'
  // loads in flight before their MFMAs
  for (int blk = 0; blk < kCgBlocks; ++blk) {
    const int t0 = (tb0 + blk) * 16;
    if (t0 >= a.T) break;  // wave-uniform
    const int t = t0 + n;
    const T* xrow = x + (size_t)(t < a.T ? t : a.T - 1) * dm;
    f32x4 acc = zero4();
    for (int k0 = 0; k0 < dm; k0 += U * KS) {
      u32x4 xb[U], wb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * KS + g * EPC;
        const bool in = k0 + u * KS < dm;
        xb[u] = in ? *reinterpret_cast<const u32x4*>(xrow + k) : u32x4{0, 0, 0, 0};
        wb[u] = in ? *reinterpret_cast<const u32x4*>(arow + k) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) contract(acc, wb[u], xb[u]);
    }
    store_block(acc, t);
  }
}

// ---------------------------------------------------------------------------
// backward: dx and per-chunk dW partials
// A thread owns 4 feature columns (8-byte bf16 / 16-byte f32 loads, 16-byte
// dx stores); the chunk's tokens are split over kCgSub sub-groups of
// threads, each streaming a contiguous run with kCgU tokens in flight.  The
// sub-groups' dW sums are added in LDS in sub-group order.
// ---------------------------------------------------------------------------
constexpr int kCgThreads = 768;  // threads per cg_bwd workgroup (at most)

template <typename T>
struct TypeTag {
  using type = T;
};

// NJ: output columns 2H rounded up to a multiple of 4 (registers held per feature)
template <typename T, int NJ>
__global__ __launch_bounds__(kCgThreads) void cg_bwd_kernel(const CgBwdArgs a) {
  constexpr int kCgU = NJ > 12 ? 4 : 8;  // tokens in flight (registers: 4 x NJ weights and sums)
  __shared__ float s_d[kCgChunk * kCgCols];  // dCG of the chunk: [token][j], j < 2H
  extern __shared__ __attribute__((aligned(16))) float s_acc[];  // [kCgCols][dm]
  const int dm = a.dm, H = a.H, J = 2 * H;
  const int nf = dm / 4;  // feature threads per sub-group
  const int t0 = blockIdx.x * kCgChunk;
  const int nt = a.T - t0 < kCgChunk ? a.T - t0 : kCgChunk;
  // loads unconditional (from a valid address, then selected), so that a
  // thread's loads are in flight together rather than waited for one by one
  {
    constexpr int NE = kCgChunk * kCgCols;
    constexpr int R = (NE + 511) / 512;  // rounds for the smallest block (512 threads)
    float v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = threadIdx.x + r * (int)blockDim.x;
      const int tt = e / kCgCols, j = e - tt * kCgCols;
      const int tc = t0 + (tt < nt ? tt : 0);
      const float* src = j < H ? a.dc + (size_t)tc * H + j : a.dg + (size_t)tc * H + (j < J ? j - H : 0);
      v[r] = *src;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = threadIdx.x + r * (int)blockDim.x;
      const int tt = e / kCgCols, j = e - tt * kCgCols;
      if (e < NE) s_d[e] = (tt < nt && j < J) ? v[r] : 0.f;
    }
  }
  __syncthreads();
  const int nsub = blockDim.x / nf;  // token sub-groups
  const int sub = threadIdx.x / nf, f = threadIdx.x - sub * nf;
  const int i0 = 4 * f;  // this thread's feature columns i0 .. i0+3
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ wc = static_cast<const T*>(a.wc);
  const T* __restrict__ wg = static_cast<const T*>(a.wg);
  auto tof = [](T v) -> float {
    if constexpr (Elem<T>::bf16)
      return __uint_as_float((uint32_t)v << 16);
    else
      return v;
  };
  float wv[4][NJ], acc[4][NJ];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const size_t r = (size_t)(i0 + c) * H;
      const T* src = j < H ? wc + r + j : wg + r + (j < J ? j - H : 0);
      const float wj = tof(*src);
      wv[c][j] = j < J ? wj : 0.f;
      acc[c][j] = 0.f;
    }
  // this sub-group's tokens: [lo, hi) of the chunk
  const int per = (kCgChunk + nsub - 1) / nsub;
  const int lo = sub * per, hi = lo + per < nt ? lo + per : nt;
  for (int tt = lo; tt < hi; tt += kCgU) {
    float xv[kCgU][4];
#pragma unroll
    for (int u = 0; u < kCgU; ++u) {
      const int tk = t0 + (tt + u < hi ? tt + u : hi - 1);
      const T* p = x + (size_t)tk * dm + i0;
      if constexpr (Elem<T>::bf16) {
        const uint2 b = *reinterpret_cast<const uint2*>(p);
        xv[u][0] = __uint_as_float(b.x << 16);
        xv[u][1] = __uint_as_float(b.x & 0xffff0000u);
        xv[u][2] = __uint_as_float(b.y << 16);
        xv[u][3] = __uint_as_float(b.y & 0xffff0000u);
      } else {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
        for (int c = 0; c < 4; ++c) xv[u][c] = v[c];
      }
    }
#pragma unroll
    for (int u = 0; u < kCgU; ++u) {
      if (tt + u >= hi) break;
      const float* d = s_d + (tt + u) * kCgCols;
      f32x4 dx = zero4();
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float dj = d[j];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          dx[c] = fmaf(dj, wv[c][j], dx[c]);
          acc[c][j] = fmaf(xv[u][c], dj, acc[c][j]);
        }
      }
      __builtin_nontemporal_store(dx, reinterpret_cast<f32x4*>(a.dx + (size_t)(t0 + tt + u) * dm + i0));
    }
  }
  // sum the sub-groups' dW in LDS, in sub-group order
  for (int s = 0; s < nsub; ++s) {
    if (sub == s) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        f32x4* dst = reinterpret_cast<f32x4*>(s_acc + (size_t)j * dm + i0);
        const f32x4 v = f32x4{acc[0][j], acc[1][j], acc[2][j], acc[3][j]};
        *dst = s == 0 ? v : *dst + v;
      }
    }
    __syncthreads();
  }
  // this chunk's partial: [chunk][j][i]
  float* part = a.partial + (size_t)blockIdx.x * kCgCols * dm;
  for (int e = threadIdx.x; e < J * nf; e += blockDim.x) {
    const int j = e / nf, ff = e - j * nf;
    *reinterpret_cast<f32x4*>(part + (size_t)j * dm + 4 * ff) =
        *reinterpret_cast<const f32x4*>(s_acc + (size_t)j * dm + 4 * ff);
  }
}

// dW[i, j] = sum over chunks of the partials.  A workgroup takes 64
// consecutive outputs (one per lane) and kRedWaves waves; wave s sums the
// chunks s, s + kRedWaves, ... in order, then wave 0 adds the waves' sums in
// wave order (deterministic).
constexpr int kRedWaves = 8;
__global__ __launch_bounds__(kRedWaves * kWave) void cg_reduce_kernel(const CgBwdArgs a, int nchunks) {
  __shared__ float s_part[kRedWaves][kWave];
  const int J = 2 * a.H, lane = threadIdx.x & 63, w = wave_id();
  const int e = blockIdx.x * kWave + lane;  // (j, i)
  const bool on = e < J * a.dm;
  const int j = on ? e / a.dm : 0, i = on ? e - j * a.dm : 0;
  float sum = 0.f;
  if (on) {
    const float* p = a.partial + (size_t)j * a.dm + i;
    const size_t stride = (size_t)kCgCols * a.dm;
#pragma unroll 8
    for (int c = w; c < nchunks; c += kRedWaves) sum += p[(size_t)c * stride];
  }
  s_part[w][lane] = sum;
  __syncthreads();
  if (w == 0 && on) {
    float tot = s_part[0][lane];
#pragma unroll
    for (int k = 1; k < kRedWaves; ++k) tot += s_part[k][lane];
    if (j < a.H)
      a.dwc[(size_t)i * a.H + j] = tot;
    else
      a.dwg[(size_t)i * a.H + (j - a.H)] = tot;
  }
}

size_t cg_partial_bytes(int64_t T, int dm) {
  return (size_t)((T + kCgChunk - 1) / kCgChunk) * kCgCols * (size_t)dm * sizeof(float);
}

hipError_t cg_fwd_dispatch(int dtype, const CgArgs& a, hipStream_t st) {
  const int per_wg = kCgWaves * kCgBlocks * 16;
  const int nblk = (int)((a.T + per_wg - 1) / per_wg);
  const size_t lds = (size_t)kCgCols * (a.dm + (dtype == 0 ? 8 : 4)) * (dtype == 0 ? 2 : 4);
  auto go = [&](auto tc) {
    using TT = typename decltype(tc)::type;
    const int per_batch = 8 * 4 * (16 / (int)sizeof(TT));  // features per batch of eight k-steps
    const int bpb = a.dm % per_batch == 0 ? a.dm / per_batch : 0;
    const dim3 grid(nblk), block(kCgWaves * kWave);
    if (bpb == 1)
      hipLaunchKernelGGL((cg_fwd_kernel<TT, 1>), grid, block, lds, st, a);
    else if (bpb == 2)
      hipLaunchKernelGGL((cg_fwd_kernel<TT, 2>), grid, block, lds, st, a);
    else if (bpb == 3)
      hipLaunchKernelGGL((cg_fwd_kernel<TT, 3>), grid, block, lds, st, a);
    else if (bpb == 4)
      hipLaunchKernelGGL((cg_fwd_kernel<TT, 4>), grid, block, lds, st, a);
    else
      hipLaunchKernelGGL((cg_fwd_kernel<TT, 0>), grid, block, lds, st, a);
  };
  if (dtype == 0)
    go(TypeTag<bf16_t>{});
  else
    go(TypeTag<float>{});
  return hipGetLastError();
}

hipError_t cg_bwd_dispatch(int dtype, const CgBwdArgs& a, hipStream_t st) {
  const int nchunks = (int)((a.T + kCgChunk - 1) / kCgChunk);
  const int nf = a.dm / 4;                             // a multiple of 16
  const int threads = (kCgThreads / nf) * nf;          // whole token sub-groups
  const size_t lds = (size_t)kCgCols * a.dm * sizeof(float);
  const int nj = (2 * a.H + 3) / 4 * 4;
  if (nchunks > 0) {  // T == 0: only the reduction, which writes zero dW
    auto go = [&](auto tc, auto jc) {
      using TT = typename decltype(tc)::type;
      hipLaunchKernelGGL((cg_bwd_kernel<TT, decltype(jc)::value>), dim3(nchunks), dim3(threads), lds, st, a);
    };
    auto by_nj = [&](auto tc) {
      if (nj == 4) go(tc, std::integral_constant<int, 4>{});
      else if (nj == 8) go(tc, std::integral_constant<int, 8>{});
      else if (nj == 12) go(tc, std::integral_constant<int, 12>{});
      else go(tc, std::integral_constant<int, 16>{});
    };
    if (dtype == 0)
      by_nj(TypeTag<bf16_t>{});
    else
      by_nj(TypeTag<float>{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int outs = 2 * a.H * a.dm;
  hipLaunchKernelGGL(cg_reduce_kernel, dim3((outs + kWave - 1) / kWave), dim3(kRedWaves * kWave), 0, st, a,
                     nchunks);
  return hipGetLastError();
}

}  // namespace ldc
