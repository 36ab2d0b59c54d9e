// Double-buffered stage pipeline shared by the Lightweight DC kernels.
//
// A kernel walks "stages": one head of one staged tensor each, grouped in
// phases (e.g. all heads' K, then all heads' V).  Stage j of a phase computes
// from LDS buffer j%2 while the DMA of the next stage fills the other buffer.
// Buffer roles must be compile-time constants: with a runtime-selected buffer
// the compiler can no longer tell that the reads of one buffer do not alias
// the DMA into the other and serialises them.  Phases therefore run over an
// even number of stages (a trailing empty stage when H is odd), two stages
// per loop iteration, and each stage body receives its buffer index as a type.
#pragma once

#include <type_traits>

namespace ldc {

template <int B>
using Buf = std::integral_constant<int, B>;

// Loop j over [0, Hp) two stages at a time (Hp even); body(j, Buf<j%2>).
template <typename F>
__device__ __forceinline__ void for_stage_pairs(int Hp, F&& body) {
  for (int j = 0; j < Hp; j += 2) {
    body(j, Buf<0>{});
    body(j + 1, Buf<1>{});
  }
}

// The stage that follows stage j of phase `phase` in padded order, as
// (phase, head); head < 0 when nothing must be loaded now: the end of the
// pipeline, or an empty padding stage (the stage after it is then issued by
// the empty stage, whose buffer is the other one).  Callers still issue a
// zero-byte DMA in that case, so every stage has the same memory-op sequence.
struct NextStage {
  int phase, head;
};
__device__ __forceinline__ NextStage next_stage(int phase, int j, int H, int Hp, int nphases) {
  int np = phase, nj = j + 1;
  if (nj == Hp) {
    np = phase + 1;
    nj = 0;
  }
  if (np >= nphases || nj >= H) return {np, -1};
  return {np, nj};
}

// Three-buffer variant, for kernels that run one workgroup per CU: stage j
// computes from LDS buffer j%3 while the DMAs of stages j+1 and j+2 are in
// flight, so every tile gets two stages of lead instead of one.  Phases run
// over a multiple of three stages (trailing empty stages when 3 does not
// divide H); body(j, Buf<j%3>).
template <typename F>
__device__ __forceinline__ void for_stage_triples(int Hp, F&& body) {
  for (int j = 0; j < Hp; j += 3) {
    body(j, Buf<0>{});
    body(j + 1, Buf<1>{});
    body(j + 2, Buf<2>{});
  }
}

// The stage two after stage j of phase `phase`, in the padded order of
// for_stage_triples (Hp >= 3), with the conventions of next_stage.  Every
// stage issues exactly one such DMA (zero bytes when head < 0).
__device__ __forceinline__ NextStage stage_after_next(int phase, int j, int H, int Hp, int nphases) {
  int np = phase, nj = j + 2;
  if (nj >= Hp) {
    np = phase + 1;
    nj -= Hp;
  }
  if (np >= nphases || nj >= H) return {np, -1};
  return {np, nj};
}

// The next stage's DMA is issued in kIssueParts parts spread over the
// current stage: a wave that issues its whole share right after the barrier
// can wait thousands of cycles for the memory pipeline to take it while its
// SIMD partner computes alone.  Part p covers instructions
// [p*N/kIssueParts, (p+1)*N/kIssueParts) of a wave's N.
constexpr int kIssueParts = 4;

}  // namespace ldc
