/*
 * mudd.h — C ABI of multiway dynamic dense (MUDD) layer mixing for AMD
 * Instinct MI355X (gfx950).  Built into the same library as ldc.h and using
 * its status and dtype codes.
 *
 * The mix (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
 * section "第一刀—砍层间", and the MUDD remarks of section "和业界其他工作的
 * 联系"): the input a layer receives is, per token, a weighted sum of the
 * outputs of earlier layers, with weights generated from the current hidden
 * state that are not softmax-normalised and may be negative.  The full method
 * keeps four such mixes ("ways": the Q, K, V and residual inputs); the
 * skip-connection variant keeps one.  For J streams X_j, W ways and weights
 * A[t, w, j]:
 *   Y_w[t, :]   = sum_j A[t, w, j] * X_j[t, :]                (forward)
 *   dX_j[t, :]  = sum_w A[t, w, j] * dY_w[t, :]               (backward)
 *   dA[t, w, j] = <dY_w[t, :], X_j[t, :]>
 * The weights are inputs: the page does not give the generator's form, so it
 * stays upstream of this library.
 *
 * Layout: X_j, dY_w: [T, dm] row-major in the storage dtype (LDC_BF16 or
 * LDC_F32); Y_w, dX_j: [T, dm] float32; A, dA: [T, W, J] float32, element
 * (t, w, j) at (t*W + w)*J + j.  `xs`, `ys`, `dys`, `dxs` are HOST arrays of J
 * (or W) DEVICE pointers; every device pointer is owned by the caller, must be
 * 16-byte aligned and must not alias an output.  Supported shapes: T >= 0
 * (T == 0 is a no-op), 1 <= J <= MUDD_MAX_STREAMS, 1 <= W <= MUDD_MAX_WAYS,
 * 4 <= dm <= MUDD_MAX_DIM with dm % 4 == 0, T*dm < 2^40.
 *
 * Execution: enqueued on `stream` (a hipStream_t; NULL = the default stream),
 * returns without synchronising; no allocation, no global state, reentrant;
 * outputs are fully overwritten.  Each output element is an fp32 sum of fp32
 * products of the stored values.
 *
 * Errors: arguments are validated before any HIP call (LDC_ERR_NULL,
 * LDC_ERR_SHAPE, LDC_ERR_DTYPE, LDC_ERR_ALIGN; no side effects); a failed
 * launch returns LDC_ERR_HIP.
 */
#ifndef MUDD_H_
#define MUDD_H_

#include <stddef.h>
#include <stdint.h>

#include "ldc.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MUDD_MAX_STREAMS 16
#define MUDD_MAX_WAYS 4
#define MUDD_MAX_DIM 16384

/* Forward: ys[w] <- Y_w for w < W. */
int mudd_fwd(int dtype, int64_t T, int dm, int W, int J,
             const void* const* xs, const float* a, float* const* ys, void* stream);

/* Backward: dxs[j] <- dX_j for j < J and da <- dA, given dys[w] = dL/dY_w in
 * the storage dtype. */
int mudd_bwd(int dtype, int64_t T, int dm, int W, int J,
             const void* const* xs, const float* a, const void* const* dys,
             float* const* dxs, float* da, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUDD_H_ */
