/*
 * ldc_cg.h — C ABI of the generator of the Lightweight DC weights C and G for
 * AMD Instinct MI355X (gfx950).
 *
 * The AITNT page ("一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
 * section "第二刀-砍层内") says the composition is decided from the current
 * input (DCMHA paragraph) and that the heads' maps are composed dynamically,
 * each head's Value scaled by its own head scale (Lightweight DC paragraph);
 * it gives no formula.  Read here as linear projections of the layer's input
 * hidden state x (no bias, no nonlinearity):
 *   C[t,h] = sum_i x[t,i] WC[i,h]            G[t,h] = sum_i x[t,i] WG[i,h]
 * Backward, given dC and dG:
 *   dx[t,i] = sum_h dC[t,h] WC[i,h] + dG[t,h] WG[i,h]
 *   dWC[i,h] = sum_t x[t,i] dC[t,h]          dWG[i,h] = sum_t x[t,i] dG[t,h]
 *
 * Layout: x [T, dm] and WC, WG [dm, H] row-major in the storage dtype
 * (LDC_BF16 or LDC_F32); C, G, dC, dG [T, H], dx [T, dm] and dWC, dWG [dm, H]
 * float32.  Device pointers owned by the caller, 16-byte aligned.  Supported:
 * 1 <= H <= 8; dm a multiple of 64 with 64 <= dm <= 1024 (LDC_F32: <= 768);
 * T >= 0 (T == 0: the forward does nothing, the backward writes zero dWC and
 * dWG); T*dm < 2^31.  Status codes as in ldc.h,
 * validation before any HIP call.  Deterministic: dWC and dWG are summed in a
 * fixed order (within 256-token chunks, then over the chunks in a fixed
 * grouping), so equal inputs give bitwise-equal results.
 */
#ifndef LDC_CG_H_
#define LDC_CG_H_

#include <stddef.h>
#include <stdint.h>

#include "ldc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C and G from x. */
int ldc_cg_fwd(int dtype, int64_t T, int dm, int H, const void* x, const void* wc, const void* wg,
               float* c, float* g, void* stream);

/* dx, dWC, dWG from dC and dG.  workspace: device scratch of at least
 * ldc_cg_bwd_workspace_bytes(...) bytes (the per-chunk dW partials). */
int ldc_cg_bwd(int dtype, int64_t T, int dm, int H, const void* x, const void* wc, const void* wg,
               const float* dc, const float* dg, float* dx, float* dwc, float* dwg,
               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of ldc_cg_bwd (0 for unsupported sizes or T == 0). */
size_t ldc_cg_bwd_workspace_bytes(int dtype, int64_t T, int dm, int H);

#ifdef __cplusplus
}
#endif

#endif /* LDC_CG_H_ */
