/*
 * ldc_fused.h — C ABI of the Lightweight DC layer fused with the attention
 * block's main attention (forward), for AMD Instinct MI355X (gfx950).
 *
 * The AITNT page ("一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
 * section "第二刀-砍层内", Lightweight DC paragraph) says the branch reuses the
 * block's Q and K over a short local window and keeps its overhead down with a
 * dedicated kernel.  Read here as one kernel for the block's whole attention
 * output:
 *   O[t,h,:] = M[t,h,:] + G[t,h] * sum_{s in A(t)} Pbar[t,s] * V[s,h,:]
 * where
 *   run_start(t) = first token of the run of equal doc_ids holding t,
 *   M[t,h,:]     = sum_{s=run_start(t)}^{t} softmax_s(scale <Q[t,h],K[s,h]>) V[s,h,:]
 * (causal attention of each head over the query's own document), and the
 * second term is the Lightweight DC layer of ldc.h exactly (its window A(t),
 * document cut by equal ids, Pbar[t,s] = sum_h C[t,h] P_h[t,s]).
 *
 * Layout, ownership and stream semantics as in ldc.h: Q, K, V [T,H,d] bf16
 * (LDC_BF16 only), C and G [T,H] float32, doc_ids [T] int32, O [T,H,d]
 * float32 (written, never read); device pointers owned by the caller, 16-byte
 * aligned; the call only enqueues work on `stream` (NULL: the default stream)
 * and allocates nothing.  Supported: d in {64, 128}; H >= 1;
 * 1 <= window <= 128; T >= 0 (T == 0 is a no-op); T*H*d < 2^31.  Arguments are
 * validated before any HIP call; errors return a non-zero ldc_status with no
 * side effects.  The main attention's work grows with the document length
 * (every query reads its whole run).
 *
 * Workspace (device memory, 16-byte aligned, at least the size the matching
 * *_workspace_bytes call returns, contents need not be initialised, used
 * only by work enqueued by the call): the first ldc_saved_bytes(dtype, T, H,
 * d, window) bytes of the fused call's workspace receive the Lightweight DC
 * layer's saved state exactly as ldc_fwd writes it (the composed-map band
 * and the softmax statistics), so it can be passed to ldc_bwd as `saved`
 * until the next call that writes it; the rest holds every token's run start
 * and the order in which the main attention takes its 128-query tiles (most
 * key stages first, so that long documents' tiles do not trail at the end).
 * Too small or missing: LDC_ERR_WORKSPACE.
 */
#ifndef LDC_FUSED_H_
#define LDC_FUSED_H_

#include <stddef.h>
#include <stdint.h>

#include "ldc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes of ldc_fused_fwd (0 for invalid arguments or T == 0). */
size_t ldc_fused_fwd_workspace_bytes(int dtype, int64_t T, int H, int d, int window);

/* The block's attention output O = M + the Lightweight DC layer (above). */
int ldc_fused_fwd(int dtype, int64_t T, int H, int d, int window, float scale,
                  const void* q, const void* k, const void* v,
                  const float* c, const float* g, const int32_t* doc_ids,
                  float* o, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of ldc_main_attention_fwd (0 for T <= 0 or T > 2^30). */
size_t ldc_main_attention_workspace_bytes(int64_t T);

/* The main attention M alone (the same kernel without the Lightweight DC
 * terms), for comparison and as the unfused block's first half. */
int ldc_main_attention_fwd(int dtype, int64_t T, int H, int d, float scale,
                           const void* q, const void* k, const void* v,
                           const int32_t* doc_ids, float* o,
                           void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LDC_FUSED_H_ */
