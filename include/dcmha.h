/*
 * dcmha.h — C ABI of the full DCMHA composition (dynamically composable
 * multi-head attention: attention scores and weights composed across heads)
 * on the Lightweight DC window, for AMD Instinct MI355X (gfx950).
 *
 * The layer (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
 * section "第二刀-砍层内", DCMHA paragraph) has a Compose module that transforms
 * the attention scores and the attention weights across heads, decided by the
 * input.  Read here as per-query H x H matrices applied over the head axis at
 * every (query, key) pair: CS[t] to the scores before the softmax, CW[t] to the
 * softmax weights after it (row = target head, column = source head; any real
 * values).  With A(t) = { s : max(0, t-window+1) <= s <= t and
 * doc_ids[s] == doc_ids[t] }:
 *   S_h[t,s] = scale * <Q[t,h,:], K[s,h,:]>                  s in A(t)
 *   Z_h[t,s] = sum_h' CS[t,h,h'] S_h'[t,s]
 *   P_h[t,:] = softmax over A(t) of Z_h[t,:]
 *   R_h[t,s] = sum_h' CW[t,h,h'] P_h'[t,s]
 *   O[t,h,:] = sum_{s in A(t)} R_h[t,s] * V[s,h,:]
 * With CS = I and CW[t,h,:] = G[t,h] C[t,:] this is the Lightweight DC layer of
 * ldc.h; with CS = CW = I it is windowed multi-head attention.
 *
 * Layout, ownership, stream semantics, status codes and dtypes as in ldc.h:
 *   Q, K, V, dO, O, dQ, dK, dV : [T, H, d] row-major; Q, K, V, dO in the
 *                                storage dtype, O and the gradients float32;
 *   CS, CW, dCS, dCW           : [T, H, H] float32, element (t,h,h') at
 *                                (t*H + h)*H + h';
 *   doc_ids                    : [T] int32.
 * Device pointers owned by the caller, 16-byte aligned.  Supported shapes:
 * 1 <= H <= 6 (a wave keeps every head's map of its queries in registers);
 * d in {64, 128} for LDC_BF16, d == 64 for LDC_F32; 1 <= window <= 113;
 * T >= 0 (T == 0 is a no-op); T*H*d < 2^31.  Arguments are validated before
 * any HIP call; errors return a non-zero ldc_status with no side effects.
 */
#ifndef DCMHA_H_
#define DCMHA_H_

#include <stddef.h>
#include <stdint.h>

#include "ldc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Forward pass: writes O[T,H,d] in float32.
 * saved: NULL (nothing saved) or a device buffer of at least
 *   dcmha_saved_bytes(...) bytes that receives the state dcmha_bwd reads:
 *   every head's softmax map P_h, then every head's composed map R_h, each as
 *   16-query x 128-key band blocks (2,048 4-byte words per block and head; the
 *   bf16 path stores bf16 hi and lo parts of each value). */
int dcmha_fwd(int dtype, int64_t T, int H, int d, int window, float scale,
              const void* q, const void* k, const void* v,
              const float* cs, const float* cw, const int32_t* doc_ids,
              float* o, void* saved, size_t saved_bytes, void* stream);

/* Backward pass: given dO, writes dq, dk, dv [T,H,d] and dcs, dcw [T,H,H], all
 * float32.  saved: the state dcmha_fwd wrote for these inputs, or NULL: the
 * pass then first recomputes it (the forward without O) into the front of the
 * workspace.  workspace: device scratch of at least
 * dcmha_bwd_workspace_bytes(...) bytes (with `saved` given, that size minus
 * dcmha_saved_bytes(...) rounded up to 256 is enough); contents on entry do
 * not matter.  Deterministic: equal inputs give bitwise-equal outputs. */
int dcmha_bwd(int dtype, int64_t T, int H, int d, int window, float scale,
              const void* q, const void* k, const void* v,
              const float* cs, const float* cw, const int32_t* doc_ids,
              const void* saved, size_t saved_bytes, const void* dO,
              float* dq, float* dk, float* dv, float* dcs, float* dcw,
              void* workspace, size_t workspace_bytes, void* stream);

/* The two kernels of dcmha_bwd, one at a time (for per-kernel timing):
 * dcmha_bwd_q writes dq, dcs, dcw and each head's dS band (into the
 * workspace; with saved NULL it first recomputes the saved state there);
 * dcmha_bwd_kv reads the saved R bands and the dS bands and writes dk, dv.
 * dcmha_bwd is dcmha_bwd_q then dcmha_bwd_kv with the same arguments. */
int dcmha_bwd_q(int dtype, int64_t T, int H, int d, int window, float scale,
                const void* q, const void* k, const void* v,
                const float* cs, const float* cw, const int32_t* doc_ids,
                const void* saved, size_t saved_bytes, const void* dO,
                float* dq, float* dk, float* dv, float* dcs, float* dcw,
                void* workspace, size_t workspace_bytes, void* stream);
int dcmha_bwd_kv(int dtype, int64_t T, int H, int d, int window, float scale,
                 const void* q, const void* k, const void* v,
                 const float* cs, const float* cw, const int32_t* doc_ids,
                 const void* saved, size_t saved_bytes, const void* dO,
                 float* dq, float* dk, float* dv, float* dcs, float* dcw,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the state dcmha_fwd saves (0 for T == 0 or unsupported sizes). */
size_t dcmha_saved_bytes(int dtype, int64_t T, int H, int d, int window);

/* Bytes of workspace dcmha_bwd needs, with or without saved state (0 for
 * T == 0 or unsupported sizes). */
size_t dcmha_bwd_workspace_bytes(int dtype, int64_t T, int H, int d, int window);

#ifdef __cplusplus
}
#endif

#endif /* DCMHA_H_ */
