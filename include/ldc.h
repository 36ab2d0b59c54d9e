/*
 * ldc.h — C ABI of the Lightweight DC (LDC) attention layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (AITNT page "一个国产AI小透明，连续两次刷新NanoGPT Speedrun世界纪录",
 * section "第二刀-砍层内", Lightweight DC paragraph) reuses the attention
 * block's Q and K, runs a per-head causal softmax over a local window of
 * `window` tokens (112 in the GPT-2 small speedrun model), composes the heads'
 * attention maps after the softmax into one shared map with per-token weights,
 * and lets that shared map act on each head's Value through a per-head scale.
 *
 * With A(t) = { s : max(0, t-window+1) <= s <= t and doc_ids[s] == doc_ids[t] }:
 *   S_h[t,s] = scale * <Q[t,h,:], K[s,h,:]>                 s in A(t)
 *   P_h[t,:] = softmax over A(t) of S_h[t,:]
 *   Pbar[t,s] = sum_h C[t,h] * P_h[t,s]          (C any real, not renormalised)
 *   O[t,h,:] = G[t,h] * sum_{s in A(t)} Pbar[t,s] * V[s,h,:]
 * The document cut and the use of query-indexed C and G are readings of the
 * page, which leaves them open.
 *
 * Layout (all entry points): tokens are a flattened stream of T rows;
 *   Q, K, V, dO, O, dQ, dK, dV : [T, H, d] row-major, element (t,h,j) at
 *                                ((t*H)+h)*d + j;  Q, K, V, dO in the storage
 *                                dtype, O and the gradients float32;
 *   C, G, dC, dG               : [T, H] float32 row-major;
 *   doc_ids                    : [T] int32, any values (only equality matters).
 * Pointers are DEVICE pointers owned by the caller; base addresses must be
 * 16-byte aligned.  Supported shapes: d in {16, 64, 128} for both dtypes;
 * 1 <= window <= 128 (LDC_F32 with d = 128:
 * up to 113, else LDC_ERR_UNSUPPORTED); H >= 1; T >= 0 (T == 0 is a no-op);
 * T*H*d < 2^31.
 *
 * Execution: work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns without synchronising.  The library allocates
 * no device memory; apart from the static scratch of ldc_bwd_noalloc it keeps
 * no global state, and every other entry point is reentrant.  Outputs are
 * fully overwritten (no accumulate mode).
 *
 * Errors: arguments are validated before any HIP call; a validation failure
 * returns a non-zero ldc_status and has no side effects.  A failed kernel
 * launch returns LDC_ERR_HIP.  Faults during execution surface at the caller's
 * next synchronisation.
 */
#ifndef LDC_H_
#define LDC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LDC_OK = 0,
  LDC_ERR_NULL = 1,        /* a required pointer is NULL                    */
  LDC_ERR_SHAPE = 2,       /* T<0, H<1, window or scale out of range, overflow */
  LDC_ERR_DTYPE = 3,       /* dtype is not an ldc_dtype value               */
  LDC_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned              */
  LDC_ERR_UNSUPPORTED = 5, /* head dim (or window) not available for dtype  */
  LDC_ERR_WORKSPACE = 6,   /* saved state / workspace missing or too small  */
  LDC_ERR_HIP = 7,         /* a HIP launch failed                           */
  LDC_ERR_SCRATCH = 8      /* ldc_bwd_noalloc: problem exceeds its scratch  */
} ldc_status;

typedef enum {
  LDC_BF16 = 0, /* Q, K, V, dO stored as bfloat16; fp32 accumulation  */
  LDC_F32 = 1   /* Q, K, V, dO stored as float32                      */
} ldc_dtype;

/* Forward pass: writes O[T,H,d] in float32.
 * q, k, v: [T,H,d] in `dtype`; c, g: [T,H] float32; doc_ids: [T] int32.
 * scale: the softmax scale, positive and finite (1/sqrt(d) for the
 *   textbook choice); other values return LDC_ERR_SHAPE.
 * saved: NULL (inference: nothing saved) or a device buffer of at least
 *   ldc_saved_bytes(...) bytes (16-byte aligned) that receives the state
 *   ldc_bwd needs: the shared map Pbar over each 16-query block's key band
 *   (NB blocks of 16 keys, NB = 8 for windows up to 113 and 10 above: NB*256
 *   words per 16-query block; bf16 path: bf16 hi and lo parts) followed by
 *   each head's softmax statistics [T,H] (row max in log2 units, 1/row sum).
 * O is float32 for both storage dtypes: a bf16 store alone would round
 * outputs of magnitude above ~5 by more than 2e-2. */
int ldc_fwd(int dtype, int64_t T, int H, int d, int window, float scale,
            const void* q, const void* k, const void* v,
            const float* c, const float* g, const int32_t* doc_ids,
            float* o, void* saved, size_t saved_bytes, void* stream);

/* Backward pass: given dO, writes every gradient of the forward above in
 * float32: dq, dk, dv [T,H,d] and dc, dg [T,H].  Same inputs as ldc_fwd, plus:
 * saved: the state ldc_fwd wrote for these inputs (saved_bytes at least
 *   ldc_saved_bytes(...)), or NULL: the pass then recomputes the shared map and
 *   the softmax statistics from Q, K, C (the forward's score phase) into the
 *   workspace first.
 * workspace: device scratch, 16-byte aligned, owned by the caller.
 *   ldc_bwd_workspace_bytes(...) bytes cover both cases; with `saved` given,
 *   that size minus ldc_saved_bytes(...) rounded up to a multiple of 256 is
 *   enough.  Its contents on entry do not matter and are undefined on return;
 *   too small a workspace returns LDC_ERR_WORKSPACE.
 * The pass is deterministic: equal inputs give bitwise-equal outputs, with or
 * without `saved` (the recomputed state equals the saved one bit for bit). */
int ldc_bwd(int dtype, int64_t T, int H, int d, int window, float scale,
            const void* q, const void* k, const void* v,
            const float* c, const float* g, const int32_t* doc_ids,
            const void* saved, size_t saved_bytes, const void* dO,
            float* dq, float* dk, float* dv, float* dc, float* dg,
            void* workspace, size_t workspace_bytes, void* stream);

/* The two kernels of ldc_bwd, callable one at a time (for per-kernel timing).
 * ldc_bwd is exactly ldc_bwd_q followed by ldc_bwd_kv with the same
 * arguments on the same stream:
 *   ldc_bwd_q  writes dq, dc, dg and dPbar (into the workspace); with saved
 *              NULL it first recomputes the saved state into the workspace;
 *   ldc_bwd_kv reads dc and the workspace (and the saved state, or with saved
 *              NULL the state ldc_bwd_q recomputed there) and writes dk, dv.
 * Arguments, validation and errors as for ldc_bwd; pointers the kernel does
 * not touch are still validated. */
int ldc_bwd_q(int dtype, int64_t T, int H, int d, int window, float scale,
              const void* q, const void* k, const void* v,
              const float* c, const float* g, const int32_t* doc_ids,
              const void* saved, size_t saved_bytes, const void* dO,
              float* dq, float* dk, float* dv, float* dc, float* dg,
              void* workspace, size_t workspace_bytes, void* stream);
int ldc_bwd_kv(int dtype, int64_t T, int H, int d, int window, float scale,
               const void* q, const void* k, const void* v,
               const float* c, const float* g, const int32_t* doc_ids,
               const void* saved, size_t saved_bytes, const void* dO,
               float* dq, float* dk, float* dv, float* dc, float* dg,
               void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ldc_bwd
 * without the workspace arguments.  Its workspace is a static device array of
 * ldc_bwd_noalloc_max_workspace() bytes (64 MiB) per GPU, part of the loaded
 * library and held until the process ends; the first call on a GPU looks up
 * that GPU's copy (a HIP call that allocates nothing).  The GPU is the one
 * `stream` belongs to.  Nothing in it must start at zero: each call writes
 * every word it later reads.
 * Other arguments, validation, errors and results as for ldc_bwd (results are
 * bitwise equal to ldc_bwd's on the same inputs).  A call whose workspace
 * (ldc_bwd_workspace_bytes minus the room for saved state when `saved` is
 * given, as for ldc_bwd) exceeds the scratch returns LDC_ERR_SCRATCH: with
 * saved state that allows T up to 131,072 tokens; without, about
 * 64 MiB / (1,024 + 8*H) bytes per token.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (concurrent streams, or host threads) race and give undefined results;
 * serialise them on one stream. */
int ldc_bwd_noalloc(int dtype, int64_t T, int H, int d, int window, float scale,
                    const void* q, const void* k, const void* v,
                    const float* c, const float* g, const int32_t* doc_ids,
                    const void* saved, size_t saved_bytes, const void* dO,
                    float* dq, float* dk, float* dv, float* dc, float* dg, void* stream);

/* Size in bytes of ldc_bwd_noalloc's static scratch (per GPU). */
size_t ldc_bwd_noalloc_max_workspace(void);

/* Bytes of the state ldc_fwd saves for ldc_bwd (0 for T == 0). */
size_t ldc_saved_bytes(int dtype, int64_t T, int H, int d, int window);

/* Bytes of workspace ldc_bwd needs for these sizes, with or without saved
 * state (0 for T == 0 or unsupported sizes). */
size_t ldc_bwd_workspace_bytes(int dtype, int64_t T, int H, int d, int window);

/* Human-readable name of a status code (static storage). */
const char* ldc_status_str(int status);

/* ABI version: major*10000 + minor*100 + patch. */
int ldc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LDC_H_ */
