/*
 * nsa_dense.h -- dense causal GQA attention forward, the baseline the NSA
 * selection kernel (nsa_sel.h) is measured against, and its sliding-window
 * variant (fp16 and bf16).
 *
 * Operation: the attention that selection attention replaces.  Wave issue
 * "[wave] NSA: selection attention forward kernel", section Performance
 * target, sets the selection forward's goal relative to a dense flash
 * attention at the same sequence length; this is that dense operation, with
 * the same tensors and conventions as nsa_sel_fwd and every causal key
 * visible: for every batch b, query m and head h (KV group g = h / (H/G)),
 * O[b, m, h, :] is the softmax over keys n <= m (n < N) of the scores
 * Q[b, m, h, :] . K[b, n, g, :] / sqrt(D), applied to V[b, n, g, :], and
 * LSE[b, h, m] is the natural-log log-sum-exp of those scaled scores.  It
 * equals nsa_sel_fwd with every block 0 .. m / block_size selected.  Matrix
 * products take fp16 operands and accumulate in fp32.  The FlyDSL pull
 * request "[Kernel][MI350] Add 8 wave GQA sliding-window attention kernel"
 * describes a kernel for this operation family on the same chip; it is prior
 * art, not the design used here.
 */
#ifndef NSA_DENSE_H
#define NSA_DENSE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "nsa_sel.h" /* status codes */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nsa_dense_fwd -- dense causal GQA attention forward.
 *
 * Arguments (device pointers to contiguous row-major memory owned by the
 * caller; the library allocates nothing and keeps no pointer):
 *   Q     fp16 [B, M, H, D]   queries
 *   K, V  fp16 [B, N, G, D]   keys and values, one head per group
 *   O     fp16 [B, M, H, D]   output, fully overwritten
 *   LSE   fp32 [B, H, M]      output, fully overwritten (head-major)
 *   B, M, N, H, G  batch, queries, keys, query heads, KV groups (H % G == 0)
 *   D     head dim: 64 or 128
 *   stream  HIP stream (0 = default stream)
 *
 * Behaviour: as nsa_sel_fwd -- every argument is checked on the host before
 * any HIP call (NSA_SEL_ERR_NULL, _SHAPE, _UNSUPPORTED for D not 64/128 or
 * H/G > 16, _ALIGN for Q/K/V/O not 16-byte or LSE not 4-byte aligned,
 * _RANGE, _ALIAS for outputs overlapping inputs or each other); on success
 * one kernel is queued on `stream` and NSA_SEL_OK is returned, without
 * synchronising or allocating.  Every query sees at least key 0, so no row is
 * empty.
 */
int nsa_dense_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M, int N, int H,
                  int G, int D, hipStream_t stream);

/*
 * nsa_window_fwd -- sliding-window GQA attention forward, fp16.
 *
 * Operation: the FlyDSL pull request "[Kernel][MI350] Add 8 wave GQA
 * sliding-window attention kernel" (section What it does) describes a kernel
 * for windows (LEFT, RIGHT): query i attends to the keys [i - LEFT, i + RIGHT].
 * Here query m of (b, h) attends to the keys n < N with
 * m - left <= n <= m + right; a negative bound leaves that side unbounded, so
 * (left, right) = (-1, 0) is nsa_dense_fwd and (-1, -1) full (non-causal)
 * attention.  Scores, scale, GQA mapping, O and LSE as for nsa_dense_fwd; a
 * query whose window holds no key gets O = 0 and LSE = -inf.
 *
 * Arguments and behaviour as nsa_dense_fwd (same checks and status codes;
 * NSA_SEL_ERR_RANGE also when M + N exceeds INT_MAX).  A workgroup streams
 * only the keys its queries' windows cover, so the work is proportional to
 * the window.
 */
int nsa_window_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M, int N, int H,
                   int G, int D, int left, int right, hipStream_t stream);

/*
 * nsa_window_fwd_bf16 -- nsa_window_fwd with bfloat16 Q, K, V and O (the
 * dtype of the FlyDSL kernel, section Summary: bf16 I/O).  Products take bf16
 * operands (P is rounded to bf16 for the PV product) and accumulate in fp32;
 * LSE stays fp32.
 */
int nsa_window_fwd_bf16(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M, int N,
                        int H, int G, int D, int left, int right, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_DENSE_H */
