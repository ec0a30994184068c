/*
 * nsa_sel_bwd.h -- C ABI of the NSA selection-attention backward pass.
 *
 * Operation: the gradients of the selection attention of nsa_sel_fwd
 * (nsa_sel.h).  Wave issue "[wave] NSA: selection attention forward kernel",
 * section Requirements, gives the backward pass as the reason the forward
 * returns LSE: with it the probabilities can be recomputed without a second
 * softmax pass.  For each (b, m, h) whose group g = h / (H/G) selects the key
 * set S(b, m, g) (the union of the counted blocks of the index row, keys
 * n <= m, n < N, exactly as in the forward), with scores
 * s_n = Q[b,m,h,:] . K[b,n,g,:] / sqrt(D) and P_n = exp(s_n - LSE[b,h,m]):
 *
 *   dP_n  = dO[b,m,h,:] . V[b,n,g,:]
 *   Delta = dO[b,m,h,:] . O[b,m,h,:]          (= sum_n P_n dP_n)
 *   dS_n  = P_n (dP_n - Delta)
 *   dQ[b,m,h,:]  = sum_{n in S} dS_n K[b,n,g,:] / sqrt(D)
 *   dK[b,n,g,:]  = sum over (m, h) whose set holds n of dS_n Q[b,m,h,:] / sqrt(D)
 *   dV[b,n,g,:]  = sum over (m, h) whose set holds n of P_n dO[b,m,h,:]
 *
 * Keys no query selects get dK = dV = 0; a query with an empty set gets
 * dQ = 0.  Matrix products take fp16 operands (P and dS are rounded to fp16
 * for the products that consume them) and accumulate in fp32; the gradients
 * are written in fp32.  Results are deterministic: no floating-point atomics
 * are used, and partial sums are added in a fixed order.
 */
#ifndef NSA_SEL_BWD_H
#define NSA_SEL_BWD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "nsa_sel.h" /* status codes */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nsa_sel_bwd_workspace_size -- bytes of device workspace nsa_sel_bwd needs
 * for these sizes on the current device (an upper bound that does not depend
 * on the index values).  It holds the inverted index and partial sums of the
 * key-major pass and the schedule of the query-major dQ pass, which runs as
 * one persistent dispatch (as nsa_sel_fwd_ws does) when one group's K and V
 * exceed the L2 of one XCD.  Sizes are checked as for nsa_sel_fwd; returns
 * NSA_SEL_OK and stores the size in *bytes, or an error code
 * (NSA_SEL_ERR_NULL when bytes is NULL).  Reads the current device's
 * compute-unit and XCD counts and L2 size (HIP device attributes, cached per
 * device); queues nothing.
 */
int nsa_sel_bwd_workspace_size(int B, int M, int N, int H, int G, int D, int block_size, int T, size_t *bytes);

/*
 * nsa_sel_bwd -- selection-attention backward pass.
 *
 * Arguments (device pointers to contiguous row-major memory owned by the
 * caller; the library allocates nothing and keeps no pointer):
 *   Q, K, V, block_indices   the forward's inputs (layouts as nsa_sel_fwd)
 *   O     fp16 [B, M, H, D]  the forward's output
 *   LSE   fp32 [B, H, M]     the forward's log-sum-exp
 *   dO    fp16 [B, M, H, D]  gradient of the loss with respect to O
 *   dQ    fp32 [B, M, H, D]  output, fully overwritten
 *   dK    fp32 [B, N, G, D]  output, fully overwritten
 *   dV    fp32 [B, N, G, D]  output, fully overwritten
 *   workspace, workspace_bytes  device scratch of at least
 *         nsa_sel_bwd_workspace_size() bytes, 256-byte aligned; its contents
 *         on entry do not matter.  Once the queued work has completed, the
 *         32-bit word at byte offset 4 of the workspace is 0; a nonzero value
 *         means an internal capacity bound of the key-major pass was exceeded
 *         and dK/dV are incomplete (the bounds are derived from the sizes, so
 *         this is a guard, not an expected outcome).  The rest of the
 *         workspace is unspecified on return
 *   B, M, N, H, G, D, block_size, T, stream   as for nsa_sel_fwd
 *
 * Behaviour: every argument is checked on the host before any work is queued, with
 * the forward's status codes (Q/K/V/O/dO and dQ/dK/dV must be 16-byte
 * aligned, block_indices and LSE 4-byte aligned; outputs and workspace may
 * not overlap the inputs or each other; NSA_SEL_ERR_WORKSPACE for a NULL,
 * misaligned or short workspace; NSA_SEL_ERR_RANGE also when one batch of Q
 * exceeds 2^32 - 1 bytes).  On success a short sequence of kernels is queued on
 * `stream` and NSA_SEL_OK is returned, without synchronising.  Two calls that
 * share a workspace must be ordered (same stream, or synchronised).
 */
int nsa_sel_bwd(const void *Q, const void *K, const void *V, const int32_t *block_indices, const void *O,
                const float *LSE, const void *dO, float *dQ, float *dK, float *dV, void *workspace,
                size_t workspace_bytes, int B, int M, int N, int H, int G, int D, int block_size, int T,
                hipStream_t stream);

/*
 * nsa_sel_bwd_noalloc -- nsa_sel_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments (minus workspace and workspace_bytes), checks,
 * status codes and results as nsa_sel_bwd: the two are bitwise equal.  The
 * workspace is a 64 MiB array inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call allocates nothing
 * and calls no allocating routine.  Sizes whose workspace
 * (nsa_sel_bwd_workspace_size) exceeds 64 MiB return NSA_SEL_ERR_SCRATCH
 * before any work is queued (for example the 8192-query shape with 32 heads in 2
 * groups, D = 128, block_size 64, T = 16 fits; a 64k-query shape does not).
 * Every call on a GPU shares that GPU's array and leaves its last contents
 * there: calls that may overlap on one GPU (different streams, or threads
 * without ordering) race and must be serialised by the caller.
 */
int nsa_sel_bwd_noalloc(const void *Q, const void *K, const void *V, const int32_t *block_indices, const void *O,
                        const float *LSE, const void *dO, float *dQ, float *dK, float *dV, int B, int M, int N,
                        int H, int G, int D, int block_size, int T, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_SEL_BWD_H */
