/*
 * nsa_sel.h -- C ABI of the NSA selection-attention forward library for
 * AMD MI355X (gfx950).
 *
 * Operation (wave issue "[wave] NSA: selection attention forward kernel",
 * sections Operation, Algorithm and Requirements): for every batch b, query
 * position m and KV group g, the T entries of block_indices[b, m, g, :] name
 * key blocks t; each selected block contributes the keys
 * n in [t*block_size, (t+1)*block_size).  The heads of group g (the H/G query
 * heads g*H/G .. (g+1)*H/G - 1, which share the group's index row) attend to
 * those keys with the causal mask n <= m, through one softmax across all
 * selected blocks, scaled by 1/sqrt(D).  The output is the attention result
 * O_slc and, per head and query, the natural-log log-sum-exp of the scaled
 * scores LSE_slc (kept for a backward pass).  Matrix products take fp16
 * operands and accumulate in fp32.
 *
 * Index entries: an entry t counts when 0 <= t <= m / block_size and
 * t * block_size < N.  Any other value (negative padding such as -1, a block
 * after the query's own block, a block past the end) contributes nothing.
 * The selected key set is the union of the counted blocks: a block a row
 * repeats counts once, for any T and any order of the row.  A query with no
 * counted entry gets O = 0 and LSE = -inf.
 */
#ifndef NSA_SEL_H
#define NSA_SEL_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by the entry points of this library. */
enum {
    NSA_SEL_OK = 0,
    NSA_SEL_ERR_NULL = 1,        /* a pointer argument is NULL                      */
    NSA_SEL_ERR_SHAPE = 2,       /* a size < 1, or H not a multiple of G            */
    NSA_SEL_ERR_UNSUPPORTED = 3, /* D not 64/128, block_size not 32/64, H/G > 16    */
    NSA_SEL_ERR_ALIGN = 4,       /* Q/K/V/O not 16-byte aligned, idx/LSE not 4-byte */
    NSA_SEL_ERR_RANGE = 5,       /* B*M*G units or a tensor size beyond the limits  */
    NSA_SEL_ERR_ALIAS = 6,       /* an output buffer overlaps an input or the other */
    NSA_SEL_ERR_HIP = 7,         /* the HIP runtime reported an error at launch     */
    NSA_SEL_ERR_WORKSPACE = 8,   /* workspace NULL, misaligned or too small         */
    NSA_SEL_ERR_SCRATCH = 9      /* sizes need more than the fixed scratch (bwd)    */
};

/*
 * nsa_sel_fwd -- selection-attention forward pass.
 *
 * Arguments (all tensors are device pointers to contiguous row-major memory
 * owned by the caller; the library allocates nothing and keeps no pointer
 * after the call returns):
 *   Q             fp16 [B, M, H, D]   queries
 *   K, V          fp16 [B, N, G, D]   keys and values, one head per group
 *   block_indices int32 [B, M, G, T]  selected block ids per (b, m, g)
 *   O             fp16 [B, M, H, D]   output, fully overwritten
 *   LSE           fp32 [B, H, M]      output, fully overwritten (head-major)
 *   B, M, N, H, G batch, queries, keys, query heads, KV groups
 *   D             head dim: 64 or 128
 *   block_size    32 or 64
 *   T             entries per index row (>= 1)
 *   stream        HIP stream the kernel is queued on (0 = default stream)
 *
 * Behaviour: every argument is checked on the host before any HIP call; a
 * failed check returns its NSA_SEL_ERR_* code and touches nothing.  On success
 * the work is queued asynchronously on `stream` (as a short sequence of
 * kernel dispatches) and NSA_SEL_OK is returned; the call never synchronises
 * and allocates no memory.  Faults inside the kernel surface at the caller's
 * next synchronisation, as for any HIP launch.  Inputs are only read; outputs
 * must not overlap inputs or each other.  Calls on different streams may run
 * concurrently; the only global state is a per-device cache of the compute
 * unit count, filled on the first call on each device.
 */
int nsa_sel_fwd(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                int block_size, int T, hipStream_t stream);

/*
 * nsa_sel_fwd_bf16 -- nsa_sel_fwd with bfloat16 Q, K, V and O (bf16 I/O, the
 * dtype of the FlyDSL pull request "[Kernel][MI350] Add 8 wave GQA
 * sliding-window attention kernel", section Summary).  Same arguments, checks
 * and behaviour; products take bf16 operands (P is rounded to bf16 for the PV
 * product) and accumulate in fp32; LSE stays fp32.
 */
int nsa_sel_fwd_bf16(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                     void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                     int block_size, int T, hipStream_t stream);

/*
 * nsa_sel_fwd_workspace_size -- bytes of device workspace nsa_sel_fwd_ws and
 * nsa_sel_fwd_bf16_ws need for these sizes on the current device: an upper
 * bound that does not depend on the index values (on MI355X about 260 KiB
 * for one batch of 65536 queries in 8 groups, 520 KiB for 131072).
 * Sizes are checked as for nsa_sel_fwd; returns NSA_SEL_OK and stores the
 * size in *bytes, or an error code (NSA_SEL_ERR_NULL when bytes is NULL).
 * Reads the current device's compute-unit and XCD counts and L2 size (HIP
 * device attributes, cached per device); queues nothing.
 */
int nsa_sel_fwd_workspace_size(int B, int M, int N, int H, int G, int D, int block_size, int T, size_t *bytes);

/*
 * nsa_sel_fwd_ws, nsa_sel_fwd_bf16_ws -- nsa_sel_fwd and nsa_sel_fwd_bf16
 * with a workspace, which lets them run as one persistent dispatch.
 *
 * Same operation, arguments, checks and results (bitwise) as nsa_sel_fwd and
 * nsa_sel_fwd_bf16, plus:
 *   workspace, workspace_bytes  device memory of at least
 *         nsa_sel_fwd_workspace_size() bytes, 256-byte aligned, overlapping
 *         no input or output; its contents on entry do not matter (the call
 *         clears what it uses, on `stream`, with a kernel, not a memset) and
 *         are unspecified on return.
 *
 * Where one (b, g)'s K and V exceed one XCD's L2 (N * D * 4 bytes), the call
 * queues that clearing kernel and one persistent dispatch in place of one
 * dispatch per generation: the workgroups of each XCD still run one
 * generation of wavefront slots at a time, all starting together, but they
 * wait only for each other, and an XCD whose own share is done takes over
 * generations of the others.  A share that runs slower (K/V rows at some
 * address offsets are fetched more slowly) then no longer holds every XCD
 * back.  For other sizes the call does what nsa_sel_fwd does.
 *
 * NSA_SEL_ERR_WORKSPACE for a NULL, misaligned or short workspace,
 * NSA_SEL_ERR_ALIAS when it overlaps an input or an output.  Two calls that
 * share a workspace must be ordered (same stream, or synchronised).  The
 * dispatch expects its workgroups to be resident together (it launches one
 * per workgroup slot of the device): work of other streams on the same GPU
 * slows it, since its waits end only after about 0.5 ms, but does not change
 * its results.
 */
int nsa_sel_fwd_ws(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                   void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                   int block_size, int T, void *workspace, size_t workspace_bytes, hipStream_t stream);
int nsa_sel_fwd_bf16_ws(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                        void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                        int block_size, int T, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nsa_sel_fwd_unpipelined -- verification aid: nsa_sel_fwd (fp16) with the
 * copy of the next gathered block into LDS issued only after the current
 * block's math, and every block waiting for all of its copies, so no copy is
 * in flight while a wavefront reads LDS.  Same arguments, checks and
 * arithmetic in the same order: its outputs are bitwise those of nsa_sel_fwd,
 * which is how a copy that overwrote LDS still being read would show.
 * Slower; not meant for production use.
 */
int nsa_sel_fwd_unpipelined(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                            void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                            int block_size, int T, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *nsa_sel_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* NSA_SEL_H */
