/*
 * nsa_topk.h -- top-k block selection, the producer of the block_indices that
 * nsa_sel_fwd (nsa_sel.h) consumes.
 *
 * Operation: the wave issue "[wave] NSA: selection attention forward kernel",
 * section Depends on, takes block_indices from a top-k kernel and gives no
 * algorithm for it.  Plain reading: every row (b, m, g) holds one importance
 * score per key block; the candidates are the blocks query m may select,
 * t = 0 .. min(m / block_size, NB - 1); the T candidates with the highest
 * scores are chosen (ties to the smaller block index; a NaN score counts as
 * -inf and -0 as +0) and written in ascending block order, padded with -1
 * when the row has fewer than T candidates.  How the scores are computed (in
 * NSA, from the compressed-attention branch, summed over the group's heads)
 * is the caller's; a block the caller wants always selected can be given the
 * score +inf.
 */
#ifndef NSA_TOPK_H
#define NSA_TOPK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "nsa_sel.h" /* status codes */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nsa_topk_blocks -- top-k block selection.
 *
 * Arguments (device pointers to contiguous row-major memory owned by the
 * caller; the library allocates nothing and keeps no pointer):
 *   scores         fp32 [B, M, G, NB]   block scores per (b, m, g); only the
 *                  candidates t <= min(m / block_size, NB - 1) are read
 *   block_indices  int32 [B, M, G, T]   output, fully overwritten
 *   B, M, G        batch, queries, KV groups
 *   NB             key blocks per row (ceil(N / block_size)), 1 .. 4096
 *   block_size     keys per block (>= 1)
 *   T              entries per output row (>= 1)
 *   stream         HIP stream (0 = default stream)
 *
 * Behaviour: every argument is checked on the host before any HIP call:
 * NSA_SEL_ERR_NULL, NSA_SEL_ERR_SHAPE (a size < 1), NSA_SEL_ERR_UNSUPPORTED
 * (NB > 4096), NSA_SEL_ERR_ALIGN (a pointer not 4-byte aligned),
 * NSA_SEL_ERR_RANGE (B * M * G beyond INT_MAX), NSA_SEL_ERR_ALIAS (the output
 * overlaps the scores).  On success one kernel is queued on `stream` and
 * NSA_SEL_OK is returned, without synchronising.  The result is exact (no
 * floating-point arithmetic on the scores: they are compared as ordered
 * 32-bit keys) and equals the plain definition above bit for bit.
 */
int nsa_topk_blocks(const float *scores, int32_t *block_indices, int B, int M, int G, int NB, int block_size, int T,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_TOPK_H */
