/*
 * nsa_gather_probe.h -- C ABI of the gather-ceiling probe that accompanies
 * the NSA selection-attention forward library (nsa_sel.h).
 *
 * What it measures (wave issue "[wave] NSA: selection attention forward
 * kernel", sections Algorithm and "MI350 considerations": gathering the
 * selected, irregular K/V blocks is the performance-critical part): the probe
 * replays the forward kernel's block-gather stream and nothing else.  For the
 * same arguments it launches the same workgroups and generations, merges the
 * same index rows into the same ascending block sequence per wavefront slot,
 * copies every merged K and V block into LDS with the same direct-to-LDS
 * loads and waits, and reads the staged fragments back with the same LDS
 * instructions.  It computes no scores, no softmax and no output, and it does
 * not read Q.  Its duration is therefore the time the forward kernel's
 * memory traffic needs on its own: the forward kernel's distance from it is
 * the cost of the math that the copies do not hide.
 *
 * It is a measurement aid, not part of the attention operation.
 */
#ifndef NSA_GATHER_PROBE_H
#define NSA_GATHER_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "nsa_sel.h" /* status codes */

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nsa_gather_probe -- stream the forward kernel's block gathers.
 *
 * Arguments:
 *   K, V          fp16 [B, N, G, D] device pointers, as for nsa_sel_fwd
 *   block_indices int32 [B, M, G, T] device pointer, as for nsa_sel_fwd
 *   staged        device pointer to one uint64 counter; the probe adds the
 *                 number of blocks it stages (summed over wavefront slots)
 *                 to it.  The caller zeroes it first.
 *   B, M, N, H, G, D, block_size, T   as for nsa_sel_fwd (H sets how many
 *                 queries share a wavefront slot, as it does there)
 *   workspace, workspace_bytes  NULL and 0: the launches of nsa_sel_fwd;
 *                 otherwise a workspace as nsa_sel_fwd_ws takes (at least
 *                 nsa_sel_fwd_workspace_size() bytes, 256-byte aligned): the
 *                 launches of nsa_sel_fwd_ws
 *   queries_per_slot  host pointer or NULL; receives the number of
 *                 consecutive queries of one (b, g) that each wavefront slot
 *                 carries (slots start at m = 0, that many apart)
 *   stream        HIP stream (0 = default stream)
 *
 * Behaviour: the checks of nsa_sel_fwd apply (NULL pointers, sizes,
 * supported D / block_size / H/G, alignment: K and V 16 bytes, block_indices
 * 4 bytes, staged 8 bytes; a misaligned or short workspace is
 * NSA_SEL_ERR_WORKSPACE), all on the host before any HIP call, with the
 * same status codes.  On success the work is queued on `stream` and
 * NSA_SEL_OK is returned; nothing is allocated and nothing synchronises.
 * Inputs are only read.
 */
int nsa_gather_probe(const void *K, const void *V, const int32_t *block_indices, uint64_t *staged, int B,
                     int M, int N, int H, int G, int D, int block_size, int T, void *workspace,
                     size_t workspace_bytes, int *queries_per_slot, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_GATHER_PROBE_H */
