// Top-k block selection for AMD MI355X (gfx950): scores [B, M, G, NB] ->
// block_indices [B, M, G, T] (include/nsa_topk.h).
//
// Operation: the top-k step the wave issue "[wave] NSA: selection attention
// forward kernel" (section Depends on) names as the producer of
// block_indices; the header states the reading taken (the pages give no
// algorithm).
//
// MI355X mapping: one wavefront per row.  Lane l holds the candidates
// t = 64*j + l (coalesced 256-byte loads per j) as order-preserving 32-bit
// keys in registers; key 0 marks "not a candidate".  A radix select finds
// the T-th largest key K bit by bit from the top (32 wave-wide counts); the
// row is then written in ascending block order with ballots: every key > K,
// and keys == K in index order until T are taken.  The work per row is a
// fixed 32 count steps whatever T is, and only the causal prefix of the row
// is read, so the kernel streams its scores at memory speed.
#include "nsa_sel_common.h"
#include "nsa_topk.h"

namespace {

// Larger score -> larger key; NaN takes the key of -inf and -0 that of +0;
// every score maps to a key >= 0x007FFFFF, leaving 0 free.
__device__ __forceinline__ unsigned score_key(float x) {
    unsigned u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;  // NaN
    if (u == 0x80000000u) u = 0u;                           // -0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
    return __builtin_amdgcn_readlane(x, 15) + __builtin_amdgcn_readlane(x, 31) +
           __builtin_amdgcn_readlane(x, 47) + __builtin_amdgcn_readlane(x, 63);
}

template <int KREG>
__global__ __launch_bounds__(256) void nsa_topk_kernel(const float *scores, int32_t *out, int rows, int M, int G,
                                                       int NB, int bs, int T) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (row >= rows) return;  // whole wavefront
    const int m = (row / G) % M;
    const int nc = min(m / bs, NB - 1) + 1;  // candidates 0 .. nc-1
    int32_t *dst = out + (size_t)row * T;
    if (nc <= T) {
        for (int i = lane; i < T; i += kWaveSize) dst[i] = i < nc ? i : -1;
        return;
    }
    const float *src = scores + (size_t)row * NB;
    unsigned key[KREG];
#pragma unroll
    for (int j = 0; j < KREG; ++j) {
        const int t = j * kWaveSize + lane;
        key[j] = t < nc ? score_key(__builtin_nontemporal_load(src + t)) : 0u;
    }
    // K = the largest value with at least T keys >= K: the T-th largest key.
    unsigned kth = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const unsigned cand = kth | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < KREG; ++j) cnt += key[j] >= cand ? 1 : 0;
        if (wave_sum(cnt) >= T) kth = cand;
    }
    int greater = 0;
#pragma unroll
    for (int j = 0; j < KREG; ++j) greater += key[j] > kth ? 1 : 0;
    int ties_left = T - wave_sum(greater);  // >= 1 keys equal to K are taken
    const uint64_t below = (1ull << lane) - 1ull;
    int pos = 0;
#pragma unroll
    for (int j = 0; j < KREG; ++j) {
        const bool eq = key[j] == kth;
        const uint64_t eqm = __ballot(eq);
        const bool take = key[j] > kth || (eq && __builtin_popcountll(eqm & below) < ties_left);
        const int n_eq = __builtin_popcountll(eqm);
        ties_left -= n_eq < ties_left ? n_eq : ties_left;
        const uint64_t tm = __ballot(take);
        if (take) dst[pos + __builtin_popcountll(tm & below)] = j * kWaveSize + lane;
        pos += __builtin_popcountll(tm);
    }
}

template <int KREG>
hipError_t launch_topk(const float *scores, int32_t *out, int rows, int M, int G, int NB, int bs, int T,
                       hipStream_t stream) {
    hipLaunchKernelGGL((nsa_topk_kernel<KREG>), dim3((rows + 3) / 4), dim3(256), 0, stream, scores, out, rows, M, G,
                       NB, bs, T);
    return hipGetLastError();
}

}  // namespace

extern "C" int nsa_topk_blocks(const float *scores, int32_t *block_indices, int B, int M, int G, int NB,
                               int block_size, int T, hipStream_t stream) {
    if (!scores || !block_indices) return NSA_SEL_ERR_NULL;
    if (B < 1 || M < 1 || G < 1 || NB < 1 || block_size < 1 || T < 1) return NSA_SEL_ERR_SHAPE;
    if (NB > 64 * kWaveSize) return NSA_SEL_ERR_UNSUPPORTED;
    if (((uintptr_t)scores | (uintptr_t)block_indices) & 3) return NSA_SEL_ERR_ALIGN;
    if ((int64_t)B * M * G > INT_MAX) return NSA_SEL_ERR_RANGE;
    const int rows = B * M * G;
    if (ranges_overlap(block_indices, (size_t)rows * T * 4, scores, (size_t)rows * NB * 4)) return NSA_SEL_ERR_ALIAS;
    hipError_t e;
    const int kreg = (NB + kWaveSize - 1) / kWaveSize;
    if (kreg <= 1)
        e = launch_topk<1>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    else if (kreg <= 2)
        e = launch_topk<2>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    else if (kreg <= 4)
        e = launch_topk<4>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    else if (kreg <= 8)
        e = launch_topk<8>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    else if (kreg <= 16)
        e = launch_topk<16>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    else if (kreg <= 32)
        e = launch_topk<32>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    else
        e = launch_topk<64>(scores, block_indices, rows, M, G, NB, block_size, T, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}
