// Top-k block selection for AMD MI355X (gfx950): scores [B, M, G, NB] ->
// block_indices [B, M, G, T] (include/nsa_topk.h).
//
// Operation: the top-k step the wave issue "[wave] NSA: selection attention
// forward kernel" (section Depends on) names as the producer of
// block_indices; the header states the reading taken (the pages give no
// algorithm).
//
// MI355X mapping: one wavefront per row, four consecutive rows per wavefront,
// the next row's scores loading while the current one is selected.  Lane l
// holds the candidates t = 64*j + l (coalesced 256-byte loads per j) as
// order-preserving 32-bit keys in registers; key 0 marks "not a candidate".
// The selection code is instantiated per number of registers that hold
// candidates (a size bucket chosen once per row), so rows shorter than the
// longest cost only their own registers.
//
// A radix select finds the threshold bit by bit from the top: the count of
// keys at or above a candidate prefix is one v_cmp per register with its
// ballot popcounted on the scalar unit for even registers and on the VALU
// for odd ones (no cross-lane arithmetic).  As soon as at most 64 keys lie at or above the accepted prefix
// (for random scores, after the sign, the exponent and a mantissa bit or
// two), they are compacted through LDS into one register in ascending block
// order, and the remaining bits cost one compare each.  The search stops when
// exactly T keys lie at or above the prefix (they are the answer); keys tied
// at the T-th place run it to all 32 bits, which yields the T-th largest key
// itself.  The row is written in ascending block order with ballots: every
// key above the threshold, then keys equal to it in index order until T are
// taken.
#include "nsa_sel_common.h"
#include "nsa_topk.h"

namespace {

// Consecutive rows per wavefront (measured: 4 beats 8, 16 and 32, and loading
// two rows ahead beats none of them).
constexpr int kRowsPerWave = 4;

// Larger score -> larger key; NaN takes the key of -inf and -0 that of +0;
// every score maps to a key >= 0x007FFFFF, leaving 0 free.
__device__ __forceinline__ unsigned score_key(unsigned u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;  // NaN
    if (u == 0x80000000u) u = 0u;                           // -0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int ballot_count(bool p) { return __builtin_popcountll(__ballot(p)); }

// Candidates of the row whose first candidate is src: 0 .. nc-1 (nc wave-uniform).
template <int KREG>
__device__ __forceinline__ void load_row(const float *src, int nc, int lane, unsigned (&raw)[KREG]) {
    const unsigned *s = reinterpret_cast<const unsigned *>(src);
#pragma unroll
    for (int j = 0; j < KREG; ++j) {
        const int t = j * kWaveSize + lane;
        if (j * kWaveSize < nc && t < nc) raw[j] = __builtin_nontemporal_load(s + t);
    }
}

// The number of keys >= cand in registers 0 .. NJ-1.  The compare masks of
// even registers are popcounted on the scalar unit, those of odd registers on
// the VALU (v_bcnt_u32_b32 reading the mask from scalar registers): the CU
// has one scalar ALU for its four SIMDs, and with every count there it was
// ~93% busy (SQ counters) while the VALU had room.  The s_nop gives the two
// wait states gfx950 needs between a VALU write of an SGPR (the compare) and
// a VALU read of it; the compiler cannot insert them for inline assembly, and
// without them the counts came out wrong.
template <int NJ, int KREG>
__device__ __forceinline__ int count_ge(const unsigned (&key)[KREG], unsigned cand) {
    int cs = 0;
    unsigned cv = 0u;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const uint64_t m = __ballot(key[j] >= cand);
        if (j & 1) {
            asm("s_nop 1\n\tv_bcnt_u32_b32 %0, %1, %2" : "=v"(cv) : "s"((unsigned)m), "v"(cv));
            asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(cv) : "s"((unsigned)(m >> 32)), "v"(cv));
        } else {
            cs += __builtin_popcountll(m);
        }
        if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    if (NJ > 1) cs += (int)__builtin_amdgcn_readfirstlane(cv);
    return cs;
}

// Lane-prefix popcount: the number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

// Writes the T largest of the keys held in registers 0 .. NJ-1 (one key per
// lane and register, block index 64*j + lane; key 0 for "no candidate"),
// given kth, the T-th largest key or a prefix with exactly T keys at or above
// it: every key above kth, then keys equal to kth in index order until T are
// taken, compacted in ascending block order.
template <int NJ>
__device__ __forceinline__ void write_selection(const unsigned (&key)[NJ], const int (&idx)[NJ], unsigned kth,
                                                int T, int32_t *dst) {
    int greater = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        greater += ballot_count(key[j] > kth);
        if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    int ties_left = T - greater;  // >= 1 keys equal to kth are taken
    // An opaque copy of kth keeps the compiler from reusing the counting
    // compares above, which would hold every register's compare mask in
    // scalar registers until here.
    unsigned thr = kth;
    asm volatile("" : "+v"(thr));
    int pos = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool eq = key[j] == thr;
        const uint64_t eqm = __ballot(eq);
        const bool take = key[j] > thr || (eq && lanes_below(eqm) < ties_left);
        const int n_eq = __builtin_popcountll(eqm);
        ties_left -= n_eq < ties_left ? n_eq : ties_left;
        const uint64_t tm = __ballot(take);
        if (take) dst[pos + lanes_below(tm)] = idx[j];
        pos += __builtin_popcountll(tm);
        if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
}

// Selects the row's T largest keys among registers 0 .. NJ-1 (the later ones
// hold no candidate) and writes their block indices in ascending order.
// `sh` is this wavefront's 128-word LDS scratch.
template <int NJ, int KREG>
__device__ __forceinline__ void select_row(const unsigned (&keyr)[KREG], int T, int lane, int32_t *dst,
                                           unsigned *sh) {
    unsigned key[NJ];
    int idx[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        key[j] = keyr[j];
        idx[j] = j * kWaveSize + lane;
    }
    // kth: the largest prefix with at least T keys >= kth, found bit by bit
    // from the top; cnt = the number of keys >= kth.
    unsigned kth = 0;
    int cnt = 0x7FFFFFFF;
    int bit = 31;
    for (; bit >= 0; --bit) {
        const unsigned cand = kth | (1u << bit);
        const int c = count_ge<NJ>(key, cand);
        if (c >= T) {
            kth = cand;
            cnt = c;
            if (c <= kWaveSize || c == T) break;  // they fit one register, or are the answer
        }
    }
    if (NJ == 1 || cnt > kWaveSize) {
        // Done on the registers themselves: exactly T > 64 keys are >= kth,
        // or the search ran through all 32 bits (more than 64 keys tie at
        // the T-th place), or the row fits one register anyway.
        if (NJ == 1) {
            for (--bit; bit >= 0 && cnt != T; --bit) {
                const unsigned cand = kth | (1u << bit);
                const int c = ballot_count(key[0] >= cand);
                if (c >= T) {
                    kth = cand;
                    cnt = c;
                }
            }
        }
        write_selection<NJ>(key, idx, kth, T, dst);
        return;
    }
    // Compact the cnt <= 64 keys >= kth (with their block indices) into one
    // register, in ascending block order: the later bits and the write-out
    // touch that register only.  Keys below kth can no longer be selected.
    int base = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool keep = key[j] >= kth;
        const uint64_t km = __ballot(keep);
        if (keep) {
            const int p = base + lanes_below(km);
            sh[p] = key[j];
            sh[kWaveSize + p] = (unsigned)idx[j];
        }
        base += __builtin_popcountll(km);
        if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the scattered words are in LDS
    __builtin_amdgcn_wave_barrier();
    unsigned k1[1];
    int i1[1];
    k1[0] = lane < cnt ? sh[lane] : 0u;
    i1[0] = (int)sh[kWaveSize + lane];
    __builtin_amdgcn_wave_barrier();  // the next row's compaction comes after these reads
    for (--bit; bit >= 0 && cnt != T; --bit) {
        const unsigned cand = kth | (1u << bit);
        const int c = ballot_count(k1[0] >= cand);
        if (c >= T) {
            kth = cand;
            cnt = c;
        }
    }
    write_selection<1>(k1, i1, kth, T, dst);
}

// Dispatch on the number of registers that hold candidates (wave-uniform),
// rounded up to a size bucket no larger than KREG.
template <int KREG>
__device__ __forceinline__ void select_any(const unsigned (&key)[KREG], int nc, int T, int lane, int32_t *dst,
                                           unsigned *sh) {
    const int nj = (nc + kWaveSize - 1) / kWaveSize;
    if (KREG <= 2 || nj <= 2) { select_row<(KREG < 2 ? KREG : 2)>(key, T, lane, dst, sh); return; }
    if (KREG <= 4 || nj <= 4) { select_row<(KREG < 4 ? KREG : 4)>(key, T, lane, dst, sh); return; }
    if (KREG <= 6 || nj <= 6) { select_row<(KREG < 6 ? KREG : 6)>(key, T, lane, dst, sh); return; }
    if (KREG <= 8 || nj <= 8) { select_row<(KREG < 8 ? KREG : 8)>(key, T, lane, dst, sh); return; }
    if (KREG <= 12 || nj <= 12) { select_row<(KREG < 12 ? KREG : 12)>(key, T, lane, dst, sh); return; }
    if (KREG <= 16 || nj <= 16) { select_row<(KREG < 16 ? KREG : 16)>(key, T, lane, dst, sh); return; }
    if (KREG <= 24 || nj <= 24) { select_row<(KREG < 24 ? KREG : 24)>(key, T, lane, dst, sh); return; }
    if (KREG <= 32 || nj <= 32) { select_row<(KREG < 32 ? KREG : 32)>(key, T, lane, dst, sh); return; }
    if (KREG <= 48 || nj <= 48) { select_row<(KREG < 48 ? KREG : 48)>(key, T, lane, dst, sh); return; }
    select_row<KREG>(key, T, lane, dst, sh);
}

template <int KREG>
__global__ __launch_bounds__(256) void nsa_topk_kernel(const float *scores, int32_t *out, int rows, int M, int G,
                                                       int NB, int bs, int T) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int r0 = __builtin_amdgcn_readfirstlane((blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * kRowsPerWave);
    if (r0 >= rows) return;  // whole wavefront
    const int r1 = min(rows, r0 + kRowsPerWave);
    __shared__ unsigned lds[4][2 * kWaveSize];
    unsigned *sh = lds[threadIdx.x >> 6];
    auto cands = [&](int row) { return min(((row / G) % M) / bs, NB - 1) + 1; };  // candidates 0 .. nc-1
    unsigned raw[KREG] = {};
    int nc_next = cands(r0);
    if (nc_next > T) load_row<KREG>(scores + (size_t)r0 * NB, nc_next, lane, raw);
    for (int row = r0; row < r1; ++row) {
        const int nc = nc_next;
        int32_t *dst = out + (size_t)row * T;
        unsigned key[KREG];
        if (nc > T) {
            // A per-lane select on every register measured faster than
            // skipping the registers past the prefix with scalar branches.
#pragma unroll
            for (int j = 0; j < KREG; ++j) key[j] = (j * kWaveSize + lane < nc) ? score_key(raw[j]) : 0u;
        }
        if (row + 1 < r1) {  // the next row's scores load during this row's selection
            nc_next = cands(row + 1);
            if (nc_next > T) load_row<KREG>(scores + (size_t)(row + 1) * NB, nc_next, lane, raw);
        }
        if (nc <= T) {
            for (int i = lane; i < T; i += kWaveSize) dst[i] = i < nc ? i : -1;
        } else {
            select_any<KREG>(key, nc, T, lane, dst, sh);
        }
    }
}

template <int KREG>
hipError_t launch_topk(const float *scores, int32_t *out, int rows, int M, int G, int NB, int bs, int T,
                       hipStream_t stream) {
    const int waves = (rows + kRowsPerWave - 1) / kRowsPerWave;
    hipLaunchKernelGGL((nsa_topk_kernel<KREG>), dim3((waves + 3) / 4), dim3(256), 0, stream, scores, out, rows, M,
                       G, NB, bs, T);
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
