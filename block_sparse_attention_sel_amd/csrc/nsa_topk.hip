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
// ballot popcounted on the scalar unit (no cross-lane arithmetic).  As soon
// as at most 64 keys lie at or above the accepted prefix
// (for random scores, after the sign, the exponent and a mantissa bit or
// two), they are compacted through LDS into one register in ascending block
// order, and the remaining bits cost one compare each.  The search stops when
// exactly T keys lie at or above the prefix (they are the answer); keys tied
// at the T-th place run it to all 32 bits, which yields the T-th largest key
// itself.  The row is written in ascending block order with ballots: every
// key above the threshold, then keys equal to it in index order until T are
// taken.
//
// Both the scalar unit (one per CU, shared by its four SIMDs) and the VALU
// run close to an instruction per clock per CU here, so the per-row code
// avoids work on either: row coordinates come from multiply-shift divisions
// set up on the host, loads need no lane masks, keys come from branch-free
// integer arithmetic, and the search loops keep single exits.
#include "nsa_sel_common.h"
#include "nsa_topk.h"

namespace {

// Consecutive rows per wavefront (measured: 4 beats 8, 16 and 32, and loading
// two rows ahead beats none of them).
constexpr int kRowsPerWave = 4;

// Larger score -> larger key; NaN takes the key of -inf and -0 that of +0;
// every score maps to a key >= kMinKey (the key of -inf), leaving 0 free.
// Branch-free: -0 becomes +0 by adding +0 (in inline assembly, so that the
// compiler cannot reason about NaN inputs; f32 denormals are kept, so the
// sum is exact) and the usual sign flip orders the bit patterns.  The keys
// of NaNs then lie above +inf's and below -inf's; shifting every key by
// 0x007FFFFF wraps both ranges under -inf's, the maximum gathers them there,
// and the shift is undone.  (Left shifted, the keys would straddle the
// exponent boundaries and the bitwise search would need about three times
// the passes on 2048-candidate rows.)  No compares, so no lane-mask hazards.
constexpr unsigned kMinKey = 0x007FFFFFu;
constexpr unsigned kNanShift = 0x007FFFFFu;

__device__ __forceinline__ unsigned score_key(unsigned u) {
    asm("v_add_f32 %0, 0, %1" : "=v"(u) : "v"(u));
    const unsigned flip = (unsigned)((int)u >> 31) | 0x80000000u;
    return max((u ^ flip) + kNanShift, kMinKey + kNanShift) - kNanShift;
}

__device__ __forceinline__ int ballot_count(bool p) { return __builtin_popcountll(__ballot(p)); }

// Candidates 0 .. nc-1 of the row whose first candidate is src: register j
// holds candidates 64*j .. 64*j+63 and is loaded while 64*j < nc (one scalar
// test per register).  Lanes past the last candidate re-read it (their keys
// are masked when converted), so no lane mask is set per register.
template <int KREG>
__device__ __forceinline__ void load_row(const float *src, int nc, int lane, unsigned (&raw)[KREG]) {
    const unsigned *s = reinterpret_cast<const unsigned *>(src);
    const unsigned last = (unsigned)nc - 1u;
#pragma unroll
    for (int j = 0; j < KREG; ++j) {
        if (j * kWaveSize >= nc) break;
        raw[j] = __builtin_nontemporal_load(s + min((unsigned)(j * kWaveSize + lane), last));
    }
}

// The number of keys >= cand in registers 0 .. NJ-1: one compare and one
// scalar popcount per register.
template <int NJ, int KREG>
__device__ __forceinline__ int count_ge(const unsigned (&key)[KREG], unsigned cand) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        c += ballot_count(key[j] >= cand);
        if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    return c;
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
    unsigned thr = __builtin_amdgcn_readfirstlane(kth);
    asm volatile("" : "+s"(thr));
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

// Continues the bitwise search on one register of keys, from bit `bit` down,
// until exactly T keys lie at or above kth.  One loop exit on one scalar
// value (the next bit, or -1 once the count is exact): separate exits made
// the compiler build lane-mask booleans around them.
__device__ __forceinline__ unsigned refine_one(unsigned k, int T, int bit, unsigned kth, int cnt) {
    int b = cnt == T ? -1 : bit;
    while (b >= 0) {
        const unsigned cand = kth | (1u << b);
        const int c = ballot_count(k >= cand);
        const bool take = c >= T;
        kth = take ? cand : kth;
        b = (take && c == T) ? -1 : b - 1;
    }
    return kth;
}

// Selects the row's T largest keys and writes their block indices in
// ascending order.  The row's raw scores sit in registers 0 .. NJ-1 (lane l
// of register j: candidate 64*j + l, valid below nc); they are turned into
// keys first, then `next` issues the following row's loads into the same
// registers, so that they land while this row is selected.  `sh` is this
// wavefront's 256-word LDS scratch.
template <int NJ, int KREG, typename Next>
__device__ __forceinline__ void select_row(unsigned (&raw)[KREG], int nc, int T, int lane, int32_t *dst,
                                           unsigned *sh, Next &&next) {
    // Registers below the next smaller size bucket are full (the bucket was
    // chosen on nc), so only the upper ones need the per-lane mask.
    // (NJ = 2 also takes rows with one register.)
    constexpr int FULL = NJ <= 2 ? 0 : NJ <= 8 ? NJ - 2 : NJ <= 16 ? NJ - 4 : NJ <= 32 ? NJ - 8 : NJ - 16;
    unsigned key[NJ];
    int idx[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        idx[j] = j * kWaveSize + lane;
        key[j] = (j < FULL || idx[j] < nc) ? score_key(raw[j]) : 0u;
    }
    next(raw);
    // kth: the largest prefix with at least T keys >= kth, found bit by bit
    // from the top; cnt = the number of keys >= kth.  The search stops early
    // once T <= cnt <= max(T, 64): the keys fit one register (or are exactly
    // the answer).  One unsigned compare tests both bounds.
    // The loop has a single exit on one scalar value (separate exits made
    // the compiler build lane-mask booleans around them).  `bit` ends one
    // below the last bit tried.
    const unsigned stop = (unsigned)((T > kWaveSize ? T : kWaveSize) - T);
    unsigned kth = 0;
    int cnt = 0x7FFFFFFF;
    int bit = 31;
    int go;
    do {
        const unsigned cand = kth | (1u << bit);
        const int c = count_ge<NJ>(key, cand);
        const bool take = c >= T;  // (c - T) <= stop implies it
        kth = take ? cand : kth;
        cnt = take ? c : cnt;
        go = (unsigned)(c - T) <= stop ? 0 : bit;
        --bit;
    } while (go > 0);
    if (NJ == 1 || cnt > kWaveSize) {
        // Done on the registers themselves: exactly T > 64 keys are >= kth,
        // or the search ran through all 32 bits (more than 64 keys tie at
        // the T-th place), or the row fits one register anyway.
        if (NJ == 1) {
            kth = refine_one(key[0], T, bit, kth, cnt);
        }
        write_selection<NJ>(key, idx, kth, T, dst);
        return;
    }
    // Compact the cnt <= 64 keys >= kth (with their block indices) into one
    // register, in ascending block order: the later bits and the write-out
    // touch that register only.  Keys below kth can no longer be selected.
    // Every lane writes (the others into their own spare words 128 + lane
    // and 192 + lane), so no lane mask is set per register.
    int base = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool keep = key[j] >= kth;
        const uint64_t km = __ballot(keep);
        const int p = keep ? base + lanes_below(km) : 2 * kWaveSize + lane;
        sh[p] = key[j];
        sh[kWaveSize + p] = (unsigned)idx[j];
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
    kth = refine_one(k1[0], T, bit, kth, cnt);
    write_selection<1>(k1, i1, kth, T, dst);
}

// Dispatch on the number of registers that hold candidates (wave-uniform),
// rounded up to a size bucket no larger than KREG.
template <int KREG, typename Next>
__device__ __forceinline__ void select_any(unsigned (&raw)[KREG], int nc, int T, int lane, int32_t *dst,
                                           unsigned *sh, Next &&next) {
    const int nj = (nc + kWaveSize - 1) / kWaveSize;
    if (KREG <= 2 || nj <= 2) { select_row<(KREG < 2 ? KREG : 2)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 4 || nj <= 4) { select_row<(KREG < 4 ? KREG : 4)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 6 || nj <= 6) { select_row<(KREG < 6 ? KREG : 6)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 8 || nj <= 8) { select_row<(KREG < 8 ? KREG : 8)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 12 || nj <= 12) { select_row<(KREG < 12 ? KREG : 12)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 16 || nj <= 16) { select_row<(KREG < 16 ? KREG : 16)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 24 || nj <= 24) { select_row<(KREG < 24 ? KREG : 24)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 32 || nj <= 32) { select_row<(KREG < 32 ? KREG : 32)>(raw, nc, T, lane, dst, sh, next); return; }
    if (KREG <= 48 || nj <= 48) { select_row<(KREG < 48 ? KREG : 48)>(raw, nc, T, lane, dst, sh, next); return; }
    select_row<KREG>(raw, nc, T, lane, dst, sh, next);
}

// Division of n < 2^31 by a divisor fixed for the launch, with a multiplier
// and shift made on the host (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994): q = (mulhi(n, mul) + n)
// >> shift.  Three scalar instructions instead of a division sequence.
struct FastDiv {
    unsigned mul;
    unsigned shift;
};

__device__ __forceinline__ unsigned fast_div(unsigned n, FastDiv d) { return (__umulhi(n, d.mul) + n) >> d.shift; }

FastDiv make_fast_div(unsigned d) {
    unsigned shift = 0;
    while ((1ull << shift) < d) ++shift;
    const uint64_t mul = (((1ull << 32) * ((1ull << shift) - d)) / d) + 1;
    return FastDiv{(unsigned)mul, shift};
}

struct TopkArgs {
    const float *scores;
    int32_t *out;
    int rows, M, NB, T;
    FastDiv div_G, div_M, div_bs;
};

template <int KREG>
__global__ __launch_bounds__(256) void nsa_topk_kernel(TopkArgs a) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int r0 = __builtin_amdgcn_readfirstlane((blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * kRowsPerWave);
    if (r0 >= a.rows) return;  // whole wavefront
    const int r1 = min(a.rows, r0 + kRowsPerWave);
    __shared__ unsigned lds[4][4 * kWaveSize];
    unsigned *sh = lds[threadIdx.x >> 6];
    // Candidates 0 .. nc-1 of row (b*M + m)*G + g: the blocks t <= m / bs.
    auto cands = [&](int row) {
        const unsigned x = fast_div((unsigned)row, a.div_G);              // b*M + m
        const unsigned m = x - fast_div(x, a.div_M) * (unsigned)a.M;
        return min((int)fast_div(m, a.div_bs), a.NB - 1) + 1;
    };
    unsigned raw[KREG];
    int nc_next = cands(r0);
    if (nc_next > a.T) load_row<KREG>(a.scores + (size_t)r0 * a.NB, nc_next, lane, raw);
    for (int row = r0; row < r1; ++row) {
        const int nc = nc_next;
        int32_t *dst = a.out + (size_t)row * a.T;
        // The next row's scores load during this row's selection.
        auto next = [&](unsigned (&r)[KREG]) {
            if (row + 1 < r1) {
                nc_next = cands(row + 1);
                if (nc_next > a.T) load_row<KREG>(a.scores + (size_t)(row + 1) * a.NB, nc_next, lane, r);
            }
        };
        if (nc <= a.T) {
            next(raw);
            for (int i = lane; i < a.T; i += kWaveSize) dst[i] = i < nc ? i : -1;
        } else {
            select_any<KREG>(raw, nc, a.T, lane, dst, sh, next);
        }
    }
}

template <int KREG>
hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
    const int waves = (a.rows + kRowsPerWave - 1) / kRowsPerWave;
    hipLaunchKernelGGL((nsa_topk_kernel<KREG>), dim3((waves + 3) / 4), dim3(256), 0, stream, a);
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
    TopkArgs a;
    a.scores = scores;
    a.out = block_indices;
    a.rows = rows;
    a.M = M;
    a.NB = NB;
    a.T = T;
    a.div_G = make_fast_div((unsigned)G);
    a.div_M = make_fast_div((unsigned)M);
    a.div_bs = make_fast_div((unsigned)block_size);
    hipError_t e;
    const int kreg = (NB + kWaveSize - 1) / kWaveSize;
    if (kreg <= 1)
        e = launch_topk<1>(a, stream);
    else if (kreg <= 2)
        e = launch_topk<2>(a, stream);
    else if (kreg <= 4)
        e = launch_topk<4>(a, stream);
    else if (kreg <= 8)
        e = launch_topk<8>(a, stream);
    else if (kreg <= 16)
        e = launch_topk<16>(a, stream);
    else if (kreg <= 32)
        e = launch_topk<32>(a, stream);
    else
        e = launch_topk<64>(a, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}
