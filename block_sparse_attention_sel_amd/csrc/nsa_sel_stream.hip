// Shared-stream variant of the NSA selection-attention forward for gfx950.
//
// Operation: as nsa_sel_fwd (wave issue "[wave] NSA: selection attention
// forward kernel", sections Operation, Algorithm and Requirements).  The page
// asks for LDS staging of the irregular block gathers (section "MI350
// considerations"); this variant shares each staged block among more queries
// than one wavefront carries:
//   * a workgroup of 8 wavefronts (two per SIMD, one workgroup per CU) holds
//     QWG = 8 x 2 tiles x PACK consecutive queries of one (b, g);
//   * their index rows are folded into one map in LDS (a 32-bit mask of the
//     selecting queries per block), and the workgroup streams the union of
//     the selected blocks, in ascending order, through a ring of 8 sub-blocks
//     of 32 keys that all wavefronts fill together (each issues 1/8 of every
//     sub-block's copy instructions) -- every block is staged once for the
//     workgroup instead of once per wavefront;
//   * every wavefront walks the same map and passes the same LDS barrier
//     every 4 sub-blocks (the ring's free half is refilled there), but
//     multiplies only the sub-blocks one of its own queries selected.
// The per-tile step (S^T = K Q^T, lazy running max, P in registers, PV) is
// the forward kernel's.  Workgroups run in generations, each XCD walking a
// contiguous range of (b, g, query) slots, as the forward kernel's wavefronts
// do.
#include "nsa_sel_common.h"

namespace {

constexpr int kSwWaves = 8;          // wavefronts per workgroup (two per SIMD)
constexpr int kSwTiles = 2;          // 16-column tiles per wavefront
constexpr int kSwStages = 8;         // ring of 32-key sub-blocks (128 KiB at D = 128)
constexpr int kSwGroup = 4;          // sub-blocks per LDS barrier: the ring holds two groups
constexpr int kSwSbs = 32;
constexpr int kSwMapBlocks = 2048;   // blocks the union map covers (8 KiB)

// Walks the nonzero entries of the union map in ascending block order: lane
// l holds the mask of block cb + l of the current 64-block chunk, a ballot
// marks the blocks left.  The map reads are inline assembly (no compiler wait
// for the copies in flight).
struct MapCursor {
    unsigned base;  // LDS byte address of the map
    int lim;        // last block to visit
    int cb;         // first block of the loaded chunk
    unsigned word;
    uint64_t nz;
    int lane;

    __device__ __forceinline__ void init(unsigned base_, int lim_, int lane_) {
        base = base_;
        lim = lim_;
        lane = lane_;
        cb = -kWaveSize;
        word = 0;
        nz = 0;
    }
    __device__ __forceinline__ int next(unsigned &mask) {
        for (;;) {
            if (nz) {
                const int l = __builtin_ctzll(nz);
                mask = (unsigned)__builtin_amdgcn_readlane((int)word, l);
                nz &= nz - 1;
                return cb + l;
            }
            cb += kWaveSize;
            if (cb > lim) {
                mask = 0;
                return kDone;
            }
            unsigned w = 0;
            const unsigned addr = base + (unsigned)(cb + lane) * 4u;
            if (cb + lane <= lim) asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(w) : "v"(addr) : "memory");
            word = w;
            nz = __ballot(word != 0u);
        }
    }
};

template <int BS, int D, int PACK, bool BF16>
__global__ __launch_bounds__(kWaveSize * kSwWaves) void nsa_sel_stream_kernel(Params p) {
    constexpr int SPLIT = BS / kSwSbs;
    constexpr int SBS = kSwSbs;
    constexpr int NT = kSwTiles;
    constexpr int QWG = kSwWaves * NT * PACK;
    static_assert(QWG <= 32, "the query mask takes 32 bits");
    constexpr int DC = D / 32;
    constexpr int KT = SBS / 16;
    constexpr int NI = Stage<SBS, D>::NI;
    constexpr int IPW = (2 * NI) / kSwWaves;
    static_assert((2 * NI) % kSwWaves == 0 && IPW >= 1, "copy instructions must split evenly");
    __shared__ __attribute__((aligned(16))) _Float16 kbuf[kSwStages][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf[kSwStages][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) unsigned qmap[kSwMapBlocks];

    const int tid = threadIdx.x;
    const int lane = tid & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // This workgroup's slot: QWG consecutive queries of one (b, g).
    const int w = blockIdx.x;
    const int loc = p.gen * p.gen_step + w / p.nxcd;
    const int ws = (w % p.nxcd) * p.per_xcd + loc;
    if (loc >= p.per_xcd || ws >= p.wslots) return;  // the whole workgroup
    const int bg = ws / p.wslots_per_bg;
    const int q0 = (ws - bg * p.wslots_per_bg) * QWG;
    const int nq = min(QWG, p.M - q0);
    const int g = bg % p.G;
    const int b = bg / p.G;
    const int c_max = min((q0 + nq - 1) / BS, p.NB - 1);

    // The union map: bit q of block t set when query q0 + q counts entry t.
    const unsigned map_base = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned *)qmap;
    {
        const int4v zero = {0, 0, 0, 0};
        asm volatile("ds_write_b128 %0, %1" ::"v"(map_base + (unsigned)tid * 16u), "v"(zero) : "memory");
        static_assert(kSwMapBlocks * 4 == kWaveSize * kSwWaves * 16, "one 16-byte clear per thread");
        lds_barrier();
        const int32_t *rows = p.idx + ((size_t)(b * (size_t)p.M + q0) * p.G + g) * p.T;
        for (int e = tid; e < nq * p.T; e += kWaveSize * kSwWaves) {
            const int qi = e / p.T;
            const int t = __builtin_nontemporal_load(&rows[(size_t)qi * p.G * p.T + (e - qi * p.T)]);
            if (t >= 0 && t <= (q0 + qi) / BS && t < p.NB)
                asm volatile("ds_or_b32 %0, %1" ::"v"(map_base + (unsigned)t * 4u), "v"(1u << qi) : "memory");
        }
        lds_barrier();
    }
    // Sub-blocks of the stream: SPLIT per selected block.
    int nblk = 0;
    for (int c0 = 0; c0 <= c_max; c0 += kWaveSize) {
        unsigned wd = 0;
        if (c0 + lane <= c_max)
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(wd) : "v"(map_base + (unsigned)(c0 + lane) * 4u)
                         : "memory");
        nblk += __builtin_popcountll(__ballot(wd != 0u));
    }
    const int nsub = nblk * SPLIT;

    Stage<SBS, D> st;
    init_stage(st, p, b, g, lane);

    // This wavefront's tiles: tile nt carries queries q0 + (wave*NT + nt)*PACK + 0 .. PACK-1.
    const int r = lane & 15;
    const int q4 = lane >> 4;
    const int h0 = g * p.gs;
    const int q_in_tile = r / p.gs;
    const int my_h = h0 + (r - q_in_tile * p.gs);
    bool live[NT];
    int my_m[NT], first_m[NT];
    half8 qf[NT][DC];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int qb = (wave * NT + nt) * PACK;
        first_m[nt] = q0 + qb;
        live[nt] = q_in_tile < PACK && qb + q_in_tile < nq;
        my_m[nt] = live[nt] ? q0 + qb + q_in_tile : q0;
        const _Float16 *qrow = p.Q + ((size_t)(b * (size_t)p.M + my_m[nt]) * p.H + (live[nt] ? my_h : h0)) * D;
        const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const half8 x = __builtin_nontemporal_load((const half8 *)(qrow + c * 32 + q4 * 8));
            qf[nt][c] = live[nt] ? x : zero8;
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // Q is in registers before the copies start counting

    float m_run[NT], l_run[NT], alpha[NT];
    float4v acc[NT][DC][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
        alpha[nt] = 1.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            acc[nt][c][0] = float4v{0.f, 0.f, 0.f, 0.f};
            acc[nt][c][1] = float4v{0.f, 0.f, 0.f, 0.f};
        }
    }

    // Producer: issues this wavefront's share of sub-block j's copies, j in
    // stream order (its own walk of the map, one group ahead of the reads).
    MapCursor prod;
    prod.init(map_base, c_max, lane);
    int p_blk = 0;
    auto issue = [&](int j) {
        unsigned mk;
        if (j % SPLIT == 0) p_blk = prod.next(mk);
        const int sb = p_blk * SPLIT + j % SPLIT;  // 32-key sub-block of the key axis
        const int slot = j % kSwStages;
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int i = wave + k * kSwWaves;
            if (i < NI)
                st.issue_part(st.rk, kbuf[slot], sb, i, lane);
            else
                st.issue_part(st.rv, vbuf[slot], sb, i - NI, lane);
        }
    };
#pragma unroll
    for (int j = 0; j < kSwGroup; ++j)
        if (j < nsub) issue(j);
    // Group barriers, passed in order before the first read of a group: this
    // wavefront's copies of the group landed, then everyone's (one LDS
    // barrier), and everyone is done with the other half of the ring, which
    // is refilled with the next group.  Every wavefront passes every barrier.
    int bar_next = 0;
    auto ensure = [&](int j) {
        while (bar_next <= j / kSwGroup) {
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
            lds_barrier();
            const int first = (bar_next + 1) * kSwGroup;
#pragma unroll
            for (int k = 0; k < kSwGroup; ++k)
                if (first + k < nsub) issue(first + k);
            ++bar_next;
        }
    };

    MapCursor cons;
    cons.init(map_base, c_max, lane);
    const unsigned tile_bits = (1u << PACK) - 1u;
    const int my_shift = wave * NT * PACK;
    half8 kf[KT][DC];
    half4 vt[SBS / 32][DC][2][2];
    half4 pf[NT][KT];
    int c_blk = 0;
    unsigned c_mask = 0;
    for (int j = 0; j < nsub; ++j) {
        if (j % SPLIT == 0) c_blk = cons.next(c_mask);
        ensure(j);
        const unsigned mine = (c_mask >> my_shift) & ((1u << (NT * PACK)) - 1u);
        if (mine == 0) continue;  // wave-uniform: none of this wavefront's queries selected the block
        const int slot = j % kSwStages;
        const int key0 = (c_blk * SPLIT + j % SPLIT) * SBS;
        Stage<SBS, D>::read(kf, kbuf[slot], r, q4);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const unsigned tb = (mine >> (nt * PACK)) & tile_bits;
            if (tb == 0) continue;
            const bool causal = (key0 + SBS - 1 > first_m[nt]) || (key0 + SBS > p.N);
            const bool col_on = live[nt] && ((tb >> q_in_tile) & 1u);
            score_block<SBS, D, BF16>(kf, qf[nt], key0, causal, true, col_on, INT_MIN, min(my_m[nt], p.N - 1),
                                      p.scale_log2, m_run[nt], l_run[nt], alpha[nt], pf[nt], q4);
        }
        __builtin_amdgcn_s_setprio(0);
        Stage<SBS, D>::read_vt(vt, vbuf[slot], lane);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (((mine >> (nt * PACK)) & tile_bits) == 0) continue;
            accumulate_block<SBS, D, BF16>(vt, pf[nt], alpha[nt], acc[nt]);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // Epilogue: total row sum over the 4 lanes of a column, normalise, store.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const float l = col_sum(l_run[nt]);
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        if (live[nt]) {
            _Float16 *orow = p.O + ((size_t)(b * (size_t)p.M + my_m[nt]) * p.H + my_h) * D;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const half4 lo = pack4<BF16>(acc[nt][c][0] * inv);
                const half4 hi = pack4<BF16>(acc[nt][c][1] * inv);
                __builtin_nontemporal_store(cat8(lo, hi), (half8 *)(orow + c * 32 + q4 * 8));
            }
            if (q4 == 0) {
                const float lse = l > 0.f ? m_run[nt] * kLn2 + logf(l) : -INFINITY;
                __builtin_nontemporal_store(lse, &p.LSE[((size_t)b * p.H + my_h) * p.M + my_m[nt]]);
            }
        }
    }
}

template <int BS, int D, int PACK, bool BF16>
hipError_t launch_stream(Params p, const Topology &tp, hipStream_t stream) {
    constexpr int QWG = kSwWaves * kSwTiles * PACK;
    p.nxcd = tp.nxcd;
    p.wslots_per_bg = (p.M + QWG - 1) / QWG;
    p.wslots = p.B * p.G * p.wslots_per_bg;
    p.per_xcd = (p.wslots + p.nxcd - 1) / p.nxcd;
    p.gen_step = tp.cus / p.nxcd > 0 ? tp.cus / p.nxcd : 1;  // one workgroup per CU
    const int gens = (p.per_xcd + p.gen_step - 1) / p.gen_step;
    for (int gi = 0; gi < gens; ++gi) {
        p.gen = gi;
        hipLaunchKernelGGL((nsa_sel_stream_kernel<BS, D, PACK, BF16>), dim3(p.gen_step * p.nxcd),
                           dim3(kWaveSize * kSwWaves), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

extern "C" int nsa_sel_fwd_stream(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                                  void *O, float *LSE, int B, int M, int N, int H, int G, int D, int block_size,
                                  int T, hipStream_t stream) {
    if (!Q || !K || !V || !block_indices || !O || !LSE) return NSA_SEL_ERR_NULL;
    Params p;
    const int st = check_sizes(B, M, N, H, G, D, block_size, T, p);
    if (st != NSA_SEL_OK) return st;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15) return NSA_SEL_ERR_ALIGN;
    if (((uintptr_t)block_indices | (uintptr_t)LSE) & 3) return NSA_SEL_ERR_ALIGN;
    // This variant covers D = 128, at most 2 queries per 16-column tile (H/G
    // >= 5) and causal ranges of up to 2048 blocks.
    if (D != 128 || p.pack > 2 || (M - 1) / block_size >= kSwMapBlocks) return NSA_SEL_ERR_UNSUPPORTED;
    const Topology tp = device_topology();
    p.Q = (const _Float16 *)Q;
    p.K = (const _Float16 *)K;
    p.V = (const _Float16 *)V;
    p.idx = block_indices;
    p.O = (_Float16 *)O;
    p.LSE = LSE;
    hipError_t e;
    if (block_size == 64)
        e = p.pack == 2 ? launch_stream<64, 128, 2, false>(p, tp, stream) : launch_stream<64, 128, 1, false>(p, tp, stream);
    else
        e = p.pack == 2 ? launch_stream<32, 128, 2, false>(p, tp, stream) : launch_stream<32, 128, 1, false>(p, tp, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}
