// NSA selection-attention forward for AMD MI355X (gfx950, CDNA4).
//
// Operation: wave issue "[wave] NSA: selection attention forward kernel",
// sections Operation, Algorithm, Requirements and "MI350 considerations".
// The page's program instance is one unit (b, m, g): all H/G heads of group g
// for query m attend, through one online softmax, to the keys of the blocks
// that block_indices[b, m, g, :] selects, under the causal mask; O and the
// natural-log log-sum-exp are written at the end.
//
// MI355X mapping (the design notes give the measurements behind each choice):
//  * A wavefront carries a slot of 1-8 consecutive queries of one (b, g):
//    PACK queries (gs heads each) fill a 16-column MFMA tile, and a wavefront
//    holds one or two tiles.  Their index rows are merged into one ascending
//    sequence of distinct blocks; each block is gathered once for the slot and
//    multiplied only for the tiles whose queries selected it.
//  * Scores are computed transposed, S^T = K * Q^T, on v_mfma_f32_16x16x32_f16:
//    keys are the 16 MFMA rows, heads (and packed queries) the columns.  The
//    S^T result layout is already the B-operand layout of the PV product, so
//    P never leaves registers.
//  * Each block is copied global -> LDS as 32-key sub-blocks with 128-bit
//    direct-to-LDS buffer loads whose lanes walk whole key rows (coalesced).
//    K fragments come from XOR-swizzled ds_read_b128, V^T fragments straight
//    from ds_read_b64_tr_b16.  The next sub-block's K copy is issued once this
//    one's K fragments are in registers, its V copy once the V fragments are.
//  * Four wavefronts per workgroup, two workgroups per CU (two wavefronts per
//    SIMD).  Workgroup w runs on XCD w % 8; slots are launched in generations
//    that fill every workgroup slot, each XCD walking a contiguous range of
//    (b, g, m), so the wavefronts resident on an XCD sweep the same key range
//    in step and share its L2.
#include "nsa_sel_common.h"

#include <type_traits>

namespace {

// One wavefront slot: QW = PACK * NT consecutive queries m0 .. m0+nq-1 of one
// (b, g), from index rows to stored O and LSE.  The wavefront's MFMA columns
// form NT tiles of 16; tile nt carries queries nt*PACK .. nt*PACK+PACK-1, gs
// heads each.  Every block of the merged sequence is staged once (kbuf/vbuf
// are the wavefront's LDS buffers) and multiplied only for the tiles whose
// queries selected it.
//
// SPLIT > 1 stages and computes each selected block as SPLIT consecutive
// sub-blocks of SBS = BS / SPLIT keys: half the LDS per wavefront, so twice as
// many wavefronts fit a CU.
//
// PIPE false is the unpipelined check build: the copies of sub-block s1 are
// issued only after all of s0's math, and each sub-block waits for every copy,
// so no copy is ever in flight while the wavefront reads LDS.  It runs the
// same arithmetic in the same order, so its results are bitwise those of the
// pipelined kernel unless a pipelined copy overwrote LDS still being read.
template <int BS, int SPLIT, int D, int PACK, int NT, class Merger, bool BF16, bool PIPE = true>
__device__ __forceinline__ void run_slot(const Params &p, int ws, int lane, _Float16 *kbuf, _Float16 *vbuf,
                                         void *mbuf) {
    constexpr int SBS = BS / SPLIT;
    constexpr int DC = D / 32;
    constexpr int KT = SBS / 16;
    constexpr int QW = PACK * NT;
    const Slot sl = decode_slot(p, ws, QW);
    const int b = sl.b, g = sl.g, m0 = sl.m0, nq = sl.nq;
    const int r = lane & 15;
    const int q4 = lane >> 4;
    const int h0 = g * p.gs;
    // Column r of tile nt carries head h0 + r % gs of query nt*PACK + r / gs.
    const int q_in_tile = r / p.gs;
    const int my_h = h0 + (r - q_in_tile * p.gs);
    bool live[NT];
    int my_m[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int qi = nt * PACK + q_in_tile;
        live[nt] = q_in_tile < PACK && qi < nq;
        my_m[nt] = m0 + (live[nt] ? qi : 0);
    }

    // Staging descriptors first: set up before the per-lane index and Q
    // loads, the compiler keeps them in scalar registers.
    Stage<SBS, D> st;
    init_stage(st, p, b, g, lane);

    // Q^T fragments (B operand): lane l holds column l%16, head-dim slice
    // 32*c + 8*(l/16) .. +7; columns without a query are zero.  Q, O, LSE and
    // the index rows are touched once, so they use non-temporal accesses and
    // leave the L2 to the gathered K/V blocks.
    half8 qf[NT][DC];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const _Float16 *qrow = p.Q + ((size_t)(b * (size_t)p.M + my_m[nt]) * p.H + (live[nt] ? my_h : h0)) * D;
        const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const half8 x = __builtin_nontemporal_load((const half8 *)(qrow + c * 32 + q4 * 8));
            qf[nt][c] = live[nt] ? x : zero8;
        }
    }

    Merger mg;
    mg.init(p, b, g, m0, nq, lane, mbuf);

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

    constexpr int NI = Stage<SBS, D>::NI;
    const unsigned tile_bits = (1u << PACK) - 1u;
    // The columns taking part in a block as a scalar lane mask, with up to
    // four queries per tile (not with the block-map merger, whose state
    // already fills the scalar registers).
    constexpr bool kScalarMask = PACK <= 4 && !std::is_same<Merger, MapMerger<PACK, BS>>::value;
    unsigned live_bits[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) live_bits[nt] = (1u << min(max(nq - nt * PACK, 0), PACK)) - 1u;

    // Pipeline over the merged sequence of sub-blocks (block t, part h): while
    // sub-block s0 is computed, the copies of the next one s1 into LDS are in
    // flight -- its K copy is issued as soon as s0's K fragments are in
    // registers, its V copy as soon as s0's V operands are, so each copy
    // overlaps about one sub-block of math.  Loads complete in issue order,
    // so each wait names how many later loads may still be pending.
    half8 kf[KT][DC];
    half4 vt[SBS / 32][DC][2][2];
    half4 pf[NT][KT];
    unsigned a0, a1;
    const int t_first = mg.next(a0);
    int s0 = t_first == kDone ? kDone : t_first * SPLIT;  // sub-block index = key0 / SBS
    if (s0 != kDone) {
        st.issue(st.rk, kbuf, s0, lane);
        st.issue(st.rv, vbuf, s0, lane);
    }
    while (s0 != kDone) {
        int s1;
        if ((s0 + 1) % SPLIT != 0) {  // next part of the same block, same queries
            s1 = s0 + 1;
            a1 = a0;
        } else {
            const int t1 = mg.next(a1);
            s1 = t1 == kDone ? kDone : t1 * SPLIT;
        }
        const bool has1 = s1 != kDone;
        if constexpr (PIPE)
            __builtin_amdgcn_s_waitcnt(wait_vm(NI));  // K(s0) landed; V(s0) may be pending
        else
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
        Stage<SBS, D>::read(kf, kbuf, r, q4);
        if (PIPE && has1) st.issue(st.rk, kbuf, s1, lane);
        const int key0 = s0 * SBS;
        // Raised wave priority while the products and the softmax issue (the
        // copy waits and fragment reads run at the normal one): of the two
        // wavefronts of a SIMD, the one with math ready goes first (measured
        // 1% at 64k, bitwise equal).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const unsigned tb = (a0 >> (nt * PACK)) & tile_bits;
            if (tb == 0) continue;  // wave-uniform: no query of this tile selected the block
            const int first_m = m0 + nt * PACK;
            const bool causal = (key0 + SBS - 1 > first_m) || (key0 + SBS > p.N);
            const bool col_on = live[nt] && ((tb >> q_in_tile) & 1u);
            const uint64_t on_lanes = kScalarMask ? col_lanes<PACK>(tb & live_bits[nt], p.gs) : 0;
            score_block<SBS, D, BF16, false, kScalarMask>(kf, qf[nt], key0, causal, true, col_on, INT_MIN,
                                                          min(my_m[nt], p.N - 1), p.scale_log2, m_run[nt],
                                                          l_run[nt], alpha[nt], pf[nt], q4, on_lanes);
        }
        __builtin_amdgcn_s_setprio(0);
        if (PIPE && has1)
            __builtin_amdgcn_s_waitcnt(wait_vm(NI));  // V(s0) landed; K(s1) may be pending
        else
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
        Stage<SBS, D>::read_vt(vt, vbuf, lane);
        if (PIPE && has1) st.issue(st.rv, vbuf, s1, lane);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (((a0 >> (nt * PACK)) & tile_bits) == 0) continue;
            accumulate_block<SBS, D, BF16>(vt, pf[nt], alpha[nt], acc[nt]);
        }
        __builtin_amdgcn_s_setprio(0);
        if (!PIPE && has1) {  // all of s0's LDS reads are done: stage s1
            st.issue(st.rk, kbuf, s1, lane);
            st.issue(st.rv, vbuf, s1, lane);
        }
        s0 = s1;
        a0 = a1;
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


// MODE 0: rows streamed through cursors (any T), one tile.  MODE 1/2: rows
// held in registers, NT = MODE tiles.
template <int BS, int SPLIT, int D, int PACK, int MODE, bool BF16, bool PIPE>
__global__ __launch_bounds__(kWaveSize * waves_per_wg(BS / SPLIT)) void nsa_sel_fwd_kernel(Params p) {
    constexpr int SBS = BS / SPLIT;
    constexpr int WAVES = waves_per_wg(SBS);
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ __attribute__((aligned(16))) _Float16 kbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf_all[WAVES][Stage<SBS, D>::HALVES];
    // Block maps of the rows of any length (MODE 0 only).
    __shared__ __attribute__((aligned(16))) unsigned char mbuf_all[MODE == 0 ? WAVES : 1][MODE == 0 ? kMapBlocks : 16];
    const int ws = wave_slot<WAVES>(p, wave);
    if (ws < 0) return;
    if constexpr (MODE == 0)
        run_slot<BS, SPLIT, D, PACK, 1, MapMerger<PACK, BS>, BF16, PIPE>(p, ws, lane, kbuf_all[wave], vbuf_all[wave],
                                                                 mbuf_all[wave]);
    else
        run_slot<BS, SPLIT, D, PACK, MODE, RegMerger<PACK * MODE, BS>, BF16, PIPE>(p, ws, lane, kbuf_all[wave],
                                                                               vbuf_all[wave], nullptr);
}

// The same slots as nsa_sel_fwd_kernel, run by the persistent schedule.
template <int BS, int SPLIT, int D, int PACK, int MODE, bool BF16, bool PIPE>
__global__ __launch_bounds__(kWaveSize * waves_per_wg(BS / SPLIT)) void nsa_sel_fwd_persistent_kernel(Params p) {
    constexpr int SBS = BS / SPLIT;
    constexpr int WAVES = waves_per_wg(SBS);
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ __attribute__((aligned(16))) _Float16 kbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) unsigned char mbuf_all[MODE == 0 ? WAVES : 1][MODE == 0 ? kMapBlocks : 16];
    run_persistent<WAVES>(p, wave, lane, [&](int ws) {
        if constexpr (MODE == 0)
            run_slot<BS, SPLIT, D, PACK, 1, MapMerger<PACK, BS>, BF16, PIPE>(p, ws, lane, kbuf_all[wave],
                                                                     vbuf_all[wave], mbuf_all[wave]);
        else
            run_slot<BS, SPLIT, D, PACK, MODE, RegMerger<PACK * MODE, BS>, BF16, PIPE>(p, ws, lane, kbuf_all[wave],
                                                                                   vbuf_all[wave], nullptr);
    });
}

template <bool BF16, bool PIPE = true>
struct FwdKernel {
    static constexpr bool kPersistent = true;
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    void launch(dim3 grid, dim3 block, hipStream_t stream, const Params &p) const {
        hipLaunchKernelGGL((nsa_sel_fwd_kernel<BS, SPLIT, D, PACK, MODE, BF16, PIPE>), grid, block, 0, stream, p);
    }
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    void launch_persist(dim3 grid, dim3 block, hipStream_t stream, const Params &p) const {
        hipLaunchKernelGGL((nsa_sel_fwd_persistent_kernel<BS, SPLIT, D, PACK, MODE, BF16, PIPE>), grid, block, 0,
                           stream, p);
    }
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    int resident() const {
        static std::atomic<int> cache[64];
        return resident_workgroups(cache,
                                   (const void *)nsa_sel_fwd_persistent_kernel<BS, SPLIT, D, PACK, MODE, BF16, PIPE>,
                                   kWaveSize * waves_per_wg(BS / SPLIT));
    }
};

}  // namespace

extern "C" const char *nsa_sel_status_string(int status) {
    switch (status) {
        case NSA_SEL_OK: return "ok";
        case NSA_SEL_ERR_NULL: return "nsa_sel: a pointer argument is NULL";
        case NSA_SEL_ERR_SHAPE: return "nsa_sel: a size is < 1 or H is not a multiple of G";
        case NSA_SEL_ERR_UNSUPPORTED:
            return "nsa_sel: unsupported configuration (D must be 64 or 128, block_size 32 or 64, H/G <= 16)";
        case NSA_SEL_ERR_ALIGN:
            return "nsa_sel: Q/K/V/O must be 16-byte aligned and block_indices/LSE 4-byte aligned";
        case NSA_SEL_ERR_RANGE: return "nsa_sel: problem size exceeds the supported index range";
        case NSA_SEL_ERR_ALIAS: return "nsa_sel: an output buffer overlaps an input or the other output";
        case NSA_SEL_ERR_HIP: return "nsa_sel: the HIP runtime reported an error at kernel launch";
        case NSA_SEL_ERR_WORKSPACE:
            return "nsa_sel: the workspace is NULL, not 256-byte aligned or smaller than required";
        case NSA_SEL_ERR_SCRATCH:
            return "nsa_sel: these sizes need more workspace than the 64 MiB scratch of nsa_sel_bwd_noalloc; "
                   "call nsa_sel_bwd with a workspace";
        default: return "nsa_sel: unknown status";
    }
}

namespace {

// Workspace bytes of the persistent schedule for checked sizes p on a device
// of topology tp (p is planned in place).
size_t fwd_workspace_bytes(Params &p, const Topology &tp) {
    plan_slots(p, tp);
    return (size_t)sched_words_bound(p, tp.cus) * 4;
}

// with_ws: the workspace entry points (workspace, workspace_bytes checked);
// otherwise generation launches only.
int sel_fwd(const void *Q, const void *K, const void *V, const int32_t *block_indices, void *O, float *LSE, int B,
            int M, int N, int H, int G, int D, int block_size, int T, hipStream_t stream, bool bf16,
            bool pipelined = true, bool with_ws = false, void *workspace = nullptr, size_t workspace_bytes = 0) {
    if (!Q || !K || !V || !block_indices || !O || !LSE) return NSA_SEL_ERR_NULL;
    Params p;
    const int st = check_sizes(B, M, N, H, G, D, block_size, T, p);
    if (st != NSA_SEL_OK) return st;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15) return NSA_SEL_ERR_ALIGN;
    if (((uintptr_t)block_indices | (uintptr_t)LSE) & 3) return NSA_SEL_ERR_ALIGN;

    const size_t q_bytes = (size_t)B * M * H * D * 2, kv_bytes = (size_t)B * N * G * D * 2;
    const size_t idx_bytes = (size_t)B * M * G * T * 4, lse_bytes = (size_t)B * H * M * 4;
    const void *ins[4] = {Q, K, V, block_indices};
    const size_t in_bytes[4] = {q_bytes, kv_bytes, kv_bytes, idx_bytes};
    for (int i = 0; i < 4; ++i) {
        if (ranges_overlap(O, q_bytes, ins[i], in_bytes[i]) ||
            ranges_overlap(LSE, lse_bytes, ins[i], in_bytes[i]))
            return NSA_SEL_ERR_ALIAS;
    }
    if (ranges_overlap(O, q_bytes, LSE, lse_bytes)) return NSA_SEL_ERR_ALIAS;

    const Topology tp = device_topology();
    const int cus = tp.cus;
    if (with_ws) {
        const size_t need = fwd_workspace_bytes(p, tp);
        if (need / 4 > (size_t)INT_MAX) return NSA_SEL_ERR_RANGE;
        if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < need) return NSA_SEL_ERR_WORKSPACE;
        for (int i = 0; i < 4; ++i)
            if (ranges_overlap(workspace, need, ins[i], in_bytes[i])) return NSA_SEL_ERR_ALIAS;
        if (ranges_overlap(workspace, need, O, q_bytes) || ranges_overlap(workspace, need, LSE, lse_bytes))
            return NSA_SEL_ERR_ALIAS;
        p.sched = (unsigned *)workspace;
        p.sched_cap = (int)(need / 4);
    } else {
        plan_slots(p, tp);
    }
    p.Q = (const _Float16 *)Q;
    p.K = (const _Float16 *)K;
    p.V = (const _Float16 *)V;
    p.idx = block_indices;
    p.O = (_Float16 *)O;
    p.LSE = LSE;
    const hipError_t e = !pipelined ? launch_all(FwdKernel<false, false>{}, p, block_size, D, cus, stream)
                         : bf16     ? launch_all(FwdKernel<true>{}, p, block_size, D, cus, stream)
                                    : launch_all(FwdKernel<false>{}, p, block_size, D, cus, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}

}  // namespace

extern "C" int nsa_sel_fwd(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                           void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                           int block_size, int T, hipStream_t stream) {
    return sel_fwd(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream, false);
}

extern "C" int nsa_sel_fwd_bf16(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                                void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                                int block_size, int T, hipStream_t stream) {
    return sel_fwd(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream, true);
}

extern "C" int nsa_sel_fwd_workspace_size(int B, int M, int N, int H, int G, int D, int block_size, int T,
                                          size_t *bytes) {
    if (!bytes) return NSA_SEL_ERR_NULL;
    Params p;
    const int st = check_sizes(B, M, N, H, G, D, block_size, T, p);
    if (st != NSA_SEL_OK) return st;
    const size_t b = fwd_workspace_bytes(p, device_topology());
    if (b / 4 > (size_t)INT_MAX) return NSA_SEL_ERR_RANGE;
    *bytes = b;
    return NSA_SEL_OK;
}

extern "C" int nsa_sel_fwd_ws(const void *Q, const void *K, const void *V, const int32_t *block_indices, void *O,
                              float *LSE, int B, int M, int N, int H, int G, int D, int block_size, int T,
                              void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return sel_fwd(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream, false, true, true,
                   workspace, workspace_bytes);
}

extern "C" int nsa_sel_fwd_bf16_ws(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                                   void *O, float *LSE, int B, int M, int N, int H, int G, int D, int block_size,
                                   int T, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return sel_fwd(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream, true, true, true,
                   workspace, workspace_bytes);
}

extern "C" int nsa_sel_fwd_unpipelined(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                                       void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                                       int block_size, int T, hipStream_t stream) {
    return sel_fwd(Q, K, V, block_indices, O, LSE, B, M, N, H, G, D, block_size, T, stream, false, false);
}
