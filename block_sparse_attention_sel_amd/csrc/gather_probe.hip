// Gather-ceiling probe for the NSA selection-attention forward kernel
// (gfx950).  It runs the forward kernel's block-gather stream alone: the same
// slot layout, generations, index-row merging, direct-to-LDS copies, waits
// and LDS fragment reads, without Q, scores, softmax or outputs.  Its time is
// what the forward kernel's memory traffic costs by itself.
//
// Cost centre named by wave issue "[wave] NSA: selection attention forward
// kernel", sections Algorithm and "MI350 considerations".
#include "nsa_sel_common.h"
#include "nsa_gather_probe.h"

namespace {

// The staging loop of one wavefront slot, in the forward kernel's order:
// wait for K(s0), read its fragments, issue K(s1); wait for V(s0), read its
// transposed fragments, issue V(s1).  Returns the number of blocks staged.
template <int BS, int SPLIT, int D, int PACK, int NT, class Merger>
__device__ __forceinline__ int probe_slot(const Params &p, int ws, int lane, _Float16 *kbuf, _Float16 *vbuf,
                                          void *mbuf) {
    constexpr int SBS = BS / SPLIT;
    constexpr int DC = D / 32;
    constexpr int KT = SBS / 16;
    constexpr int NI = Stage<SBS, D>::NI;
    const Slot sl = decode_slot(p, ws, PACK * NT);
    const int r = lane & 15;
    const int q4 = lane >> 4;

    Stage<SBS, D> st;
    init_stage(st, p, sl.b, sl.g, lane);
    Merger mg;
    mg.init(p, sl.b, sl.g, sl.m0, sl.nq, lane, mbuf);

    half8 kf[KT][DC];
    half4 vt[SBS / 32][DC][2][2];
    unsigned act;
    int blocks = 0;
    const int t_first = mg.next(act);
    int s0 = t_first == kDone ? kDone : t_first * SPLIT;
    if (s0 != kDone) {
        ++blocks;
        st.issue(st.rk, kbuf, s0, lane);
        st.issue(st.rv, vbuf, s0, lane);
    }
    while (s0 != kDone) {
        int s1;
        if ((s0 + 1) % SPLIT != 0) {
            s1 = s0 + 1;
        } else {
            const int t1 = mg.next(act);
            s1 = t1 == kDone ? kDone : t1 * SPLIT;
            blocks += t1 != kDone;
        }
        const bool has1 = s1 != kDone;
        __builtin_amdgcn_s_waitcnt(wait_vm(NI));
        Stage<SBS, D>::read(kf, kbuf, r, q4);
        if (has1) st.issue(st.rk, kbuf, s1, lane);
        if (has1)
            __builtin_amdgcn_s_waitcnt(wait_vm(NI));
        else
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
        Stage<SBS, D>::read_vt(vt, vbuf, lane);
        if (has1) st.issue(st.rv, vbuf, s1, lane);
        s0 = s1;
    }
    return blocks;
}

template <int BS, int SPLIT, int D, int PACK, int MODE>
__global__ __launch_bounds__(kWaveSize * waves_per_wg(BS / SPLIT)) void nsa_gather_probe_kernel(Params p,
                                                                                             uint64_t *staged) {
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
    int n;
    if constexpr (MODE == 0)
        n = probe_slot<BS, SPLIT, D, PACK, 1, MapMerger<PACK, BS>>(p, ws, lane, kbuf_all[wave], vbuf_all[wave],
                                                                 mbuf_all[wave]);
    else
        n = probe_slot<BS, SPLIT, D, PACK, MODE, RegMerger<PACK * MODE, BS>>(p, ws, lane, kbuf_all[wave],
                                                                               vbuf_all[wave], nullptr);
    if (lane == 0) atomicAdd((unsigned long long *)staged, (unsigned long long)n);
}

// The same slots run by the persistent schedule, as nsa_sel_fwd_ws runs them.
template <int BS, int SPLIT, int D, int PACK, int MODE>
__global__ __launch_bounds__(kWaveSize * waves_per_wg(BS / SPLIT)) void nsa_gather_probe_persistent_kernel(
    Params p, uint64_t *staged) {
    constexpr int SBS = BS / SPLIT;
    constexpr int WAVES = waves_per_wg(SBS);
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ __attribute__((aligned(16))) _Float16 kbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) unsigned char mbuf_all[MODE == 0 ? WAVES : 1][MODE == 0 ? kMapBlocks : 16];
    int n = 0;
    run_persistent<WAVES>(p, wave, lane, [&](int ws) {
        if constexpr (MODE == 0)
            n += probe_slot<BS, SPLIT, D, PACK, 1, MapMerger<PACK, BS>>(p, ws, lane, kbuf_all[wave], vbuf_all[wave],
                                                                      mbuf_all[wave]);
        else
            n += probe_slot<BS, SPLIT, D, PACK, MODE, RegMerger<PACK * MODE, BS>>(p, ws, lane, kbuf_all[wave],
                                                                                  vbuf_all[wave], nullptr);
    });
    if (lane == 0 && n > 0) atomicAdd((unsigned long long *)staged, (unsigned long long)n);
}

struct ProbeKernel {
    static constexpr bool kPersistent = true;
    uint64_t *staged;
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    void launch(dim3 grid, dim3 block, hipStream_t stream, const Params &p) const {
        hipLaunchKernelGGL((nsa_gather_probe_kernel<BS, SPLIT, D, PACK, MODE>), grid, block, 0, stream, p, staged);
    }
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    void launch_persist(dim3 grid, dim3 block, hipStream_t stream, const Params &p) const {
        hipLaunchKernelGGL((nsa_gather_probe_persistent_kernel<BS, SPLIT, D, PACK, MODE>), grid, block, 0, stream, p,
                           staged);
    }
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    int resident() const {
        static std::atomic<int> cache[64];
        return resident_workgroups(cache, (const void *)nsa_gather_probe_persistent_kernel<BS, SPLIT, D, PACK, MODE>,
                                   kWaveSize * waves_per_wg(BS / SPLIT));
    }
};

}  // namespace

extern "C" int nsa_gather_probe(const void *K, const void *V, const int32_t *block_indices, uint64_t *staged,
                                int B, int M, int N, int H, int G, int D, int block_size, int T, void *workspace,
                                size_t workspace_bytes, int *queries_per_slot, hipStream_t stream) {
    if (!K || !V || !block_indices || !staged) return NSA_SEL_ERR_NULL;
    Params p;
    const int st = check_sizes(B, M, N, H, G, D, block_size, T, p);
    if (st != NSA_SEL_OK) return st;
    if (((uintptr_t)K | (uintptr_t)V) & 15) return NSA_SEL_ERR_ALIGN;
    if ((uintptr_t)block_indices & 3) return NSA_SEL_ERR_ALIGN;
    if ((uintptr_t)staged & 7) return NSA_SEL_ERR_ALIGN;
    const Topology tp = device_topology();
    const int cus = tp.cus;
    plan_slots(p, tp);
    if (workspace) {
        const int64_t words = sched_words_bound(p, cus);
        if (words > INT_MAX) return NSA_SEL_ERR_RANGE;
        if (((uintptr_t)workspace & 255) || workspace_bytes < (size_t)words * 4) return NSA_SEL_ERR_WORKSPACE;
        p.sched = (unsigned *)workspace;
        p.sched_cap = (int)words;
    }
    if (queries_per_slot) *queries_per_slot = slot_queries(p);
    p.Q = nullptr;
    p.K = (const _Float16 *)K;
    p.V = (const _Float16 *)V;
    p.idx = block_indices;
    p.O = nullptr;
    p.LSE = nullptr;
    const hipError_t e = launch_all(ProbeKernel{staged}, p, block_size, D, cus, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}
