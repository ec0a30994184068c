// NSA selection-attention backward for AMD MI355X (gfx950, CDNA4).
//
// Operation (include/nsa_sel_bwd.h): the gradients dQ, dK, dV of the
// selection attention of nsa_sel_fwd, from the forward's O and LSE and the
// upstream gradient dO.  Wave issue "[wave] NSA: selection attention forward
// kernel", section Requirements, names this pass as what the returned LSE is
// for: P = exp(S - LSE) is recomputed block by block without a softmax pass.
//
// The work splits by who owns each gradient:
//  * dQ is a sum over the selected keys of one query, so it is computed
//    query-major, exactly on the forward's slot layout and plan (one or two
//    16-column tiles per wavefront): a wavefront carries a slot of
//    consecutive queries of one (b, g), merges their index rows and stages
//    each selected 32-key sub-block once.  Per sub-block it forms
//    S^T = K Q^T and dP^T = V dO^T (v_mfma_f32_16x16x32_f16, keys on the MFMA
//    rows), P^T = exp2(S^T log2(e)/sqrt(D) - LSE log2(e)), dS^T = P^T (dP^T -
//    Delta), and accumulates dQ^T += K^T dS^T with K^T from the transposing
//    LDS reads and dS^T straight from registers.  The same pass computes
//    Delta = dO . O per row and stores (LSE log2(e), Delta) for the key pass.
//  * dK and dV are sums over the queries that selected a key, so they are
//    computed key-major.  The index rows are first inverted into a bitmap per
//    key block (bit m of row (b, g, t) set when query m selects block t),
//    without atomics on global memory; each key block's query list is cut
//    into items of at most qc queries.  A workgroup takes one item: its
//    wavefronts own 16 keys each, with their K and V fragments in registers,
//    and stream the item's queries as 32-row tiles (row = query, head) of Q,
//    dO and the row statistics, gathered global -> LDS with direct-to-LDS
//    loads through a ring shared by the workgroup.  Per tile: S = Q K^T,
//    dP = dO V^T, P, dS, then dV^T += dO^T P and dK^T += Q^T dS with the
//    transposed row operands from ds_read_b64_tr_b16.
//  * A key block cut into several items writes one partial sum per item; a
//    last pass adds them in item order (and writes zeros for key blocks no
//    query selected), so results do not depend on scheduling.
#include "nsa_sel_common.h"
#include "nsa_sel_bwd.h"

#include <mutex>
#include <type_traits>

// Scratch of the allocation-free entry point (nsa_sel_bwd_noalloc): its
// workspace lives in this file-scope device array, one copy per GPU, held for
// the life of the process.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy is looked up once, with that GPU current, and
// used instead.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

#include <algorithm>

namespace {

// ---------------------------------------------------------------------------
// dQ pass (query-major).

struct DqArgs {
    const _Float16 *O;
    const _Float16 *dO;
    const float *LSE;
    float *dQ;
    float2 *rowstat;  // [B, H, M]: (LSE * log2 e, Delta)
    float scale;      // 1 / sqrt(D)
};

// One 32-key sub-block of the dQ pass for one 16-column tile (lane l holds
// column l%16, keys key0 + 16*kt + 4*(l/16) + i), in two steps so that the K
// row fragments are dead before the V fragments are read: dq_scores forms
// S^T = K Q^T; dq_grad forms dP^T = V dO^T, P^T, dS^T and dQ^T += K^T dS^T.
//   causal: some key may lie past the column's last visible key lim
//   col_on: the column's query selected the block (else P = 0)
template <int SBS, int D>
__device__ __forceinline__ void dq_scores(const half8 (&kf)[SBS / 16][D / 32], const half8 (&qf)[D / 32],
                                          float4v (&s)[SBS / 16]) {
#pragma unroll
    for (int k = 0; k < SBS / 16; ++k) {
        s[k] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) s[k] = mfma_16x16x32(kf[k][c], qf[c], s[k]);
    }
}

// The lane id, recomputed where it is used.  The dQ step holds nearly 256
// live registers, and a per-lane value kept across the sub-block loop gets
// spilled; its reload waits for every copy in flight (vmcnt(0)), which
// exposes the next sub-block's copy latency.  Two VALU instructions instead.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Query of the tile (0 .. 15) that column r (0 .. 15) belongs to, r / gs,
// as (r * ceil(2^16 / gs)) >> 16, which is exact for r < 16 and gs <= 16.
__device__ __forceinline__ int col_query(int r, unsigned gs_magic) { return (int)(__umul24((unsigned)r, gs_magic) >> 16); }

//   tbits: bit q set when query q of the tile selected the block and is live
//   first_m: the tile's first query; lim = min(first_m + (l%16) / gs, N - 1)
//   lse2e: the column's LSE log2(e), or +inf for a row with no visible key
//   SMASK: select the columns with a scalar lane mask (PACK <= 4; not with
//   the block-map merger, whose state already fills the scalar registers)
template <int SBS, int D, int PACK, bool SMASK>
__device__ __forceinline__ void dq_grad(const half8 (&vf)[SBS / 16][D / 32], const half4 (&kt)[SBS / 32][D / 32][2][2],
                                        const half8 (&df)[D / 32], float4v (&s)[SBS / 16], int key0,
                                        bool causal, unsigned tbits, int first_m, int n_keys, int gs,
                                        unsigned gs_magic, float scale_log2, float lse2e, float delta,
                                        float4v (&acc)[D / 32][2]) {
    constexpr int KT = SBS / 16;
    constexpr int DC = D / 32;
    float4v dp[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        dp[k] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DC; ++c) dp[k] = mfma_16x16x32(vf[k][c], df[c], dp[k]);
    }
    // A column whose query did not select the block gets P = exp2(-inf) = 0,
    // and so does a key past the column's last visible one (masked under a
    // wave-uniform branch: only the sub-blocks on the diagonal take it).
    float m_exp;
    if constexpr (SMASK) {
        m_exp = select_lanes(col_lanes<PACK>(tbits, gs), INFINITY, lse2e);
    } else {
        const int cq = col_query(fresh_lane() & 15, gs_magic);
        m_exp = ((tbits >> cq) & 1u) ? lse2e : INFINITY;
    }
    if (causal) {
        const int l = fresh_lane();
        const int lim = min(first_m + col_query(l & 15, gs_magic), n_keys - 1) - key0 - 4 * (l >> 4);
#pragma unroll
        for (int k = 0; k < KT; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (k * 16 + i > lim) s[k][i] = -INFINITY;
    }
    half4 dsf[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        float4v ds;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pv = fast_exp2(__builtin_fmaf(s[k][i], scale_log2, -m_exp));
            ds[i] = pv * (dp[k][i] - delta);
        }
        dsf[k] = to_half4(ds);
    }
#pragma unroll
    for (int kc = 0; kc < SBS / 32; ++kc) {
        const half8 bp = cat8(dsf[2 * kc], dsf[2 * kc + 1]);
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                acc[c][hh] = mfma_16x16x32(cat8(kt[kc][c][hh][0], kt[kc][c][hh][1]), bp, acc[c][hh]);
    }
}

// One wavefront slot of the dQ pass: the forward's run_slot with the
// gradient step in place of the online softmax.
template <int BS, int SPLIT, int D, int PACK, int NT, class Merger>
__device__ __forceinline__ void dq_slot(const Params &p, const DqArgs &x, int ws, int lane, _Float16 *kbuf,
                                        _Float16 *vbuf, void *mbuf) {
    constexpr int SBS = BS / SPLIT;
    constexpr int DC = D / 32;
    constexpr int KT = SBS / 16;
    constexpr int QW = PACK * NT;
    const Slot sl = decode_slot(p, ws, QW);
    const int b = sl.b, g = sl.g, m0 = sl.m0, nq = sl.nq;
    const int r = lane & 15;
    const int q4 = lane >> 4;
    const int h0 = g * p.gs;
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

    Stage<SBS, D> st;
    init_stage(st, p, b, g, lane);

    // Q^T and dO^T fragments (B operands, lane l: column l%16, head dims
    // 32*c + 8*(l/16) .. +7), Delta = dO . O per column, and LSE.
    half8 qf[NT][DC], df[NT][DC];
    float lse2[NT], delta[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const size_t row = ((size_t)(b * (size_t)p.M + my_m[nt]) * p.H + (live[nt] ? my_h : h0)) * D;
        const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const half8 xq = __builtin_nontemporal_load((const half8 *)(p.Q + row + c * 32 + q4 * 8));
            const half8 xd = __builtin_nontemporal_load((const half8 *)(x.dO + row + c * 32 + q4 * 8));
            const half8 xo = __builtin_nontemporal_load((const half8 *)(x.O + row + c * 32 + q4 * 8));
            qf[nt][c] = live[nt] ? xq : zero8;
            df[nt][c] = live[nt] ? xd : zero8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = __builtin_fmaf((float)xd[e], (float)xo[e], dot);
        }
        delta[nt] = col_sum(live[nt] ? dot : 0.f);
        const size_t li = ((size_t)b * p.H + (live[nt] ? my_h : h0)) * p.M + my_m[nt];
        lse2[nt] = x.LSE[li] * kLog2e;
        if (live[nt] && q4 == 0) x.rowstat[li] = make_float2(lse2[nt], delta[nt]);
    }

    Merger mg;
    mg.init(p, b, g, m0, nq, lane, mbuf);

    float4v acc[NT][DC][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            acc[nt][c][0] = float4v{0.f, 0.f, 0.f, 0.f};
            acc[nt][c][1] = float4v{0.f, 0.f, 0.f, 0.f};
        }

    constexpr int NI = Stage<SBS, D>::NI;
    constexpr bool kScalarMask = PACK <= 4 && !std::is_same<Merger, MapMerger<PACK, BS>>::value;
    const unsigned tile_bits = (1u << PACK) - 1u;
    float lse2e[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lse2e[nt] = lse2[nt] == -INFINITY ? INFINITY : lse2[nt];
    // Live queries of each tile (a query past the end of the rows is not).
    const unsigned gs_magic = (65536u + (unsigned)p.gs - 1u) / (unsigned)p.gs;
    unsigned live_bits[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n_live = min(max(nq - nt * PACK, 0), PACK);
        live_bits[nt] = (1u << n_live) - 1u;
    }

    // Same pipeline as the forward: K(s1) is issued once K(s0)'s row and
    // transposed fragments are in registers, V(s1) once V(s0)'s are.
    half8 kf[KT][DC], vf[KT][DC];
    half4 kt[SBS / 32][DC][2][2];
    unsigned a0, a1;
    const int t_first = mg.next(a0);
    int s0 = t_first == kDone ? kDone : t_first * SPLIT;
    if (s0 != kDone) {
        st.issue(st.rk, kbuf, s0, lane);
        st.issue(st.rv, vbuf, s0, lane);
    }
    while (s0 != kDone) {
        int s1;
        if ((s0 + 1) % SPLIT != 0) {
            s1 = s0 + 1;
            a1 = a0;
        } else {
            const int t1 = mg.next(a1);
            s1 = t1 == kDone ? kDone : t1 * SPLIT;
        }
        const bool has1 = s1 != kDone;
        __builtin_amdgcn_s_waitcnt(wait_vm(NI));  // K(s0) landed
        Stage<SBS, D>::read(kf, kbuf, r, q4);
        Stage<SBS, D>::read_vt(kt, kbuf, lane);
        if (has1) st.issue(st.rk, kbuf, s1, lane);
        float4v sc[NT][KT];
        // Raised wave priority while products issue, as in the forward.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            if ((a0 >> (nt * PACK)) & tile_bits) dq_scores<SBS, D>(kf, qf[nt], sc[nt]);
        __builtin_amdgcn_s_setprio(0);
        if (has1)
            __builtin_amdgcn_s_waitcnt(wait_vm(NI));  // V(s0) landed
        else
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
        Stage<SBS, D>::read(vf, vbuf, r, q4);
        if (has1) st.issue(st.rv, vbuf, s1, lane);
        const int key0 = s0 * SBS;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const unsigned tb = (a0 >> (nt * PACK)) & tile_bits;
            if (tb == 0) continue;
            const int first_m = m0 + nt * PACK;
            const bool causal = (key0 + SBS - 1 > first_m) || (key0 + SBS > p.N);
            dq_grad<SBS, D, PACK, kScalarMask>(vf, kt, df[nt], sc[nt], key0, causal, tb & live_bits[nt], first_m, p.N, p.gs,
                                  gs_magic, p.scale_log2, lse2e[nt], delta[nt], acc[nt]);
        }
        __builtin_amdgcn_s_setprio(0);
        s0 = s1;
        a0 = a1;
    }

    // dQ = dS K / sqrt(D): lane l holds rows d = 32*c + 8*(l/16) + 4*hh + i
    // of column l%16, i.e. 8 consecutive floats per c.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (!live[nt]) continue;
        float *dq = x.dQ + ((size_t)(b * (size_t)p.M + my_m[nt]) * p.H + my_h) * D;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            __builtin_nontemporal_store(acc[nt][c][0] * x.scale, (float4v *)(dq + c * 32 + q4 * 8));
            __builtin_nontemporal_store(acc[nt][c][1] * x.scale, (float4v *)(dq + c * 32 + q4 * 8 + 4));
        }
    }
}

// Two wavefronts per SIMD even with two tiles per wavefront: the compiler then
// spills a few VGPRs of the two-tile kernel (D = 128; written before the
// block loop and reloaded after it, never inside it), which measured 10%
// faster over the whole backward than one tile per wavefront (189 VGPRs) and
// than two tiles at one wavefront per SIMD (274 VGPRs).
template <int BS, int SPLIT, int D, int PACK, int MODE>
__global__ __launch_bounds__(kWaveSize * waves_per_wg(BS / SPLIT)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void nsa_sel_bwd_dq_kernel(Params p, DqArgs x) {
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
        dq_slot<BS, SPLIT, D, PACK, 1, MapMerger<PACK, BS>>(p, x, ws, lane, kbuf_all[wave], vbuf_all[wave],
                                                                 mbuf_all[wave]);
    else
        dq_slot<BS, SPLIT, D, PACK, MODE, RegMerger<PACK * MODE, BS>>(p, x, ws, lane, kbuf_all[wave],
                                                                        vbuf_all[wave], nullptr);
}

// The same slots run by the persistent schedule of the forward (run_persistent):
// one workgroup per workgroup slot of the device, the workgroups of each XCD
// taking one generation per step and, once their own range is done,
// generations of other XCDs.  Each slot runs once with the same code, so dQ
// and the row statistics are bitwise those of the generation launches.
template <int BS, int SPLIT, int D, int PACK, int MODE>
__global__ __launch_bounds__(kWaveSize * waves_per_wg(BS / SPLIT)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void nsa_sel_bwd_dq_persistent_kernel(Params p, DqArgs x) {
    constexpr int SBS = BS / SPLIT;
    constexpr int WAVES = waves_per_wg(SBS);
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ __attribute__((aligned(16))) _Float16 kbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf_all[WAVES][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) unsigned char mbuf_all[MODE == 0 ? WAVES : 1][MODE == 0 ? kMapBlocks : 16];
    run_persistent<WAVES>(p, wave, lane, [&](int ws) {
        if constexpr (MODE == 0)
            dq_slot<BS, SPLIT, D, PACK, 1, MapMerger<PACK, BS>>(p, x, ws, lane, kbuf_all[wave], vbuf_all[wave],
                                                                 mbuf_all[wave]);
        else
            dq_slot<BS, SPLIT, D, PACK, MODE, RegMerger<PACK * MODE, BS>>(p, x, ws, lane, kbuf_all[wave],
                                                                            vbuf_all[wave], nullptr);
    });
}

struct DqKernel {
    static constexpr bool kPersistent = true;
    DqArgs x;
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    void launch(dim3 grid, dim3 block, hipStream_t stream, const Params &p) const {
        hipLaunchKernelGGL((nsa_sel_bwd_dq_kernel<BS, SPLIT, D, PACK, MODE>), grid, block, 0, stream, p, x);
    }
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    void launch_persist(dim3 grid, dim3 block, hipStream_t stream, const Params &p) const {
        hipLaunchKernelGGL((nsa_sel_bwd_dq_persistent_kernel<BS, SPLIT, D, PACK, MODE>), grid, block, 0, stream, p,
                           x);
    }
    template <int BS, int SPLIT, int D, int PACK, int MODE>
    int resident() const {
        static std::atomic<int> cache[64];
        return resident_workgroups(cache, (const void *)nsa_sel_bwd_dq_persistent_kernel<BS, SPLIT, D, PACK, MODE>,
                                   kWaveSize * waves_per_wg(BS / SPLIT));
    }
};

template <int BS, int D, int PACK>
hipError_t dq_launch_mode(const DqKernel &f, const Params &p, int cus, hipStream_t stream) {
    constexpr int SPLIT = BS / 32;
    switch (p.mode) {
        case 2: return launch_generations<DqKernel, BS, SPLIT, D, PACK, 2>(f, p, cus, stream);
        case 1: return launch_generations<DqKernel, BS, SPLIT, D, PACK, 1>(f, p, cus, stream);
        default: return launch_generations<DqKernel, BS, SPLIT, D, PACK, 0>(f, p, cus, stream);
    }
}

template <int BS, int D>
hipError_t dq_launch_pack(const DqKernel &f, const Params &p, int cus, hipStream_t stream) {
    if (p.pack == 4) return dq_launch_mode<BS, D, 4>(f, p, cus, stream);
    if (p.pack == 2) return dq_launch_mode<BS, D, 2>(f, p, cus, stream);
    return dq_launch_mode<BS, D, 1>(f, p, cus, stream);
}

// ---------------------------------------------------------------------------
// Key-major passes: inverted index, dK/dV, reduction.

constexpr int kBitQ = 256;     // queries per bitmap workgroup (8 words)
constexpr int kBitWin = 512;   // key-block rows per LDS window of the bitmap pass
constexpr int kRows = 32;      // (query, head) rows per tile of the dK/dV pass
constexpr int kRing = 4;       // LDS ring depth of the dK/dV pass (two workgroups still fit a CU)
constexpr int kMaxQc = 2048;   // most queries per item

struct Bw {
    const _Float16 *Q, *K, *V, *dO;
    const int32_t *idx;
    float2 *rowstat;    // [B*H*M + 1]; the last entry is the padding row (+inf, 0)
    unsigned *bits;     // [R][MW]
    int *row_items;     // [R] items of key block row
    int *row_first;     // [R] first item of the row
    int *row_part;      // [R] first partial slot of a row with >= 2 items
    int *starts;        // [R][kmax] first query of each item
    int2 *items;        // [cap] (row, k)
    int *n_items;       // [2]: items, then the overflow flag (nonzero: a capacity bound was exceeded)
    float *part;        // [pcap][2][bs][D] partial dK, dV
    float *dK, *dV;
    int B, M, N, H, G, gs, T, bs, NB, MW, R, qc, kmax, cap, pcap, qpt;
    int sentinel;       // B*H*M
    int nxcd;           // XCDs of the device (grid rounding)
    float scale, scale_log2;
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) {
        const int y = __shfl_up(x, o, kWaveSize);
        if (lane >= o) x += y;
    }
    return x;
}

// Position of the r-th (0-based) set bit of a word holding more than r.
__device__ __forceinline__ int nth_bit(unsigned word, int r) {
    for (int i = 0; i < r; ++i) word &= word - 1u;
    return __builtin_ctz(word);
}

// Bitmap of the selections: workgroup (b, g, chunk of 256 queries), one
// thread per query, OR-ing its counted entries into LDS words (ds_or), then
// writing rows t = 0 .. (last query of the chunk) / bs of its 8 words.  Words
// of row t before query t*bs are never read, so nothing else needs clearing.
__global__ __launch_bounds__(kBitQ) void nsa_sel_bwd_bitmap_kernel(Bw w) {
    __shared__ unsigned win[kBitWin][kBitQ / 32];
    const int chunks = (w.M + kBitQ - 1) / kBitQ;
    const int bg = blockIdx.x / chunks, chunk = blockIdx.x - bg * chunks;
    const int b = bg / w.G, g = bg - b * w.G;
    const int tid = threadIdx.x;
    const int m0 = chunk * kBitQ;
    const int m = m0 + tid;
    const bool live = m < w.M;
    const int cmax = min((min(m0 + kBitQ, w.M) - 1) / w.bs, w.NB - 1);
    const int cm = live ? m / w.bs : -1;
    const int32_t *row = w.idx + ((size_t)(b * (size_t)w.M + (live ? m : m0)) * w.G + g) * w.T;
    const int w0 = chunk * (kBitQ / 32);
    for (int t0 = 0; t0 <= cmax; t0 += kBitWin) {
        const int nrows = min(kBitWin, cmax + 1 - t0);
        for (int e = tid; e < nrows * (kBitQ / 32); e += kBitQ) win[e / (kBitQ / 32)][e % (kBitQ / 32)] = 0u;
        __syncthreads();
        if (live) {
            for (int j = 0; j < w.T; ++j) {
                const int t = row[j];
                if (t >= t0 && t < t0 + nrows && t <= cm) atomicOr(&win[t - t0][tid >> 5], 1u << (tid & 31));
            }
        }
        __syncthreads();
        for (int e = tid; e < nrows * (kBitQ / 32); e += kBitQ) {
            const int tr = e / (kBitQ / 32), wi = e % (kBitQ / 32);
            if (w0 + wi < w.MW) w.bits[((size_t)bg * w.NB + t0 + tr) * w.MW + w0 + wi] = win[tr][wi];
        }
        __syncthreads();
    }
}

// Per key-block row: number of selecting queries, cut into items of qc; the
// first query of item k is the one of rank k*qc.  One wavefront per row.
__global__ __launch_bounds__(256) void nsa_sel_bwd_count_kernel(Bw w) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (row >= w.R) return;
    const int t = row % w.NB;
    const unsigned *bits = w.bits + (size_t)row * w.MW;
    int total = 0;
    for (int wb = t * w.bs / 32; wb < w.MW; wb += kWaveSize) {
        const int wi = wb + lane;
        const unsigned word = wi < w.MW ? bits[wi] : 0u;
        const int pc = __popc(word);
        const int incl = wave_incl_scan(pc, lane);
        const int lo = total + incl - pc, hi = total + incl;
        const int k = (lo + w.qc - 1) / w.qc;  // qc >= 32: at most one item starts in a word
        if (pc > 0 && k * w.qc < hi && k < w.kmax)
            w.starts[(size_t)row * w.kmax + k] = 32 * wi + nth_bit(word, k * w.qc - lo);
        total += __shfl(incl, kWaveSize - 1, kWaveSize);
    }
    if (lane == 0) w.row_items[row] = (total + w.qc - 1) / w.qc;
}

// Exclusive scans of the item counts (item list) and of the counts of rows
// with two or more items (partial slots); one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void nsa_sel_bwd_scan_kernel(Bw w) {
    __shared__ int wsum[2][16];
    const int tid = threadIdx.x, lane = tid & (kWaveSize - 1), wave = tid >> 6;
    int carry_i = 0, carry_p = 0;
    for (int base = 0; base < w.R; base += 1024) {
        const int row = base + tid;
        const int n = row < w.R ? w.row_items[row] : 0;
        const int np = n >= 2 ? n : 0;
        const int si = wave_incl_scan(n, lane), sp = wave_incl_scan(np, lane);
        if (lane == kWaveSize - 1) {
            wsum[0][wave] = si;
            wsum[1][wave] = sp;
        }
        __syncthreads();
        int off_i = carry_i, off_p = carry_p, tot_i = 0, tot_p = 0;
        for (int v = 0; v < 16; ++v) {
            const int a = wsum[0][v], c = wsum[1][v];
            if (v < wave) {
                off_i += a;
                off_p += c;
            }
            tot_i += a;
            tot_p += c;
        }
        off_i += si - n;
        off_p += sp - np;
        if (row < w.R) {
            w.row_first[row] = off_i;
            w.row_part[row] = off_p;
            for (int k = 0; k < n; ++k)
                if (off_i + k < w.cap) w.items[off_i + k] = make_int2(row, k);
        }
        carry_i += tot_i;
        carry_p += tot_p;
        __syncthreads();
    }
    if (tid == 0) {
        w.n_items[0] = min(carry_i, w.cap);
        // The plan bounds both from the sizes alone, so this stays 0; were a
        // bound ever wrong, the caller reads the flag instead of getting
        // silently clamped gradients.
        w.n_items[1] = (carry_i > w.cap || carry_p > w.pcap) ? 1 : 0;
        w.rowstat[w.sentinel] = make_float2(INFINITY, 0.f);
    }
}

typedef __attribute__((address_space(3))) _Float16 lds_half_t;

__device__ __forceinline__ unsigned lds_addr(const void *p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) char *)p;
}

// LDS reads issued as inline asm with their own lgkmcnt wait: the compiler
// would otherwise guard them with vmcnt(0), waiting for every copy in flight.
__device__ __forceinline__ int lds_read_int(unsigned a) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}

// The dK/dV pass's LDS reads of one tile at D = 128, as two batches with one
// wait each: (1) the Q and dO row fragments (MFMA A operands, the layout of
// Stage::read) and the 8 rows' statistics of this lane, (2) the transposed
// dO^T and Q^T fragments (the layout of Stage::read_vt).  aq/ad are the
// lane's addresses of head-dim chunk c in the Q and dO tiles (row part
// included), ast the lane's statistics address; tq/td the transposing-read
// addresses.
__device__ __forceinline__ void tile_rows128(half8 (&qa)[2][4], half8 (&da)[2][4], float4v (&sa)[2][2],
                                             const unsigned (&aq)[4], const unsigned (&ad)[4], unsigned ast) {
    asm volatile(
        "ds_read_b128 %0, %20 offset:0\n" "ds_read_b128 %1, %21 offset:0\n" "ds_read_b128 %2, %22 offset:0\n"
        "ds_read_b128 %3, %23 offset:0\n" "ds_read_b128 %4, %20 offset:4096\n" "ds_read_b128 %5, %21 offset:4096\n"
        "ds_read_b128 %6, %22 offset:4096\n" "ds_read_b128 %7, %23 offset:4096\n" "ds_read_b128 %8, %24 offset:0\n"
        "ds_read_b128 %9, %25 offset:0\n" "ds_read_b128 %10, %26 offset:0\n" "ds_read_b128 %11, %27 offset:0\n"
        "ds_read_b128 %12, %24 offset:4096\n" "ds_read_b128 %13, %25 offset:4096\n"
        "ds_read_b128 %14, %26 offset:4096\n" "ds_read_b128 %15, %27 offset:4096\n"
        "ds_read_b128 %16, %28 offset:0\n" "ds_read_b128 %17, %28 offset:16\n" "ds_read_b128 %18, %28 offset:128\n"
        "ds_read_b128 %19, %28 offset:144\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(qa[0][0]), "=&v"(qa[0][1]), "=&v"(qa[0][2]), "=&v"(qa[0][3]), "=&v"(qa[1][0]), "=&v"(qa[1][1]),
          "=&v"(qa[1][2]), "=&v"(qa[1][3]), "=&v"(da[0][0]), "=&v"(da[0][1]), "=&v"(da[0][2]), "=&v"(da[0][3]),
          "=&v"(da[1][0]), "=&v"(da[1][1]), "=&v"(da[1][2]), "=&v"(da[1][3]), "=&v"(sa[0][0]), "=&v"(sa[0][1]),
          "=&v"(sa[1][0]), "=&v"(sa[1][1])
        : "v"(aq[0]), "v"(aq[1]), "v"(aq[2]), "v"(aq[3]), "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ast)
        : "memory");
}

__device__ __forceinline__ void tile_tr128(half4 (&dt)[1][4][2][2], half4 (&qt)[1][4][2][2], const unsigned (&td)[4],
                                           const unsigned (&tq)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %32 offset:0\n" "ds_read_b64_tr_b16 %1, %32 offset:4096\n"
        "ds_read_b64_tr_b16 %2, %32 offset:8\n" "ds_read_b64_tr_b16 %3, %32 offset:4104\n"
        "ds_read_b64_tr_b16 %4, %33 offset:0\n" "ds_read_b64_tr_b16 %5, %33 offset:4096\n"
        "ds_read_b64_tr_b16 %6, %33 offset:8\n" "ds_read_b64_tr_b16 %7, %33 offset:4104\n"
        "ds_read_b64_tr_b16 %8, %34 offset:0\n" "ds_read_b64_tr_b16 %9, %34 offset:4096\n"
        "ds_read_b64_tr_b16 %10, %34 offset:8\n" "ds_read_b64_tr_b16 %11, %34 offset:4104\n"
        "ds_read_b64_tr_b16 %12, %35 offset:0\n" "ds_read_b64_tr_b16 %13, %35 offset:4096\n"
        "ds_read_b64_tr_b16 %14, %35 offset:8\n" "ds_read_b64_tr_b16 %15, %35 offset:4104\n"
        "ds_read_b64_tr_b16 %16, %36 offset:0\n" "ds_read_b64_tr_b16 %17, %36 offset:4096\n"
        "ds_read_b64_tr_b16 %18, %36 offset:8\n" "ds_read_b64_tr_b16 %19, %36 offset:4104\n"
        "ds_read_b64_tr_b16 %20, %37 offset:0\n" "ds_read_b64_tr_b16 %21, %37 offset:4096\n"
        "ds_read_b64_tr_b16 %22, %37 offset:8\n" "ds_read_b64_tr_b16 %23, %37 offset:4104\n"
        "ds_read_b64_tr_b16 %24, %38 offset:0\n" "ds_read_b64_tr_b16 %25, %38 offset:4096\n"
        "ds_read_b64_tr_b16 %26, %38 offset:8\n" "ds_read_b64_tr_b16 %27, %38 offset:4104\n"
        "ds_read_b64_tr_b16 %28, %39 offset:0\n" "ds_read_b64_tr_b16 %29, %39 offset:4096\n"
        "ds_read_b64_tr_b16 %30, %39 offset:8\n" "ds_read_b64_tr_b16 %31, %39 offset:4104\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(dt[0][0][0][0]), "=&v"(dt[0][0][0][1]), "=&v"(dt[0][0][1][0]), "=&v"(dt[0][0][1][1]),
          "=&v"(dt[0][1][0][0]), "=&v"(dt[0][1][0][1]), "=&v"(dt[0][1][1][0]), "=&v"(dt[0][1][1][1]),
          "=&v"(dt[0][2][0][0]), "=&v"(dt[0][2][0][1]), "=&v"(dt[0][2][1][0]), "=&v"(dt[0][2][1][1]),
          "=&v"(dt[0][3][0][0]), "=&v"(dt[0][3][0][1]), "=&v"(dt[0][3][1][0]), "=&v"(dt[0][3][1][1]),
          "=&v"(qt[0][0][0][0]), "=&v"(qt[0][0][0][1]), "=&v"(qt[0][0][1][0]), "=&v"(qt[0][0][1][1]),
          "=&v"(qt[0][1][0][0]), "=&v"(qt[0][1][0][1]), "=&v"(qt[0][1][1][0]), "=&v"(qt[0][1][1][1]),
          "=&v"(qt[0][2][0][0]), "=&v"(qt[0][2][0][1]), "=&v"(qt[0][2][1][0]), "=&v"(qt[0][2][1][1]),
          "=&v"(qt[0][3][0][0]), "=&v"(qt[0][3][0][1]), "=&v"(qt[0][3][1][0]), "=&v"(qt[0][3][1][1])
        : "v"(td[0]), "v"(td[1]), "v"(td[2]), "v"(td[3]), "v"(tq[0]), "v"(tq[1]), "v"(tq[2]), "v"(tq[3])
        : "memory");
}

template <int BS, int D>
struct KvLds {
    _Float16 q[kRing][kRows * D];
    _Float16 d[kRing][kRows * D];
    float st[kRing][BS / 16][2 * kRows];
    int list[kMaxQc];
    int nq;
};

// dK/dV of one item: key block (b, g, t), queries of rank k*qc .. k*qc+qc-1
// among those that selected it.  Wavefront v owns keys t*BS + 16v .. +15.
template <int BS, int D>
__global__ __launch_bounds__(kWaveSize * (BS / 16)) void nsa_sel_bwd_dkv_kernel(Bw w) {
    constexpr int WAVES = BS / 16;
    constexpr int DC = D / 32;
    using St = Stage<kRows, D>;
    constexpr int NI = St::NI;  // copy instructions per tile and tensor
    static_assert(NI % WAVES == 0, "copy instructions must split evenly");
    constexpr int CPW = NI / WAVES;     // per wavefront, per tensor
    constexpr int IPW = 2 * CPW + 1;    // per wavefront and tile, with the row statistics
    __shared__ __attribute__((aligned(16))) KvLds<BS, D> L;

    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Items in launch order, so the XCDs (workgroup w runs on XCD w % 8)
    // share a window of the (b, g)-major item list: one group's Q and dO rows
    // at a time, instead of every group's at once.
    const int n_items = *w.n_items;
    const int item = blockIdx.x;
    if (item >= n_items) return;  // the whole workgroup
    const int2 it = w.items[item];
    const int row = it.x, k = it.y;
    const int bg = row / w.NB, t = row - bg * w.NB;
    const int b = bg / w.G, g = bg - b * w.G;
    const int row_n = w.row_items[row];
    const int m_lo = w.starts[(size_t)row * w.kmax + k];
    const int m_hi = k + 1 < row_n ? w.starts[(size_t)row * w.kmax + k + 1] : w.M;

    // The item's queries, ascending, into LDS (wavefront 0).
    if (wave == 0) {
        const unsigned *bits = w.bits + (size_t)row * w.MW;
        const int wlo = m_lo >> 5, whi = (m_hi - 1) >> 5;
        int cnt = 0;
        for (int wb = wlo; wb <= whi; wb += kWaveSize) {
            const int wi = wb + lane;
            unsigned word = wi <= whi ? bits[wi] : 0u;
            if (wi == wlo) word &= ~0u << (m_lo & 31);
            if (wi == whi && (m_hi & 31)) word &= (1u << (m_hi & 31)) - 1u;
            const int pc = __popc(word);
            const int incl = wave_incl_scan(pc, lane);
            int pos = cnt + incl - pc;
            while (word) {
                if (pos < kMaxQc) L.list[pos] = 32 * wi + __builtin_ctz(word);
                ++pos;
                word &= word - 1u;
            }
            cnt += __shfl(incl, kWaveSize - 1, kWaveSize);
        }
        if (lane == 0) L.nq = min(cnt, kMaxQc);
    }
    __syncthreads();
    const int nq = L.nq;

    // This wavefront's keys: K and V fragments as MFMA B operands (lane l:
    // key key0 + l%16, head dims 32*c + 8*(l/16) .. +7); keys past N are
    // clamped here and masked below.
    const int r = lane & 15, q4 = lane >> 4;
    const int key0 = t * BS + wave * 16;
    const int my_key = key0 + r;
    half8 kb[DC], vb[DC];
    {
        const size_t kr = ((size_t)(b * (size_t)w.N + min(my_key, w.N - 1)) * w.G + g) * D;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            kb[c] = *(const half8 *)(w.K + kr + c * 32 + q4 * 8);
            vb[c] = *(const half8 *)(w.V + kr + c * 32 + q4 * 8);
        }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // fragments in registers before the copies start counting

    // Rows whose query precedes the key block's last key need the causal
    // mask; they are queries of the block itself (at most BS - 1), hence
    // among the first 64 of the ascending list.  A tile needs the mask when
    // it starts before them or the wavefront's keys reach past N.
    int n_early;
    {
        const int mv = lane < nq ? lds_read_int(lds_addr(L.list) + 4u * (unsigned)lane) : INT_MAX;
        n_early = __builtin_popcountll(__ballot(mv < t * BS + BS - 1));
    }
    const bool tail_keys = key0 + 16 > w.N;

    const int h0 = g * w.gs;
    const int qpt = w.qpt;
    const int ntiles = (nq + qpt - 1) / qpt;
    const size_t qb = (size_t)b * w.M * w.H * D;
    const unsigned q_bytes = (unsigned)((size_t)w.M * w.H * D * 2);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void *)(w.Q + qb), (short)0, (int)q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rd =
        __builtin_amdgcn_make_buffer_rsrc((void *)(w.dO + qb), (short)0, (int)q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)w.rowstat, (short)0, (int)((unsigned)(w.sentinel + 1) * 8u), 0x00020000);
    const unsigned list_a = lds_addr(L.list);

    // Row rr of tile i: query slot rr / gs, head rr % gs; rows past the
    // item's queries (or past qpt * gs) are padding.
    auto row_query = [&](int i, int rr, int &m, int &h) -> bool {
        const int slot = rr / w.gs;
        const int qi = i * qpt + slot;
        const bool valid = slot < qpt && qi < nq;
        m = lds_read_int(list_a + 4u * (unsigned)(valid ? qi : 0));
        h = h0 + (valid ? rr - slot * w.gs : 0);
        return valid;
    };
    auto issue = [&](int i) {
        const int slot = i % kRing;
        // The rows' queries: CPW copy rows and one statistics row per lane,
        // read from the list with one LDS wait.
        unsigned la[5];
        int rrs[5], hs[5], ms[5];
        bool vs[5];
#pragma unroll
        for (int kk = 0; kk < 5; ++kk) {
            const int rr = kk < CPW ? (wave + kk * WAVES) * St::RPI + lane / St::LPR : lane >> 1;
            const int sl = rr / w.gs;
            const int qi = i * qpt + sl;
            vs[kk] = kk <= CPW && sl < qpt && qi < nq;
            la[kk] = list_a + 4u * (unsigned)(vs[kk] ? qi : 0);
            hs[kk] = h0 + (vs[kk] ? rr - sl * w.gs : 0);
            rrs[kk] = rr;
        }
        asm volatile("ds_read_b32 %0, %5\n\tds_read_b32 %1, %6\n\tds_read_b32 %2, %7\n\tds_read_b32 %3, %8\n\t"
                     "ds_read_b32 %4, %9\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(ms[0]), "=&v"(ms[1]), "=&v"(ms[2]), "=&v"(ms[3]), "=&v"(ms[4])
                     : "v"(la[0]), "v"(la[1]), "v"(la[2]), "v"(la[3]), "v"(la[4])
                     : "memory");
#pragma unroll
        for (int kk = 0; kk < CPW; ++kk) {
            const int j = wave + kk * WAVES;
            const unsigned off = (unsigned)(((size_t)ms[kk] * w.H + hs[kk]) * D * 2) +
                                 (unsigned)(((lane % St::LPR) ^ St::swz(rrs[kk])) * 16);
            St::copy(rq, (lds_half_t *)L.q[slot], off, 0u, j);
            St::copy(rd, (lds_half_t *)L.d[slot], off, 0u, j);
        }
        {
            const int m = ms[CPW], h = hs[CPW];
            const bool valid = vs[CPW];
            const unsigned e = valid ? (unsigned)(((size_t)b * w.H + h) * w.M + m) : (unsigned)w.sentinel;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)L.st[slot][wave],
                                                     4, e * 8u + (unsigned)(lane & 1) * 4u, 0, 0, 0);
        }
    };

    // The lane's LDS byte offsets within a staged tile: row fragments (row r,
    // head-dim chunk c) and transposing reads (row 4*(l/16) + (l/4)%4, piece
    // 4*c + l%4), with the staging swizzle.
    unsigned row_off[DC], tr_off[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        row_off[c] = (unsigned)(r * D + ((c * 4 + q4) ^ St::swz(r)) * 8) * 2u;
        const int trow = 4 * q4 + ((lane >> 2) & 3);
        tr_off[c] = (unsigned)(trow * D * 2 + ((4 * c + (lane & 3)) ^ St::swz(trow)) * 16);
    }

    float4v dk[DC][2], dv[DC][2];
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            dk[c][hh] = float4v{0.f, 0.f, 0.f, 0.f};
            dv[c][hh] = float4v{0.f, 0.f, 0.f, 0.f};
        }

#pragma unroll
    for (int i = 0; i < kRing - 1; ++i)
        if (i < ntiles) issue(i);

    for (int i = 0; i < ntiles; ++i) {
        // Own copies of tile i landed, then everyone's; the slot of tile i-1
        // is free once all wavefronts passed the barrier.
        if (i + kRing - 2 < ntiles)
            __builtin_amdgcn_s_waitcnt(wait_vm(IPW * (kRing - 2)));
        else
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
        lds_barrier();
        if (i + kRing - 1 < ntiles) issue(i + kRing - 1);
        const int slot = i % kRing;

        half8 qa[2][DC], da[2][DC];
        float4v sa[2][2];  // (LSE log2 e, Delta) of rows 16*rt + 4*(l/16) + j
        const unsigned st_a = lds_addr(L.st[slot][wave]) + (unsigned)(q4 * 4 * 8);
        if constexpr (D == 128) {
            const unsigned qb = lds_addr(L.q[slot]), db = lds_addr(L.d[slot]);
            unsigned aq[4], ad[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                aq[c] = qb + row_off[c];
                ad[c] = db + row_off[c];
            }
            tile_rows128(qa, da, sa, aq, ad, st_a);
        } else {
            St::read(qa, L.q[slot], r, q4);
            St::read(da, L.d[slot], r, q4);
            asm volatile(
                "ds_read_b128 %0, %4 offset:0\n"
                "ds_read_b128 %1, %4 offset:16\n"
                "ds_read_b128 %2, %4 offset:128\n"
                "ds_read_b128 %3, %4 offset:144\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(sa[0][0]), "=&v"(sa[0][1]), "=&v"(sa[1][0]), "=&v"(sa[1][1])
                : "v"(st_a)
                : "memory");
        }
        // S = Q K^T and dP = dO V^T: lane l holds rows 16*rt + 4*(l/16) + j
        // of key my_key.
        float4v s[2], dp[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            s[rt] = float4v{0.f, 0.f, 0.f, 0.f};
            dp[rt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                s[rt] = mfma_16x16x32(qa[rt][c], kb[c], s[rt]);
                dp[rt] = mfma_16x16x32(da[rt][c], vb[c], dp[rt]);
            }
        }
        const bool need_mask = tail_keys || i * qpt < n_early;
        half4 pf[2], dsf[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float4v pv, ds;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lse2 = sa[rt][j >> 1][(j & 1) * 2];
                const float delta = sa[rt][j >> 1][(j & 1) * 2 + 1];
                float pj = fast_exp2(__builtin_fmaf(s[rt][j], w.scale_log2, -lse2));
                if (need_mask) {
                    int m, h;
                    const bool valid = row_query(i, 16 * rt + 4 * q4 + j, m, h);
                    if (!valid || my_key > min(m, w.N - 1)) pj = 0.f;
                }
                pv[j] = pj;
                ds[j] = pj * (dp[rt][j] - delta);
            }
            pf[rt] = to_half4(pv);
            dsf[rt] = to_half4(ds);
        }
        // dV^T += dO^T P and dK^T += Q^T dS (rows of the tile on the MFMA k
        // axis, in the order of the transposing reads).
        half4 qt[1][DC][2][2], dt[1][DC][2][2];
        if constexpr (D == 128) {
            const unsigned qb = lds_addr(L.q[slot]), db = lds_addr(L.d[slot]);
            unsigned td[4], tq[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                td[c] = db + tr_off[c];
                tq[c] = qb + tr_off[c];
            }
            tile_tr128(dt, qt, td, tq);
        } else {
            St::read_vt(dt, L.d[slot], lane);
            St::read_vt(qt, L.q[slot], lane);
        }
        const half8 bp = cat8(pf[0], pf[1]);
        const half8 bds = cat8(dsf[0], dsf[1]);
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                dv[c][hh] = mfma_16x16x32(cat8(dt[0][c][hh][0], dt[0][c][hh][1]), bp, dv[c][hh]);
                dk[c][hh] = mfma_16x16x32(cat8(qt[0][c][hh][0], qt[0][c][hh][1]), bds, dk[c][hh]);
            }
    }

    // Lane l holds dK^T, dV^T rows d = 32*c + 8*(l/16) + 4*hh + i of key
    // my_key: straight to the outputs when the item is the key block's only
    // one, else to the item's partial slot.
    if (my_key < w.N) {
        float *pk, *pv;
        if (row_n == 1) {
            const size_t o = ((size_t)(b * (size_t)w.N + my_key) * w.G + g) * D;
            pk = w.dK + o;
            pv = w.dV + o;
        } else {
            const int psi = w.row_part[row] + k;  // < pcap by the plan's bound (else the overflow flag is set)
            const size_t ps = (size_t)(psi < w.pcap ? psi : w.pcap - 1);
            pk = w.part + ((ps * 2 + 0) * BS + (my_key - t * BS)) * D;
            pv = w.part + ((ps * 2 + 1) * BS + (my_key - t * BS)) * D;
        }
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            __builtin_nontemporal_store(dk[c][0] * w.scale, (float4v *)(pk + c * 32 + q4 * 8));
            __builtin_nontemporal_store(dk[c][1] * w.scale, (float4v *)(pk + c * 32 + q4 * 8 + 4));
            __builtin_nontemporal_store(dv[c][0], (float4v *)(pv + c * 32 + q4 * 8));
            __builtin_nontemporal_store(dv[c][1], (float4v *)(pv + c * 32 + q4 * 8 + 4));
        }
    }
}

// Key blocks with no item get zeros; those with several items the sum of
// their partials in item order.  kReduceSlices workgroups per key block row
// (grid y), each thread holding EPT float4 sums whose loads for one partial
// (and the next) are issued together, so a thread keeps 2 * EPT loads in
// flight instead of one.  The additions follow the item order, so the result
// does not depend on the launch shape.
constexpr int kReduceSlices = 4;

template <int BS, int D>
__global__ __launch_bounds__(256) void nsa_sel_bwd_reduce_kernel(Bw w) {
    const int row = blockIdx.x;
    const int slice = blockIdx.y;
    const int n = w.row_items[row];
    if (n == 1) return;
    const int bg = row / w.NB, t = row - bg * w.NB;
    const int b = bg / w.G, g = bg - b * w.G;
    const int p0 = n >= 2 ? w.row_part[row] : 0;
    if (p0 + n > w.pcap) return;  // the plan bounds the partial slots; the scan flags an overflow
    constexpr int V4 = BS * D / 4;  // float4 per tensor; a partial holds dK then dV
    constexpr int EPT = 2 * V4 / (kReduceSlices * 256);
    static_assert(EPT >= 1 && (2 * V4) % (kReduceSlices * 256) == 0, "slices must split the row evenly");
    const float4v *src = (const float4v *)w.part + (size_t)p0 * 2 * V4;
    int e[EPT];
    float4v acc[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        e[i] = (slice * EPT + i) * 256 + (int)threadIdx.x;
        acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
    }
    int j = 0;
    for (; j + 1 < n; j += 2) {
        float4v x[EPT], y[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            x[i] = __builtin_nontemporal_load(src + (size_t)j * 2 * V4 + e[i]);
            y[i] = __builtin_nontemporal_load(src + (size_t)(j + 1) * 2 * V4 + e[i]);
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            acc[i] += x[i];
            acc[i] += y[i];
        }
    }
    if (j < n) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) acc[i] += __builtin_nontemporal_load(src + (size_t)j * 2 * V4 + e[i]);
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int tensor = e[i] / V4, f = e[i] - tensor * V4;
        const int key = f / (D / 4), d4 = f - key * (D / 4);
        const int na = t * BS + key;
        if (na >= w.N) continue;
        float *dst = (tensor ? w.dV : w.dK) + ((size_t)(b * (size_t)w.N + na) * w.G + g) * D;
        __builtin_nontemporal_store(acc[i], (float4v *)dst + d4);
    }
}

// ---------------------------------------------------------------------------
// Device address of this GPU's scratch array, or NULL if the runtime could
// not give it.  The first call on each device asks the runtime; later calls
// reuse the stored address.
void *scratch_address() {
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

// ---------------------------------------------------------------------------
// Host-side planning.

struct BwdPlan {
    int NB, MW, R, qc, kmax, qpt;
    int64_t cap, pcap;
    size_t off_rowstat, off_bits, off_row_items, off_row_first, off_row_part, off_starts, off_items, off_nitems,
        off_part, off_sched, total;
    int64_t sched_words;  // schedule of the persistent dQ pass
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sizes of the workspace for (B, M, N, H, G, D, bs, T) on a device of
// topology tp; p must hold the checked sizes and is planned in place
// (plan_slots: the dQ pass's slots, whose persistent schedule the workspace
// holds).  Returns NSA_SEL_OK or NSA_SEL_ERR_RANGE.
int bwd_plan(Params &p, const Topology &tp, int D, int bs, BwdPlan &pl) {
    plan_slots(p, tp);
    pl.sched_words = sched_words_bound(p, tp.cus);
    if (pl.sched_words > INT_MAX) return NSA_SEL_ERR_RANGE;
    pl.NB = p.NB;
    pl.MW = (p.M + 31) / 32;
    const int64_t R = (int64_t)p.B * p.G * p.NB;
    if (R > INT_MAX) return NSA_SEL_ERR_RANGE;
    pl.R = (int)R;
    int qc = (8192 / p.gs) / 32 * 32;
    qc = qc < 32 ? 32 : qc > kMaxQc ? kMaxQc : qc;
    pl.qc = qc;
    pl.kmax = (p.M + qc - 1) / qc;
    pl.qpt = kRows / p.gs;
    // Distinct (query, block) pairs per (b, g): query m counts at most
    // min(T, m / bs + 1, NB) blocks.
    int64_t pairs = 0;
    for (int64_t c = 0; c * bs < p.M; ++c) {
        const int64_t nqc = std::min<int64_t>(bs, p.M - c * bs);
        pairs += nqc * std::min<int64_t>(std::min<int64_t>(p.T, c + 1), p.NB);
    }
    const int64_t bgs = (int64_t)p.B * p.G;
    pl.cap = bgs * (p.NB + (pairs + qc - 1) / qc);
    pl.pcap = bgs * ((2 * pairs + qc - 1) / qc) + 1;
    if (pl.cap > INT_MAX || pl.pcap > INT_MAX || R * pl.kmax > INT_MAX) return NSA_SEL_ERR_RANGE;
    const int64_t rows = (int64_t)p.B * p.H * p.M;
    if (rows + 1 > (int64_t)1 << 28) return NSA_SEL_ERR_RANGE;          // rowstat byte offsets in 32 bits
    if ((int64_t)p.M * p.H * D * 2 > (int64_t)UINT_MAX) return NSA_SEL_ERR_RANGE;  // Q / dO offsets of one batch
    size_t o = 0;
    pl.off_nitems = o;  // bytes 0..3 item count, 4..7 overflow flag (documented in the header)
    o = align256(o + 8);
    pl.off_rowstat = o;
    o = align256(o + (size_t)(rows + 1) * 8);
    pl.off_bits = o;
    o = align256(o + (size_t)R * pl.MW * 4);
    pl.off_row_items = o;
    o = align256(o + (size_t)R * 4);
    pl.off_row_first = o;
    o = align256(o + (size_t)R * 4);
    pl.off_row_part = o;
    o = align256(o + (size_t)R * 4);
    pl.off_starts = o;
    o = align256(o + (size_t)R * pl.kmax * 4);
    pl.off_items = o;
    o = align256(o + (size_t)pl.cap * 8);
    pl.off_part = o;
    o = align256(o + (size_t)pl.pcap * 2 * bs * D * 4);
    pl.off_sched = o;
    o = align256(o + (size_t)pl.sched_words * 4);
    pl.total = o;
    return NSA_SEL_OK;
}

template <int BS, int D>
hipError_t launch_key_passes(const Bw &w, const BwdPlan &pl, hipStream_t stream) {
    const int chunks = (w.M + kBitQ - 1) / kBitQ;
    hipLaunchKernelGGL(nsa_sel_bwd_bitmap_kernel, dim3(w.B * w.G * chunks), dim3(kBitQ), 0, stream, w);
    hipLaunchKernelGGL(nsa_sel_bwd_count_kernel, dim3((w.R + 3) / 4), dim3(256), 0, stream, w);
    hipLaunchKernelGGL(nsa_sel_bwd_scan_kernel, dim3(1), dim3(1024), 0, stream, w);
    const int per_xcd = (int)((pl.cap + w.nxcd - 1) / w.nxcd);
    hipLaunchKernelGGL((nsa_sel_bwd_dkv_kernel<BS, D>), dim3(per_xcd * w.nxcd), dim3(kWaveSize * (BS / 16)), 0,
                       stream, w);
    hipLaunchKernelGGL((nsa_sel_bwd_reduce_kernel<BS, D>), dim3(w.R, kReduceSlices), dim3(256), 0, stream, w);
    return hipGetLastError();
}

}  // namespace

extern "C" int nsa_sel_bwd_workspace_size(int B, int M, int N, int H, int G, int D, int block_size, int T,
                                          size_t *bytes) {
    if (!bytes) return NSA_SEL_ERR_NULL;
    Params p;
    const int st = check_sizes(B, M, N, H, G, D, block_size, T, p);
    if (st != NSA_SEL_OK) return st;
    BwdPlan pl;
    const int st2 = bwd_plan(p, device_topology(), D, block_size, pl);
    if (st2 != NSA_SEL_OK) return st2;
    *bytes = pl.total;
    return NSA_SEL_OK;
}

namespace {

// The backward with its arguments checked against the workspace of
// workspace_bytes at `workspace`.  noalloc: the workspace is the library's own
// scratch array (a short one is then NSA_SEL_ERR_SCRATCH; it is looked up only
// after every other check has passed).
int sel_bwd(const void *Q, const void *K, const void *V, const int32_t *block_indices, const void *O,
            const float *LSE, const void *dO, float *dQ, float *dK, float *dV, void *workspace,
            size_t workspace_bytes, int B, int M, int N, int H, int G, int D, int block_size, int T,
            hipStream_t stream, bool noalloc) {
    if (!Q || !K || !V || !block_indices || !O || !LSE || !dO || !dQ || !dK || !dV) return NSA_SEL_ERR_NULL;
    Params p;
    const int st = check_sizes(B, M, N, H, G, D, block_size, T, p);
    if (st != NSA_SEL_OK) return st;
    const Topology tp = device_topology();
    BwdPlan pl;
    const int st2 = bwd_plan(p, tp, D, block_size, pl);
    if (st2 != NSA_SEL_OK) return st2;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O | (uintptr_t)dO | (uintptr_t)dQ |
         (uintptr_t)dK | (uintptr_t)dV) & 15)
        return NSA_SEL_ERR_ALIGN;
    if (((uintptr_t)block_indices | (uintptr_t)LSE) & 3) return NSA_SEL_ERR_ALIGN;
    if (noalloc) {
        if (pl.total > workspace_bytes) return NSA_SEL_ERR_SCRATCH;
        workspace = scratch_address();
        if (!workspace) return NSA_SEL_ERR_HIP;
    }
    if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < pl.total) return NSA_SEL_ERR_WORKSPACE;

    const size_t q_bytes = (size_t)B * M * H * D * 2, kv_bytes = (size_t)B * N * G * D * 2;
    const size_t idx_bytes = (size_t)B * M * G * T * 4, lse_bytes = (size_t)B * H * M * 4;
    const void *ins[7] = {Q, K, V, block_indices, O, LSE, dO};
    const size_t in_bytes[7] = {q_bytes, kv_bytes, kv_bytes, idx_bytes, q_bytes, lse_bytes, q_bytes};
    void *outs[4] = {dQ, dK, dV, workspace};
    const size_t out_bytes[4] = {q_bytes * 2, kv_bytes * 2, kv_bytes * 2, pl.total};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 7; ++i)
            if (ranges_overlap(outs[o], out_bytes[o], ins[i], in_bytes[i])) return NSA_SEL_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (ranges_overlap(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return NSA_SEL_ERR_ALIAS;
    }

    const int cus = tp.cus;
    p.Q = (const _Float16 *)Q;
    p.K = (const _Float16 *)K;
    p.V = (const _Float16 *)V;
    p.idx = block_indices;
    p.O = nullptr;
    p.LSE = nullptr;
    char *ws = (char *)workspace;
    p.sched = (unsigned *)(ws + pl.off_sched);
    p.sched_cap = (int)pl.sched_words;
    float2 *rowstat = (float2 *)(ws + pl.off_rowstat);
    DqKernel f;
    f.x.O = (const _Float16 *)O;
    f.x.dO = (const _Float16 *)dO;
    f.x.LSE = LSE;
    f.x.dQ = dQ;
    f.x.rowstat = rowstat;
    f.x.scale = 1.0f / sqrtf((float)D);

    Bw w;
    w.Q = (const _Float16 *)Q;
    w.K = (const _Float16 *)K;
    w.V = (const _Float16 *)V;
    w.dO = (const _Float16 *)dO;
    w.idx = block_indices;
    w.rowstat = rowstat;
    w.bits = (unsigned *)(ws + pl.off_bits);
    w.row_items = (int *)(ws + pl.off_row_items);
    w.row_first = (int *)(ws + pl.off_row_first);
    w.row_part = (int *)(ws + pl.off_row_part);
    w.starts = (int *)(ws + pl.off_starts);
    w.items = (int2 *)(ws + pl.off_items);
    w.n_items = (int *)(ws + pl.off_nitems);
    w.part = (float *)(ws + pl.off_part);
    w.dK = dK;
    w.dV = dV;
    w.B = B; w.M = M; w.N = N; w.H = H; w.G = G; w.gs = p.gs; w.T = T; w.bs = block_size;
    w.NB = pl.NB; w.MW = pl.MW; w.R = pl.R; w.qc = pl.qc; w.kmax = pl.kmax; w.cap = (int)pl.cap; w.pcap = (int)pl.pcap; w.qpt = pl.qpt;
    w.sentinel = B * H * M;
    w.nxcd = tp.nxcd;
    w.scale = 1.0f / sqrtf((float)D);
    w.scale_log2 = p.scale_log2;

    hipError_t e;
    if (block_size == 64)
        e = (D == 128) ? dq_launch_pack<64, 128>(f, p, cus, stream) : dq_launch_pack<64, 64>(f, p, cus, stream);
    else
        e = (D == 128) ? dq_launch_pack<32, 128>(f, p, cus, stream) : dq_launch_pack<32, 64>(f, p, cus, stream);
    if (e != hipSuccess) return NSA_SEL_ERR_HIP;
    if (block_size == 64)
        e = (D == 128) ? launch_key_passes<64, 128>(w, pl, stream) : launch_key_passes<64, 64>(w, pl, stream);
    else
        e = (D == 128) ? launch_key_passes<32, 128>(w, pl, stream) : launch_key_passes<32, 64>(w, pl, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}

}  // namespace

extern "C" int nsa_sel_bwd(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                           const void *O, const float *LSE, const void *dO, float *dQ, float *dK, float *dV,
                           void *workspace, size_t workspace_bytes, int B, int M, int N, int H, int G, int D,
                           int block_size, int T, hipStream_t stream) {
    return sel_bwd(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, B, M, N, H, G, D,
                   block_size, T, stream, false);
}

extern "C" int nsa_sel_bwd_noalloc(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                                   const void *O, const float *LSE, const void *dO, float *dQ, float *dK,
                                   float *dV, int B, int M, int N, int H, int G, int D, int block_size, int T,
                                   hipStream_t stream) {
    return sel_bwd(Q, K, V, block_indices, O, LSE, dO, dQ, dK, dV, nullptr, kScratchBytes, B, M, N, H, G, D,
                   block_size, T, stream, true);
}
