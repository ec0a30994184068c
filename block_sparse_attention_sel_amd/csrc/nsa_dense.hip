// Dense and sliding-window GQA attention forward for AMD MI355X (gfx950):
// the baseline the selection kernel is compared with, and the sliding-window
// variant (include/nsa_dense.h).
//
// Operation: every causal key of the query (n <= m, n < N) for all H/G heads
// of the group, one softmax, O and the natural-log LSE -- selection attention
// with every block selected (wave issue "[wave] NSA: selection attention
// forward kernel", section Performance target, names this dense attention as
// the reference point).  The window variant keeps the keys
// m - LEFT <= n <= m + RIGHT (the FlyDSL pull request "[Kernel][MI350] Add 8
// wave GQA sliding-window attention kernel", section What it does), a
// workgroup streaming only the key range its queries' windows cover; fp16 or
// bf16 operands.
//
// MI355X mapping.  The per-step math is the selection kernel's (transposed
// scores S^T = K Q^T on v_mfma_f32_16x16x32_f16 with P kept in registers as
// the PV B operand, lazy running max, V^T from ds_read_b64_tr_b16).  What
// changes is the sharing: a workgroup of 8 wavefronts (two per SIMD) carries
// 16 column tiles -- 16 * PACK consecutive queries of one (b, g) -- and all of
// them consume one stream of 32-key K/V sub-blocks, staged once per workgroup
// through a ring of kStages LDS buffers:
//   * each wavefront copies its share of every sub-block (1/8 of the K and V
//     copy instructions, 128-bit direct-to-LDS, coalesced rows);
//   * per group of 4 sub-blocks: wait for the own shares, one LDS barrier
//     (all shares in, the other half of the ring free), issue the next
//     group's copies (fewer barriers let the two wavefronts of a SIMD drift
//     out of phase, so one's softmax overlaps the other's MFMAs);
//   * runs of sub-blocks that no column masks are software-pipelined: the
//     step for sub-block s issues the PV products of s and the QK products of
//     s + 1 (both tiles) and then the softmax of s + 1, in one straight-line
//     block, so the softmax of the first tile runs beside the second tile's
//     QK products; sub-blocks at a window edge take a per-tile masked step;
//   * query tiles run longest first, and each XCD takes a contiguous range of
//     (b, g, tile) units, so the workgroups resident on an XCD sweep the same
//     group's keys.
#include "nsa_sel_common.h"
#include "nsa_dense.h"

namespace {

constexpr int kDenseWaves = 8;   // wavefronts per workgroup (two per SIMD)
constexpr int kDenseTiles = 2;   // 16-column tiles per wavefront
constexpr int kStages = 8;       // LDS ring of 32-key sub-blocks (128 KiB at D = 128)
constexpr int kGroup = 4;        // sub-blocks per LDS barrier: the ring holds two groups
constexpr int kDenseSbs = 32;

struct DenseParams {
    const _Float16 *Q;
    const _Float16 *K;
    const _Float16 *V;
    _Float16 *O;
    float *LSE;
    int B, M, N, H, G, gs;
    int qtiles;   // query tiles per (b, g)
    int units;    // B * G * qtiles
    int per_xcd;  // ceil(units / nxcd)
    int nxcd;     // XCDs workgroups are dealt to (w % nxcd)
    int left, right;  // window: keys m - left .. m + right visible (negative = unbounded)
    float scale_log2;
};

// The softmax step of score_block for a sub-block that no column masks and
// every column takes: the same arithmetic, on scores computed beforehand, so
// that one tile's softmax can be scheduled beside another tile's MFMAs.
template <int KT, bool BF16>
__device__ __forceinline__ void softmax_open(const float4v (&s)[KT], float scale_log2, float &m_run, float &l_run,
                                             float &alpha, half4 (&pf)[KT]) {
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) mloc = fmaxf(mloc, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
    mloc = col_max(mloc);
    const float m_blk = mloc * scale_log2;
    const float m_new = (m_blk > m_run + kLazyMax) ? m_blk : m_run;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        float4v pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = fast_exp2(__builtin_fmaf(s[kt][i], scale_log2, -m_use));
            psum += pv[i];
        }
        pf[kt] = pack4<BF16>(pv);
    }
    l_run = l_run * alpha + psum;
}

// softmax_open over a wavefront's NT tiles behind one wave-uniform test:
// when no lane's scaled scores exceed their column's running max by more
// than kLazyMax, every tile keeps its running max (alpha = 1) and P follows
// without the column reductions; otherwise (and on the first sub-block, where
// the running max is -inf) each tile takes softmax_open's full step.  Where
// the running max is kept both give the same P.
template <int NT, int KT, bool BF16>
__device__ __forceinline__ void softmax_open_tiles(const float4v (&s)[NT][KT], float scale_log2, float (&m_run)[NT],
                                                   float (&l_run)[NT], float (&alpha)[NT], half4 (&pf)[NT][KT]) {
    float x[NT][KT][4];
    // Ballots of plain compares, ORed on the scalar unit (one ballot of a
    // combined condition makes the compiler move it through a vector
    // register and back).
    uint64_t raise = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float xmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[nt][kt][i] = __builtin_fmaf(s[nt][kt][i], scale_log2, -m_run[nt]);
            xmax = fmaxf(xmax, fmaxf(fmaxf(x[nt][kt][0], x[nt][kt][1]), fmaxf(x[nt][kt][2], x[nt][kt][3])));
        }
        raise |= __builtin_amdgcn_ballot_w64(xmax > kLazyMax) | __builtin_amdgcn_ballot_w64(m_run[nt] == -INFINITY);
    }
    if (!raise) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float part[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                float4v pv;
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(x[nt][kt][i]);
                part[kt] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
                pf[nt][kt] = pack4<BF16>(pv);
            }
            float psum = part[0];
#pragma unroll
            for (int kt = 1; kt < KT; ++kt) psum += part[kt];
            alpha[nt] = 1.f;
            l_run[nt] += psum;
        }
        return;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) softmax_open<KT, BF16>(s[nt], scale_log2, m_run[nt], l_run[nt], alpha[nt], pf[nt]);
}

// accumulate_block split in two, so that the (rare) rescale branch can sit
// outside the straight-line step: the rescale by alpha, then PV.
template <int D>
__device__ __forceinline__ void rescale_acc(float4v (&acc)[D / 32][2], float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // wave-uniform: some column rescales
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            acc[c][0] *= alpha;
            acc[c][1] *= alpha;
        }
    }
}

template <int SBS, int D, bool BF16>
__device__ __forceinline__ void pv_tile(const half4 (&vt)[SBS / 32][D / 32][2][2], const half4 (&pf)[SBS / 16],
                                        float4v (&acc)[D / 32][2]) {
#pragma unroll
    for (int kc = 0; kc < SBS / 32; ++kc) {
        const half8 bp = cat8(pf[2 * kc], pf[2 * kc + 1]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                acc[c][hh] = mfma16<BF16>(cat8(vt[kc][c][hh][0], vt[kc][c][hh][1]), bp, acc[c][hh]);
    }
}

template <int D, int PACK, bool BF16>
__global__ __launch_bounds__(kWaveSize * kDenseWaves) void nsa_dense_kernel(DenseParams p) {
    constexpr int NT = kDenseTiles;
    constexpr int QWG = kDenseWaves * NT * PACK;  // queries per workgroup
    constexpr int SBS = kDenseSbs;
    constexpr int DC = D / 32;
    constexpr int KT = SBS / 16;
    constexpr int NI = Stage<SBS, D>::NI;              // copy instructions per K (or V) sub-block
    constexpr int IPW = (2 * NI) / kDenseWaves;        // of which each wavefront issues
    static_assert((2 * NI) % kDenseWaves == 0 && IPW >= 1, "copy instructions must split evenly");
    __shared__ __attribute__((aligned(16))) _Float16 kbuf[kStages][Stage<SBS, D>::HALVES];
    __shared__ __attribute__((aligned(16))) _Float16 vbuf[kStages][Stage<SBS, D>::HALVES];

    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = (blockIdx.x % p.nxcd) * p.per_xcd + (int)(blockIdx.x / p.nxcd);
    if (unit >= p.units) return;  // the whole workgroup
    const int bg = unit / p.qtiles;
    const int qt = p.qtiles - 1 - (unit - bg * p.qtiles);  // longest tiles first
    const int b = bg / p.G;
    const int g = bg % p.G;
    const int q0 = qt * QWG;
    const int q_last = min(q0 + QWG, p.M) - 1;
    const int r = lane & 15;
    const int q4 = lane >> 4;
    const int h0 = g * p.gs;
    const int q_in_tile = r / p.gs;
    const int my_h = h0 + (r - q_in_tile * p.gs);

    // Staging descriptors before the per-lane loads (keeps them scalar).
    Stage<SBS, D> st;
    {
        const int bb = __builtin_amdgcn_readfirstlane(b), gg = __builtin_amdgcn_readfirstlane(g);
        const size_t first = ((size_t)bb * p.N * p.G + gg) * D;
        const size_t bytes = ((size_t)p.B * p.N * p.G * D - first) * 2;
        st.init(p.K + first, p.V + first, (unsigned)(bytes < 0xFFFFFFFFu ? bytes : 0xFFFFFFFFu), p.G * D, p.N,
                lane);
    }

    // This wavefront's tiles: tile nt covers queries mt[nt] .. mt[nt]+PACK-1.
    bool live[NT];
    int my_m[NT], mt[NT];
    half8 qf[NT][DC];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        mt[nt] = q0 + (wave * NT + nt) * PACK;
        const int m = mt[nt] + q_in_tile;
        live[nt] = q_in_tile < PACK && m < p.M;
        my_m[nt] = live[nt] ? m : q0;
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

    // Keys any query of the workgroup sees: [k_lo, k_hi] (causal: 0 ..
    // min(N, q_last + 1) - 1); sub-blocks s_begin .. s_begin + nsub - 1.
    const int k_lo = p.left < 0 ? 0 : max(0, q0 - p.left);
    const int k_hi = p.right < 0 ? p.N - 1 : min(p.N - 1, q_last + p.right);
    const int s_begin = k_lo / SBS;
    const int nsub = k_hi < k_lo ? 0 : k_hi / SBS - s_begin + 1;
    // Each column's visible keys [c_lo[nt], c_hi[nt]].
    int c_lo[NT], c_hi[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        c_lo[nt] = p.left < 0 ? INT_MIN : my_m[nt] - p.left;
        c_hi[nt] = p.right < 0 ? p.N - 1 : min(my_m[nt] + p.right, p.N - 1);
    }
    auto issue = [&](int s) {
        const int slot = s % kStages;
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int j = wave + k * kDenseWaves;  // this wavefront's share of the 2*NI instructions
            if (j < NI)
                st.issue_part(st.rk, kbuf[slot], s_begin + s, j, lane);
            else
                st.issue_part(st.rv, vbuf[slot], s_begin + s, j - NI, lane);
        }
    };
#pragma unroll
    for (int s = 0; s < kGroup; ++s)
        if (s < nsub) issue(s);

    half8 kf[KT][DC];
    half4 vt[SBS / 32][DC][2][2];
    half4 pf[NT][KT];
    float4v sc[NT][KT];

    // Group barriers are passed lazily, in order, before the first read of a
    // sub-block of the group: this wavefront's copies of the group landed,
    // then everyone's (one LDS barrier), and everyone is done with the other
    // half of the ring, which is refilled with the next group.  Every
    // wavefront reads every sub-block, so all pass the same barriers.
    int bar_next = 0;
    auto ensure = [&](int t) {
        while (bar_next <= t / kGroup) {
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
            lds_barrier();
            const int first = (bar_next + 1) * kGroup;
#pragma unroll
            for (int k = 0; k < kGroup; ++k)
                if (first + k < nsub) issue(first + k);
            ++bar_next;
        }
    };
    // Per tile and sub-block (uniform over the tile): on = some key of the
    // sub-block lies in the union [t_lo, t_hi] of its queries' windows;
    // masked = some key lies outside some column's window (past the smallest
    // upper or before the largest lower bound).
    auto classify = [&](int s, bool (&on)[NT], bool (&masked)[NT]) {
        const int key0 = (s_begin + s) * SBS;
        bool open = true;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int tile_last = min(mt[nt] + PACK, p.M) - 1;
            const int t_lo = p.left < 0 ? 0 : mt[nt] - p.left;
            const int t_hi = p.right < 0 ? p.N - 1 : min(p.N - 1, tile_last + p.right);
            on[nt] = mt[nt] < p.M && key0 <= t_hi && key0 + SBS - 1 >= t_lo;
            const int min_hi = p.right < 0 ? p.N - 1 : min(p.N - 1, mt[nt] + p.right);
            masked[nt] = (key0 + SBS - 1 > min_hi) || (p.left >= 0 && key0 < tile_last - p.left);
            open = open && on[nt] && !masked[nt];
        }
        return open;  // every tile takes the whole sub-block unmasked
    };

    int s = 0;
    while (s < nsub) {
        bool on[NT], masked[NT];
        if (!classify(s, on, masked)) {
            // A sub-block at a window edge: per tile, with masks.
            ensure(s);
            const int slot = s % kStages;
            const int key0 = (s_begin + s) * SBS;
            Stage<SBS, D>::read(kf, kbuf[slot], r, q4);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (!on[nt]) continue;
                score_block<SBS, D, BF16>(kf, qf[nt], key0, masked[nt], true, live[nt], c_lo[nt], c_hi[nt],
                                          p.scale_log2, m_run[nt], l_run[nt], alpha[nt], pf[nt], q4);
            }
            Stage<SBS, D>::read_vt(vt, vbuf[slot], lane);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                if (on[nt]) accumulate_block<SBS, D, BF16>(vt, pf[nt], alpha[nt], acc[nt]);
            ++s;
            continue;
        }
        // A run of open sub-blocks, software-pipelined: the step for s issues
        // the QK products of s + 1 and the PV products of s beside the
        // softmax of s + 1, in one straight-line block; the rescale of the
        // accumulators (rare: the running max moves lazily) stays outside it.
        // Padding columns (fewer than 16 heads x queries in a tile) score
        // zero and carry finite values that are never stored; MFMA columns
        // do not mix.
        ensure(s);
        Stage<SBS, D>::read(kf, kbuf[s % kStages], r, q4);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) qk_tile<SBS, D, BF16>(kf, qf[nt], sc[nt]);
        softmax_open_tiles<NT, KT, BF16>(sc, p.scale_log2, m_run, l_run, alpha, pf);
        for (;;) {
            // V^T of s before the group barrier that may come with s + 1 (it
            // frees the half of the ring that holds s).
            Stage<SBS, D>::read_vt(vt, vbuf[s % kStages], lane);
            bool on1[NT], masked1[NT];
            const bool next = s + 1 < nsub && classify(s + 1, on1, masked1);
            if (next) ensure(s + 1);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) rescale_acc<D>(acc[nt], alpha[nt]);
            // Straight-line from here.  The K fragments of s + 1 are read once
            // the PV products of s are issued (the V^T fragments are then
            // dead, and the read's latency hides under the products).  Past
            // the run's last sub-block the slot read may hold anything; the
            // QK products and the softmax on it are dropped, which is cheaper
            // than a branch that would split the block.
            float m1[NT], l1[NT], a1[NT];
            half4 pn[NT][KT];
            // Raised wave priority while the products are issued: of the two
            // wavefronts of a SIMD, the one issuing MFMAs goes first, the
            // other's softmax fills the VALU (measured 2-3% faster; raising
            // it for the softmax instead was slower).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) pv_tile<SBS, D, BF16>(vt, pf[nt], acc[nt]);
            Stage<SBS, D>::read(kf, kbuf[(s + 1) % kStages], r, q4);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) qk_tile<SBS, D, BF16>(kf, qf[nt], sc[nt]);
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                m1[nt] = m_run[nt];
                l1[nt] = l_run[nt];
            }
            softmax_open_tiles<NT, KT, BF16>(sc, p.scale_log2, m1, l1, a1, pn);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                m_run[nt] = next ? m1[nt] : m_run[nt];
                l_run[nt] = next ? l1[nt] : l_run[nt];
                alpha[nt] = next ? a1[nt] : 1.f;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) pf[nt][kt] = pn[nt][kt];
            }
            ++s;
            if (!next) break;
        }
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

template <int D, int PACK, bool BF16>
hipError_t launch_dense(const DenseParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((nsa_dense_kernel<D, PACK, BF16>), dim3(p.per_xcd * p.nxcd), dim3(kWaveSize * kDenseWaves),
                       0, stream, p);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dense_dt(const DenseParams &p, int D, int pack, hipStream_t stream) {
    if (D == 128)
        return pack == 4 ? launch_dense<128, 4, BF16>(p, stream) : pack == 2 ? launch_dense<128, 2, BF16>(p, stream)
                                                                                : launch_dense<128, 1, BF16>(p, stream);
    return pack == 4 ? launch_dense<64, 4, BF16>(p, stream) : pack == 2 ? launch_dense<64, 2, BF16>(p, stream)
                                                                         : launch_dense<64, 1, BF16>(p, stream);
}

}  // namespace

namespace {

int window_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M, int N, int H, int G,
               int D, int left, int right, hipStream_t stream, bool bf16) {
    if (!Q || !K || !V || !O || !LSE) return NSA_SEL_ERR_NULL;
    if (B < 1 || M < 1 || N < 1 || H < 1 || G < 1 || D < 1) return NSA_SEL_ERR_SHAPE;
    if (H % G != 0) return NSA_SEL_ERR_SHAPE;
    const int gs = H / G;
    if ((D != 64 && D != 128) || gs > 16) return NSA_SEL_ERR_UNSUPPORTED;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15) return NSA_SEL_ERR_ALIGN;
    if ((uintptr_t)LSE & 3) return NSA_SEL_ERR_ALIGN;
    if ((int64_t)B * M * G > INT_MAX || (int64_t)N * G * D > INT_MAX || (int64_t)M + N > INT_MAX)
        return NSA_SEL_ERR_RANGE;
    const size_t q_bytes = (size_t)B * M * H * D * 2, kv_bytes = (size_t)B * N * G * D * 2;
    const size_t lse_bytes = (size_t)B * H * M * 4;
    const void *ins[3] = {Q, K, V};
    const size_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
    for (int i = 0; i < 3; ++i) {
        if (ranges_overlap(O, q_bytes, ins[i], in_bytes[i]) || ranges_overlap(LSE, lse_bytes, ins[i], in_bytes[i]))
            return NSA_SEL_ERR_ALIAS;
    }
    if (ranges_overlap(O, q_bytes, LSE, lse_bytes)) return NSA_SEL_ERR_ALIAS;

    const int pack = (16 / gs) >= 4 ? 4 : (16 / gs) >= 2 ? 2 : 1;
    const int qwg = kDenseWaves * kDenseTiles * pack;
    DenseParams p;
    p.Q = (const _Float16 *)Q;
    p.K = (const _Float16 *)K;
    p.V = (const _Float16 *)V;
    p.O = (_Float16 *)O;
    p.LSE = LSE;
    p.B = B; p.M = M; p.N = N; p.H = H; p.G = G; p.gs = gs;
    p.qtiles = (M + qwg - 1) / qwg;
    p.units = B * G * p.qtiles;
    p.nxcd = device_topology().nxcd;
    p.per_xcd = (p.units + p.nxcd - 1) / p.nxcd;
    // A bound that reaches past every query (left >= M) or every key
    // (right >= N) is the same as none.
    p.left = (left < 0 || left >= M) ? -1 : left;
    p.right = (right < 0 || right >= N) ? -1 : right;
    p.scale_log2 = kLog2e / sqrtf((float)D);
    const hipError_t e = bf16 ? launch_dense_dt<true>(p, D, pack, stream) : launch_dense_dt<false>(p, D, pack, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}

}  // namespace

extern "C" int nsa_dense_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M, int N,
                             int H, int G, int D, hipStream_t stream) {
    return window_fwd(Q, K, V, O, LSE, B, M, N, H, G, D, -1, 0, stream, false);
}

extern "C" int nsa_window_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M, int N,
                              int H, int G, int D, int left, int right, hipStream_t stream) {
    return window_fwd(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream, false);
}

extern "C" int nsa_window_fwd_bf16(const void *Q, const void *K, const void *V, void *O, float *LSE, int B, int M,
                                   int N, int H, int G, int D, int left, int right, hipStream_t stream) {
    return window_fwd(Q, K, V, O, LSE, B, M, N, H, G, D, left, right, stream, true);
}
