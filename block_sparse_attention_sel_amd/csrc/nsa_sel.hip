// NSA selection-attention forward for AMD MI355X (gfx950, CDNA4).
//
// Operation: wave issue "[wave] NSA: selection attention forward kernel",
// sections Operation, Algorithm, Requirements and "MI350 considerations".
// One wavefront owns one unit (b, m, g) -- the page's program instance -- and
// computes all H/G heads of the group together (the page's BLOCK_H register
// tiling).  For each counted entry t of block_indices[b, m, g, :] it gathers
// the bs keys of block t for group g, forms scores for all heads, applies the
// causal mask, and folds the block into a running-max / running-sum softmax
// (the "online softmax across all T blocks" requirement); O and the natural
// log-sum-exp are written at the end.
//
// MI355X mapping (see the design notes for the reasoning and the roofline):
//  * Scores are computed transposed, S^T = K * Q^T, on v_mfma_f32_16x16x32_f16:
//    keys are the 16 MFMA rows, the (up to 16) heads of the group are the
//    columns.  With keys as rows, one 128-bit global load per lane puts a K
//    row slice straight into the MFMA A-operand layout, and the S^T result
//    layout (lane l: head l%16, keys 4*(l/16)+i) is already the B-operand
//    layout of the PV product, so P never leaves registers.
//  * V arrives with the same 128-bit row loads.  PV needs V^T fragments; they
//    are produced in registers by v_mfma_f32_16x16x16_f16 against a one-hot
//    matrix (an exact permutation: every output is one fp16 value times 1.0).
//    No LDS is used, so waves never synchronise and occupancy is set by VGPRs.
//  * The T loop is software-pipelined: the next counted block's K/V loads are
//    issued before the current block's math (register double buffering).
//  * Workgroups (4 waves = 4 consecutive query positions of one (b, g)) are
//    mapped XCD-aware: hardware deals workgroup w to XCD w % 8, so unit ranges
//    are laid out so that each XCD walks a contiguous (b, g, m) range and its
//    L2 holds the K/V prefix of few groups.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

#include "nsa_sel.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kWaveSize = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWaveSize * kWavesPerBlock;
constexpr int kNumXcd = 8;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

struct Params {
    const _Float16 *Q;
    const _Float16 *K;
    const _Float16 *V;
    const int32_t *idx;
    _Float16 *O;
    float *LSE;
    int B, M, N, H, G, T, gs, NB;
    int units;          // B * M * G
    int slots_per_xcd;  // workgroup slots per XCD
    float scale_log2;   // log2(e) / sqrt(D)
};

__device__ __forceinline__ float4v mfma_16x16x32(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4v mfma_16x16x16(half4 a, half4 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half4 lo4(half8 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ half4 hi4(half8 v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

__device__ __forceinline__ half4 to_half4(float4v v) {
    half4 r;
    r[0] = (_Float16)v[0];
    r[1] = (_Float16)v[1];
    r[2] = (_Float16)v[2];
    r[3] = (_Float16)v[3];
    return r;
}

__device__ __forceinline__ half8 cat8(half4 a, half4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Scans one index row in chunks of 64 entries: lane j holds entry base + j and
// a wave ballot marks the counted ones, so finding the next counted entry is
// scalar bit arithmetic.
struct IndexScan {
    const int32_t *row;
    int T, cm, NB, lane;
    int base;
    uint64_t mask;
    int val;

    __device__ __forceinline__ void load(int b) {
        base = b;
        const int j = b + lane;
        const int v = (j < T) ? row[j] : -1;
        val = v;
        const bool ok = v >= 0 && v <= cm && v < NB;
        mask = __ballot(ok);
    }
    // Position of the first counted entry at or after i, or T.
    __device__ __forceinline__ int next(int i) {
        while (i < T) {
            if (i >= base + kWaveSize) load(i);
            const uint64_t mm = mask >> (i - base);
            if (mm) return i + __builtin_ctzll(mm);
            i = base + kWaveSize;
        }
        return T;
    }
    // Entry at position i; valid while i lies in the loaded chunk.
    __device__ __forceinline__ int value(int i) const {
        return __builtin_amdgcn_readlane(val, i - base);
    }
};

template <int BS, int D>
struct Tile {
    static constexpr int KT = BS / 16;  // 16-key MFMA row tiles per block
    static constexpr int DC = D / 32;   // 32-wide head-dim chunks
    half8 k[KT][DC];
    half8 v[KT][DC];
};

// Gathers block t of one (b, g) head: lane l reads key row t*BS + 16*kt + l%16,
// head-dim slice 32*c + 8*(l/16) .. +7 (16 bytes) of K and V.
template <int BS, int D>
__device__ __forceinline__ void load_block(Tile<BS, D> &tl, const _Float16 *Kg, const _Float16 *Vg,
                                           int t, int N, int row_stride, int r, int q4) {
#pragma unroll
    for (int kt = 0; kt < Tile<BS, D>::KT; ++kt) {
        int n = t * BS + kt * 16 + r;
        n = n < N ? n : N - 1;  // rows past the end are masked; keep the address in bounds
        const size_t off = (size_t)n * row_stride + q4 * 8;
#pragma unroll
        for (int c = 0; c < Tile<BS, D>::DC; ++c) {
            tl.k[kt][c] = *(const half8 *)(Kg + off + c * 32);
            tl.v[kt][c] = *(const half8 *)(Vg + off + c * 32);
        }
    }
}

// Folds one gathered block into the running softmax state of the wave.
// acc[c][hh] holds O^T rows d = 32*c + 8*(l/16) + 4*hh + i for head l%16.
template <int BS, int D>
__device__ __forceinline__ void process_block(const Tile<BS, D> &tl, const half8 (&qf)[D / 32],
                                              half4 onehot, int key0, int m, int N, float scale_log2,
                                              float &m_run, float &l_run,
                                              float4v (&acc)[D / 32][2], int q4) {
    constexpr int KT = Tile<BS, D>::KT;
    constexpr int DC = Tile<BS, D>::DC;
    // S^T = K * Q^T: lane l gets keys key0 + 16*kt + 4*(l/16) + i, head l%16.
    float4v s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        s[kt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DC; ++c) s[kt] = mfma_16x16x32(tl.k[kt][c], qf[c], s[kt]);
    }
    // Scale into the log2 domain and apply the causal mask where the block
    // reaches past the query (only the query's own block) or past N.
    const bool need_mask = (key0 + BS - 1 > m) || (key0 + BS > N);
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = s[kt][i] * scale_log2;
            if (need_mask) {
                const int key = key0 + kt * 16 + q4 * 4 + i;
                if (key > m || key >= N) x = -INFINITY;
            }
            s[kt][i] = x;
            mloc = fmaxf(mloc, x);
        }
    }
    // Row max over the 4 lanes (l, l^16, l^32, l^48) that share a head.
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    half4 pf[KT];
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        float4v p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(s[kt][i] - m_use);
            psum += p[i];
        }
        pf[kt] = to_half4(p);
    }
    l_run = l_run * alpha + psum;  // per-lane partial; lanes are summed at the end
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        acc[c][0] *= alpha;
        acc[c][1] *= alpha;
    }
    // O^T += V^T * P^T over 32-key chunks.  The B operand is P^T straight
    // from the score layout; the A operand is V^T, made by the one-hot MFMA.
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < BS / 32; ++kc) {
        const half8 bp = cat8(pf[2 * kc], pf[2 * kc + 1]);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            {
                const float4v t0 = mfma_16x16x16(lo4(tl.v[2 * kc][c]), onehot, zero);
                const float4v t1 = mfma_16x16x16(lo4(tl.v[2 * kc + 1][c]), onehot, zero);
                acc[c][0] = mfma_16x16x32(cat8(to_half4(t0), to_half4(t1)), bp, acc[c][0]);
            }
            {
                const float4v t0 = mfma_16x16x16(hi4(tl.v[2 * kc][c]), onehot, zero);
                const float4v t1 = mfma_16x16x16(hi4(tl.v[2 * kc + 1][c]), onehot, zero);
                acc[c][1] = mfma_16x16x32(cat8(to_half4(t0), to_half4(t1)), bp, acc[c][1]);
            }
        }
    }
}

template <int BS, int D>
__global__ __launch_bounds__(kThreads) void nsa_sel_fwd_kernel(Params p) {
    constexpr int DC = D / 32;
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = blockIdx.x;
    const int slot = (w % kNumXcd) * p.slots_per_xcd + (w / kNumXcd);
    const int u = slot * kWavesPerBlock + wave;
    if (u >= p.units) return;
    // Unit order (b, g, m) with m fastest.
    const int m = u % p.M;
    const int bg = u / p.M;
    const int g = bg % p.G;
    const int b = bg / p.G;
    const int r = lane & 15;
    const int q4 = lane >> 4;
    const int h0 = g * p.gs;

    // Q^T fragments (B operand): lane l holds head h0 + l%16, head-dim slice
    // 32*c + 8*(l/16) .. +7; heads past the group are zero columns.
    half8 qf[DC];
    {
        // Padding columns read a real head row (kept in bounds) and are zeroed.
        const int hq = (r < p.gs) ? h0 + r : h0;
        const _Float16 *qrow = p.Q + ((size_t)(b * (size_t)p.M + m) * p.H + hq) * D;
        const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const half8 x = *(const half8 *)(qrow + c * 32 + q4 * 8);
            qf[c] = (r < p.gs) ? x : zero8;
        }
    }
    // One-hot B operand of the V transpose: column l%16 picks head-dim
    // 8*((l%16)/4) + (l%16)%4 of the lane group's 4-wide slice.
    half4 onehot = {0, 0, 0, 0};
    if (q4 == (r >> 2)) onehot[r & 3] = (_Float16)1.0f;

    const int row_stride = p.G * D;
    const _Float16 *Kg = p.K + ((size_t)b * p.N * p.G + g) * D;
    const _Float16 *Vg = p.V + ((size_t)b * p.N * p.G + g) * D;

    IndexScan scan;
    scan.row = p.idx + ((size_t)(b * (size_t)p.M + m) * p.G + g) * p.T;
    scan.T = p.T;
    scan.cm = m / BS;
    scan.NB = p.NB;
    scan.lane = lane;
    scan.load(0);

    float m_run = -INFINITY;
    float l_run = 0.f;
    float4v acc[DC][2];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        acc[c][0] = float4v{0.f, 0.f, 0.f, 0.f};
        acc[c][1] = float4v{0.f, 0.f, 0.f, 0.f};
    }

    Tile<BS, D> ta, tb;
    int i = scan.next(0);
    int t_cur = (i < p.T) ? scan.value(i) : 0;
    if (i < p.T) load_block<BS, D>(ta, Kg, Vg, t_cur, p.N, row_stride, r, q4);
    // Two-stage pipeline, unrolled by two so the buffers never need copying.
    while (i < p.T) {
        int in = scan.next(i + 1);
        int t_n = (in < p.T) ? scan.value(in) : 0;
        if (in < p.T) load_block<BS, D>(tb, Kg, Vg, t_n, p.N, row_stride, r, q4);
        process_block<BS, D>(ta, qf, onehot, t_cur * BS, m, p.N, p.scale_log2, m_run, l_run, acc, q4);
        i = in;
        t_cur = t_n;
        if (i >= p.T) break;
        in = scan.next(i + 1);
        t_n = (in < p.T) ? scan.value(in) : 0;
        if (in < p.T) load_block<BS, D>(ta, Kg, Vg, t_n, p.N, row_stride, r, q4);
        process_block<BS, D>(tb, qf, onehot, t_cur * BS, m, p.N, p.scale_log2, m_run, l_run, acc, q4);
        i = in;
        t_cur = t_n;
    }

    // Epilogue: total row sum over the 4 lanes of a head, normalise, store.
    float l = l_run + __shfl_xor(l_run, 16);
    l += __shfl_xor(l, 32);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (r < p.gs) {
        _Float16 *orow = p.O + ((size_t)(b * (size_t)p.M + m) * p.H + h0 + r) * D;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const half4 lo = to_half4(acc[c][0] * inv);
            const half4 hi = to_half4(acc[c][1] * inv);
            *(half8 *)(orow + c * 32 + q4 * 8) = cat8(lo, hi);
        }
        if (q4 == 0) {
            const float lse = l > 0.f ? m_run * kLn2 + logf(l) : -INFINITY;
            p.LSE[((size_t)b * p.H + h0 + r) * p.M + m] = lse;
        }
    }
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

template <int BS, int D>
hipError_t launch(const Params &p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((nsa_sel_fwd_kernel<BS, D>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

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
        default: return "nsa_sel: unknown status";
    }
}

extern "C" int nsa_sel_fwd(const void *Q, const void *K, const void *V, const int32_t *block_indices,
                           void *O, float *LSE, int B, int M, int N, int H, int G, int D,
                           int block_size, int T, hipStream_t stream) {
    if (!Q || !K || !V || !block_indices || !O || !LSE) return NSA_SEL_ERR_NULL;
    if (B < 1 || M < 1 || N < 1 || H < 1 || G < 1 || D < 1 || block_size < 1 || T < 1)
        return NSA_SEL_ERR_SHAPE;
    if (H % G != 0) return NSA_SEL_ERR_SHAPE;
    const int gs = H / G;
    if ((D != 64 && D != 128) || (block_size != 32 && block_size != 64) || gs > 16)
        return NSA_SEL_ERR_UNSUPPORTED;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15) return NSA_SEL_ERR_ALIGN;
    if (((uintptr_t)block_indices | (uintptr_t)LSE) & 3) return NSA_SEL_ERR_ALIGN;

    const int64_t units = (int64_t)B * M * G;
    const int64_t wgs = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t slots = (wgs + kNumXcd - 1) / kNumXcd;
    // Element counts must fit the 64-bit offsets; unit ids and the grid use int.
    const int64_t q_elems = (int64_t)B * M * H * D;
    const int64_t kv_elems = (int64_t)B * N * G * D;
    const int64_t idx_elems = (int64_t)B * M * G * T;
    if (units > INT_MAX || slots * kNumXcd * kThreads > (int64_t)UINT32_MAX ||
        (int64_t)N * G * D > INT_MAX)
        return NSA_SEL_ERR_RANGE;

    const size_t q_bytes = (size_t)q_elems * 2, kv_bytes = (size_t)kv_elems * 2;
    const size_t idx_bytes = (size_t)idx_elems * 4, lse_bytes = (size_t)B * H * M * 4;
    const void *ins[4] = {Q, K, V, block_indices};
    const size_t in_bytes[4] = {q_bytes, kv_bytes, kv_bytes, idx_bytes};
    for (int i = 0; i < 4; ++i) {
        if (ranges_overlap(O, q_bytes, ins[i], in_bytes[i]) ||
            ranges_overlap(LSE, lse_bytes, ins[i], in_bytes[i]))
            return NSA_SEL_ERR_ALIAS;
    }
    if (ranges_overlap(O, q_bytes, LSE, lse_bytes)) return NSA_SEL_ERR_ALIAS;

    Params p;
    p.Q = (const _Float16 *)Q;
    p.K = (const _Float16 *)K;
    p.V = (const _Float16 *)V;
    p.idx = block_indices;
    p.O = (_Float16 *)O;
    p.LSE = LSE;
    p.B = B; p.M = M; p.N = N; p.H = H; p.G = G; p.T = T; p.gs = gs;
    p.NB = (N + block_size - 1) / block_size;
    p.units = (int)units;
    p.slots_per_xcd = (int)slots;
    p.scale_log2 = kLog2e / sqrtf((float)D);
    const int grid = (int)(slots * kNumXcd);

    hipError_t e;
    if (block_size == 64)
        e = (D == 128) ? launch<64, 128>(p, grid, stream) : launch<64, 64>(p, grid, stream);
    else
        e = (D == 128) ? launch<32, 128>(p, grid, stream) : launch<32, 64>(p, grid, stream);
    return e == hipSuccess ? NSA_SEL_OK : NSA_SEL_ERR_HIP;
}
