// Shared building blocks of the gfx950 selection-attention kernels: the
// parameter block, index-row merging, LDS staging of gathered K/V blocks, the
// wavefront-slot mapping with its generation launches, and the host-side
// launch planning.  It is included by exactly one source file of each
// library (the forward kernel, and the gather probe that replays the
// forward kernel's block-gather stream without the math), so everything here
// has internal linkage.
//
// Operation: wave issue "[wave] NSA: selection attention forward kernel",
// sections Operation, Algorithm, Requirements and "MI350 considerations".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>
#include <math.h>

#include <atomic>

#include "nsa_sel.h"

namespace {

// Fragments are held as 16-bit containers (half8 / half4) whatever the
// element type: the staging, the LDS reads and the transposes only move bits;
// the MFMA and the float -> 16-bit packing are the type-specific steps.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kWaveSize = 64;
// Wavefronts per workgroup: with 32-key stages (16 KiB per wavefront at
// D = 128) two 4-wavefront workgroups share a CU, two wavefronts per SIMD;
// with 64-key stages five wavefronts fill the CU's 160 KiB of LDS.
constexpr int waves_per_wg(int sbs) { return sbs == 32 ? 4 : 5; }
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
    int pack;           // queries per 16-column MFMA tile (1, 2 or 4; see nsa_sel_fwd)
    int mode;           // 0: cursor merge, one tile; 1/2: register merge with that many tiles
    int wslots_per_bg;  // wavefront slots per (b, g): ceil(M / queries per wavefront)
    int wslots;         // B * G * wslots_per_bg
    int per_xcd;        // wavefront slots owned by each XCD: ceil(wslots / 8)
    int gen_step;       // wavefront slots one XCD runs per generation (its workgroup slots x waves)
    int gen;            // first generation of this launch
    int wg_per_gen;     // workgroups of one generation (a launch carries one or all generations)
    int nxcd;           // XCDs workgroups are dealt to (w % nxcd); 1 = one contiguous range
    int l2_bytes;       // L2 of one XCD
    unsigned *sched;    // persistent schedule words (device), or nullptr: generation launches only
    int sched_cap;      // 32-bit words available at sched
    int gens;           // generations of one XCD's range (persistent launch)
    int steps_max;      // steps of the persistent loop: nxcd * gens + 1
    float scale_log2;   // log2(e) / sqrt(D)
};

constexpr int kDone = INT_MAX;

// Batched ds_read_b128 of one staged block into MFMA fragments, ending in
// s_waitcnt lgkmcnt(0).  f[kt][c] comes from address a[c] + kt * 16 rows.
template <int BS, int D>
struct LdsBatch;

#define NSA_DSR(o, a, off) "ds_read_b128 %" #o ", %" #a " offset:" #off "\n"

template <>
struct LdsBatch<64, 128> {  // 16 rows = 4096 bytes
    __device__ static __forceinline__ void run(half8 (&f)[4][4], const unsigned (&a)[4]) {
        asm volatile(NSA_DSR(0, 16, 0) NSA_DSR(1, 17, 0) NSA_DSR(2, 18, 0) NSA_DSR(3, 19, 0)
                     NSA_DSR(4, 16, 4096) NSA_DSR(5, 17, 4096) NSA_DSR(6, 18, 4096) NSA_DSR(7, 19, 4096)
                     NSA_DSR(8, 16, 8192) NSA_DSR(9, 17, 8192) NSA_DSR(10, 18, 8192) NSA_DSR(11, 19, 8192)
                     NSA_DSR(12, 16, 12288) NSA_DSR(13, 17, 12288) NSA_DSR(14, 18, 12288)
                     NSA_DSR(15, 19, 12288) "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0]), "=&v"(f[0][1]), "=&v"(f[0][2]), "=&v"(f[0][3]), "=&v"(f[1][0]),
                       "=&v"(f[1][1]), "=&v"(f[1][2]), "=&v"(f[1][3]), "=&v"(f[2][0]), "=&v"(f[2][1]),
                       "=&v"(f[2][2]), "=&v"(f[2][3]), "=&v"(f[3][0]), "=&v"(f[3][1]), "=&v"(f[3][2]),
                       "=&v"(f[3][3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};

template <>
struct LdsBatch<32, 128> {
    __device__ static __forceinline__ void run(half8 (&f)[2][4], const unsigned (&a)[4]) {
        asm volatile(NSA_DSR(0, 8, 0) NSA_DSR(1, 9, 0) NSA_DSR(2, 10, 0) NSA_DSR(3, 11, 0)
                     NSA_DSR(4, 8, 4096) NSA_DSR(5, 9, 4096) NSA_DSR(6, 10, 4096) NSA_DSR(7, 11, 4096)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0]), "=&v"(f[0][1]), "=&v"(f[0][2]), "=&v"(f[0][3]), "=&v"(f[1][0]),
                       "=&v"(f[1][1]), "=&v"(f[1][2]), "=&v"(f[1][3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};

template <>
struct LdsBatch<64, 64> {  // 16 rows = 2048 bytes
    __device__ static __forceinline__ void run(half8 (&f)[4][2], const unsigned (&a)[2]) {
        asm volatile(NSA_DSR(0, 8, 0) NSA_DSR(1, 9, 0) NSA_DSR(2, 8, 2048) NSA_DSR(3, 9, 2048)
                     NSA_DSR(4, 8, 4096) NSA_DSR(5, 9, 4096) NSA_DSR(6, 8, 6144) NSA_DSR(7, 9, 6144)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0]), "=&v"(f[0][1]), "=&v"(f[1][0]), "=&v"(f[1][1]), "=&v"(f[2][0]),
                       "=&v"(f[2][1]), "=&v"(f[3][0]), "=&v"(f[3][1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    }
};

template <>
struct LdsBatch<32, 64> {
    __device__ static __forceinline__ void run(half8 (&f)[2][2], const unsigned (&a)[2]) {
        asm volatile(NSA_DSR(0, 4, 0) NSA_DSR(1, 5, 0) NSA_DSR(2, 4, 2048) NSA_DSR(3, 5, 2048)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0]), "=&v"(f[0][1]), "=&v"(f[1][0]), "=&v"(f[1][1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    }
};

#undef NSA_DSR

// Transposing reads of one staged V block (ds_read_b64_tr_b16), ending in
// s_waitcnt lgkmcnt(0).  Within each 16-lane group the instruction hands
// lane 4a+b element b of the 8-byte pieces loaded by lanes a, a+4, a+8, a+12
// (element j from lane a+4j).  Lane (a + 4j) of group q4 points at V row
// 32*kc + 16*half + 4*q4 + j, head-dims 32*c + 8*a + 4*hh .. +3, so lane
// 4a+b receives V^T[32*c + 8*a + 4*hh + b][32*kc + 16*half + 4*q4 + j]: the
// A operand of the PV MFMA for 32-key chunk kc and head-dim set (c, hh).
// f[kc][c][hh][half]; a[c] is the lane's address for head-dim chunk c.
template <int BS, int D>
struct LdsTrBatch;

template <>
struct LdsTrBatch<64, 128> {
    __device__ static __forceinline__ void run(half4 (&f)[2][4][2][2], const unsigned (&a)[4]) {
        asm volatile("ds_read_b64_tr_b16 %0, %16 offset:0\n" "ds_read_b64_tr_b16 %1, %16 offset:4096\n" "ds_read_b64_tr_b16 %2, %16 offset:8\n" "ds_read_b64_tr_b16 %3, %16 offset:4104\n" "ds_read_b64_tr_b16 %4, %17 offset:0\n" "ds_read_b64_tr_b16 %5, %17 offset:4096\n" "ds_read_b64_tr_b16 %6, %17 offset:8\n" "ds_read_b64_tr_b16 %7, %17 offset:4104\n" "ds_read_b64_tr_b16 %8, %18 offset:0\n" "ds_read_b64_tr_b16 %9, %18 offset:4096\n" "ds_read_b64_tr_b16 %10, %18 offset:8\n" "ds_read_b64_tr_b16 %11, %18 offset:4104\n" "ds_read_b64_tr_b16 %12, %19 offset:0\n" "ds_read_b64_tr_b16 %13, %19 offset:4096\n" "ds_read_b64_tr_b16 %14, %19 offset:8\n" "ds_read_b64_tr_b16 %15, %19 offset:4104\n" "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0][0][0]), "=&v"(f[0][0][0][1]), "=&v"(f[0][0][1][0]), "=&v"(f[0][0][1][1]), "=&v"(f[0][1][0][0]), "=&v"(f[0][1][0][1]), "=&v"(f[0][1][1][0]), "=&v"(f[0][1][1][1]), "=&v"(f[0][2][0][0]), "=&v"(f[0][2][0][1]), "=&v"(f[0][2][1][0]), "=&v"(f[0][2][1][1]), "=&v"(f[0][3][0][0]), "=&v"(f[0][3][0][1]), "=&v"(f[0][3][1][0]), "=&v"(f[0][3][1][1])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
        asm volatile("ds_read_b64_tr_b16 %0, %16 offset:8192\n" "ds_read_b64_tr_b16 %1, %16 offset:12288\n" "ds_read_b64_tr_b16 %2, %16 offset:8200\n" "ds_read_b64_tr_b16 %3, %16 offset:12296\n" "ds_read_b64_tr_b16 %4, %17 offset:8192\n" "ds_read_b64_tr_b16 %5, %17 offset:12288\n" "ds_read_b64_tr_b16 %6, %17 offset:8200\n" "ds_read_b64_tr_b16 %7, %17 offset:12296\n" "ds_read_b64_tr_b16 %8, %18 offset:8192\n" "ds_read_b64_tr_b16 %9, %18 offset:12288\n" "ds_read_b64_tr_b16 %10, %18 offset:8200\n" "ds_read_b64_tr_b16 %11, %18 offset:12296\n" "ds_read_b64_tr_b16 %12, %19 offset:8192\n" "ds_read_b64_tr_b16 %13, %19 offset:12288\n" "ds_read_b64_tr_b16 %14, %19 offset:8200\n" "ds_read_b64_tr_b16 %15, %19 offset:12296\n" "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[1][0][0][0]), "=&v"(f[1][0][0][1]), "=&v"(f[1][0][1][0]), "=&v"(f[1][0][1][1]), "=&v"(f[1][1][0][0]), "=&v"(f[1][1][0][1]), "=&v"(f[1][1][1][0]), "=&v"(f[1][1][1][1]), "=&v"(f[1][2][0][0]), "=&v"(f[1][2][0][1]), "=&v"(f[1][2][1][0]), "=&v"(f[1][2][1][1]), "=&v"(f[1][3][0][0]), "=&v"(f[1][3][0][1]), "=&v"(f[1][3][1][0]), "=&v"(f[1][3][1][1])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};

template <>
struct LdsTrBatch<32, 128> {
    __device__ static __forceinline__ void run(half4 (&f)[1][4][2][2], const unsigned (&a)[4]) {
        asm volatile("ds_read_b64_tr_b16 %0, %16 offset:0\n" "ds_read_b64_tr_b16 %1, %16 offset:4096\n" "ds_read_b64_tr_b16 %2, %16 offset:8\n" "ds_read_b64_tr_b16 %3, %16 offset:4104\n" "ds_read_b64_tr_b16 %4, %17 offset:0\n" "ds_read_b64_tr_b16 %5, %17 offset:4096\n" "ds_read_b64_tr_b16 %6, %17 offset:8\n" "ds_read_b64_tr_b16 %7, %17 offset:4104\n" "ds_read_b64_tr_b16 %8, %18 offset:0\n" "ds_read_b64_tr_b16 %9, %18 offset:4096\n" "ds_read_b64_tr_b16 %10, %18 offset:8\n" "ds_read_b64_tr_b16 %11, %18 offset:4104\n" "ds_read_b64_tr_b16 %12, %19 offset:0\n" "ds_read_b64_tr_b16 %13, %19 offset:4096\n" "ds_read_b64_tr_b16 %14, %19 offset:8\n" "ds_read_b64_tr_b16 %15, %19 offset:4104\n" "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0][0][0]), "=&v"(f[0][0][0][1]), "=&v"(f[0][0][1][0]), "=&v"(f[0][0][1][1]), "=&v"(f[0][1][0][0]), "=&v"(f[0][1][0][1]), "=&v"(f[0][1][1][0]), "=&v"(f[0][1][1][1]), "=&v"(f[0][2][0][0]), "=&v"(f[0][2][0][1]), "=&v"(f[0][2][1][0]), "=&v"(f[0][2][1][1]), "=&v"(f[0][3][0][0]), "=&v"(f[0][3][0][1]), "=&v"(f[0][3][1][0]), "=&v"(f[0][3][1][1])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    }
};

template <>
struct LdsTrBatch<64, 64> {
    __device__ static __forceinline__ void run(half4 (&f)[2][2][2][2], const unsigned (&a)[2]) {
        asm volatile("ds_read_b64_tr_b16 %0, %8 offset:0\n" "ds_read_b64_tr_b16 %1, %8 offset:2048\n" "ds_read_b64_tr_b16 %2, %8 offset:8\n" "ds_read_b64_tr_b16 %3, %8 offset:2056\n" "ds_read_b64_tr_b16 %4, %9 offset:0\n" "ds_read_b64_tr_b16 %5, %9 offset:2048\n" "ds_read_b64_tr_b16 %6, %9 offset:8\n" "ds_read_b64_tr_b16 %7, %9 offset:2056\n" "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0][0][0]), "=&v"(f[0][0][0][1]), "=&v"(f[0][0][1][0]), "=&v"(f[0][0][1][1]), "=&v"(f[0][1][0][0]), "=&v"(f[0][1][0][1]), "=&v"(f[0][1][1][0]), "=&v"(f[0][1][1][1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
        asm volatile("ds_read_b64_tr_b16 %0, %8 offset:4096\n" "ds_read_b64_tr_b16 %1, %8 offset:6144\n" "ds_read_b64_tr_b16 %2, %8 offset:4104\n" "ds_read_b64_tr_b16 %3, %8 offset:6152\n" "ds_read_b64_tr_b16 %4, %9 offset:4096\n" "ds_read_b64_tr_b16 %5, %9 offset:6144\n" "ds_read_b64_tr_b16 %6, %9 offset:4104\n" "ds_read_b64_tr_b16 %7, %9 offset:6152\n" "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[1][0][0][0]), "=&v"(f[1][0][0][1]), "=&v"(f[1][0][1][0]), "=&v"(f[1][0][1][1]), "=&v"(f[1][1][0][0]), "=&v"(f[1][1][0][1]), "=&v"(f[1][1][1][0]), "=&v"(f[1][1][1][1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    }
};

template <>
struct LdsTrBatch<32, 64> {
    __device__ static __forceinline__ void run(half4 (&f)[1][2][2][2], const unsigned (&a)[2]) {
        asm volatile("ds_read_b64_tr_b16 %0, %8 offset:0\n" "ds_read_b64_tr_b16 %1, %8 offset:2048\n" "ds_read_b64_tr_b16 %2, %8 offset:8\n" "ds_read_b64_tr_b16 %3, %8 offset:2056\n" "ds_read_b64_tr_b16 %4, %9 offset:0\n" "ds_read_b64_tr_b16 %5, %9 offset:2048\n" "ds_read_b64_tr_b16 %6, %9 offset:8\n" "ds_read_b64_tr_b16 %7, %9 offset:2056\n" "s_waitcnt lgkmcnt(0)"
                     : "=&v"(f[0][0][0][0]), "=&v"(f[0][0][0][1]), "=&v"(f[0][0][1][0]), "=&v"(f[0][0][1][1]), "=&v"(f[0][1][0][0]), "=&v"(f[0][1][0][1]), "=&v"(f[0][1][1][0]), "=&v"(f[0][1][1][1])
                     : "v"(a[0]), "v"(a[1])
                     : "memory");
    }
};


// LDS staging of one gathered block (K and V, BS rows of D fp16 each).
//
// The block is copied global -> LDS with 128-bit direct-to-LDS buffer loads
// (buffer_load_dwordx4 ... lds).  One such instruction moves 1 KiB: lane l
// writes bytes [16*l, 16*l + 16) of the instruction's LDS window, and the
// global address of every lane is free.  Lanes are given consecutive 16-byte
// pieces of the same key row (a row is D*2 bytes = LPR lanes), so each
// instruction reads whole rows and coalesces into full cache lines.
//
// In LDS a row occupies D*2 contiguous bytes; its 16-byte pieces are stored
// XOR-permuted, piece c at slot c ^ swz(row).  The permutation comes from the
// LDS's service pattern, measured with single-instruction probes on gfx950:
// 64 banks of 4 bytes; a ds_read_b128 is served in four passes of 16 lanes,
// pass = (lane / 32, parity of bits 2..4 of the lane), and a ds_read_b64 (and
// its transposing form) in two passes of 32 consecutive lanes; lanes of one
// pass that touch the same bank in different rows serialise.  The two read
// patterns are the MFMA-fragment reads (lane l: row l % 16, piece 4c + l / 16)
// and the transposing V^T reads (lane l: row 4 (l / 16) + (l / 4) % 4, piece
// 4c + l % 4, one 8-byte half of it).  swz makes the first conflict-free and
// the second 2-way, which is the least possible: every lane of a transposing
// read takes the same half of its piece, so it reaches only 32 of the banks.
// (Measured per instruction: 4.2 and 4.1 cycles, against 4.2 / 8.1 for
// slot = c ^ row and 8.1 / 4.1 for c ^ row ^ ((row & 3) << 2).)
//
// Addressing: the per-lane part of the byte offset repeats every 16/RPI
// instructions (the swizzle depends on row % 16), so it lives in NV VGPRs;
// the per-instruction row step and the block start are uniform (SGPR).
template <int BS, int D>
struct Stage {
    static constexpr int LPR = D / 8;                // lanes (16-byte pieces) per row
    static constexpr int RPI = kWaveSize / LPR;      // rows per 1 KiB instruction
    static constexpr int NI = BS / RPI;              // instructions per K (or V) block
    static constexpr int NV = 16 / RPI;              // distinct per-lane offsets
    static constexpr int HALVES = BS * D;            // fp16 elements per K (or V) block

    // A function of row % 16 (the per-lane copy offsets repeat with it).
    // D = 128 (16 slots per row): row bits 0, 1 -> slot bits 2, 3 and row bit
    // 2 -> slot bit 1.  D = 64 (8 slots; two rows share the 64 banks): row
    // bits 1, 2, 3 -> slot bits 0, 2, 1.
    __device__ static __forceinline__ int swz(int row) {
        static_assert(LPR == 16 || LPR == 8, "D must be 64 or 128");
        if constexpr (LPR == 16) return ((row & 3) << 2) | ((row & 4) >> 1);
        return ((row >> 1) & 1) | ((row >> 2) & 1) << 2 | ((row >> 3) & 1) << 1;
    }

    __amdgpu_buffer_rsrc_t rk, rv;  // K and V of this (b, g), byte-addressed
    unsigned lane_off[NV];          // lane part of the offset for instruction s % NV
    unsigned row_bytes;             // bytes between consecutive keys (G * D * 2)
    int N;

    __device__ __forceinline__ void init(const _Float16 *Kg, const _Float16 *Vg, unsigned bytes,
                                         int row_stride, int n_keys, int lane) {
        rk = __builtin_amdgcn_make_buffer_rsrc((void *)Kg, (short)0, (int)bytes, 0x00020000);
        rv = __builtin_amdgcn_make_buffer_rsrc((void *)Vg, (short)0, (int)bytes, 0x00020000);
        row_bytes = (unsigned)row_stride * 2u;
        N = n_keys;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int row = v * RPI + lane / LPR;
            lane_off[v] = (unsigned)(lane / LPR) * row_bytes + (unsigned)(((lane % LPR) ^ swz(row)) * 16);
        }
    }

    typedef __attribute__((address_space(3))) _Float16 lds_half;

    __device__ static __forceinline__ void copy(__amdgpu_buffer_rsrc_t rs, lds_half *lds, unsigned voff,
                                                unsigned soff, int s) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)(lds + s * (kWaveSize * 8)), 16, voff, soff, 0, 0);
    }

    // Issues the copy of block t of K (rs = rk) or V (rs = rv) into buf;
    // completes on vmcnt.
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, _Float16 *buf_generic, int t,
                                          int lane) const {
        lds_half *buf = (lds_half *)buf_generic;  // one address-space conversion per block
        if (t * BS + BS <= N) {
            const unsigned base = (unsigned)(t * BS) * row_bytes;
#pragma unroll
            for (int s = 0; s < NI; ++s)
                copy(rs, buf, lane_off[s % NV], base + (unsigned)(s * RPI) * row_bytes, s);
        } else {
            // Last, partial block: clamp rows past the end into bounds (they are
            // masked out of the softmax), with the whole offset per lane.
#pragma unroll
            for (int s = 0; s < NI; ++s) {
                const int row = s * RPI + lane / LPR;
                int n = t * BS + row;
                n = n < N ? n : N - 1;
                const unsigned off = (unsigned)n * row_bytes + (unsigned)(((lane % LPR) ^ swz(row)) * 16);
                copy(rs, buf, off, 0u, s);
            }
        }
    }

    // Issues only instruction i (0 <= i < NI) of block t's copy, rows
    // i*RPI .. i*RPI+RPI-1, so that several wavefronts can share one copy.
    __device__ __forceinline__ void issue_part(__amdgpu_buffer_rsrc_t rs, _Float16 *buf_generic, int t, int i,
                                               int lane) const {
        lds_half *buf = (lds_half *)buf_generic;
        const int row = i * RPI + lane / LPR;
        int n = t * BS + row;
        n = n < N ? n : N - 1;  // rows past the end are clamped (and masked later)
        const unsigned off = (unsigned)(n - t * BS) * row_bytes + (unsigned)(((lane % LPR) ^ swz(row)) * 16);
        copy(rs, buf, off, (unsigned)(t * BS) * row_bytes, i);
    }

    // MFMA A-operand fragments of one staged block: lane l gets row
    // 16*kt + l%16, head-dim 32*c + 8*(l/16) .. +7.  The reads are issued
    // as one inline-asm batch that ends in its own lgkmcnt(0) wait: the
    // compiler would otherwise guard every LDS read with vmcnt(0), i.e.
    // wait for all copies in flight, including the other buffer's.
    __device__ static __forceinline__ void read(half8 (&f)[BS / 16][D / 32], const _Float16 *buf, int r,
                                                int q4) {
        const unsigned base = (unsigned)(size_t)(const __attribute__((address_space(3))) _Float16 *)buf;
        unsigned a[D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c) a[c] = base + (unsigned)(r * D + ((c * 4 + q4) ^ swz(r)) * 8) * 2;
        LdsBatch<BS, D>::run(f, a);
    }

    // V^T operands of one staged block for the PV MFMAs (see LdsTrBatch).
    __device__ static __forceinline__ void read_vt(half4 (&f)[BS / 32][D / 32][2][2], const _Float16 *buf,
                                                   int lane) {
        const unsigned base = (unsigned)(size_t)(const __attribute__((address_space(3))) _Float16 *)buf;
        const int q4 = lane >> 4, a = lane & 3, j = (lane >> 2) & 3;
        const int row = 4 * q4 + j;  // row within a 16-row group; the group offset is immediate
        unsigned addr[D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
            addr[c] = base + (unsigned)(row * D * 2 + ((4 * c + a) ^ swz(row)) * 16);
        LdsTrBatch<BS, D>::run(f, addr);
    }
};

// The queries of one wavefront slot: QW consecutive positions m0 .. m0+nq-1
// of one (b, g).  A merger yields the union of their counted index entries in
// ascending block order (for any row order) together with the mask of the
// queries whose rows hold that block.

// Any T (rows of any length): a per-wavefront map in LDS with one byte per
// block, bit k set when query k of the slot selects the block, built for a
// window of kMapBlocks blocks at a time from every counted entry of the rows
// and walked in ascending order (a 256-block chunk per step: lane l holds
// blocks 4l .. 4l+3 of the chunk in one register, a ballot marks the lanes
// with a block left).  A block that a row repeats, or that several rows
// select, is returned once, for any row order, as by RegMerger.  The map's
// LDS accesses are inline assembly so the compiler does not guard them with
// waits for the direct-to-LDS copies in flight.
constexpr int kMapBlocks = 2048;  // bytes of LDS per wavefront

template <int QW, int BS>
struct MapMerger {
    static_assert(QW <= 8, "the query mask takes one byte");
    const int32_t *rows;  // index row of query m0
    int row_stride;       // elements between consecutive queries' rows (G * T)
    int T, m0, nq, NB, lane;
    unsigned base;        // LDS byte address of the map
    int lo, lim;          // window start; one past the last block any query may select
    int cb;               // first block of the loaded chunk
    unsigned word;        // this lane's four blocks of the chunk
    uint64_t nz;          // lanes with a block left in the chunk

    __device__ __forceinline__ void init(const Params &p, int b, int g, int m0_, int nq_, int lane_, void *lds) {
        rows = p.idx + ((size_t)(b * (size_t)p.M + m0_) * p.G + g) * p.T;
        row_stride = p.G * p.T;
        T = p.T;
        m0 = m0_;
        nq = nq_;
        NB = p.NB;
        lane = lane_;
        base = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)lds;
        lim = min(NB, (m0 + nq - 1) / BS + 1);
        lo = 0;
        build();
    }
    // Map of blocks lo .. lo + kMapBlocks - 1 from every counted entry.
    __device__ __forceinline__ void build() {
        const int4v zero = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kMapBlocks / (kWaveSize * 16); ++i)
            asm volatile("ds_write_b128 %0, %1" ::"v"(base + (unsigned)(i * kWaveSize + lane) * 16u), "v"(zero)
                         : "memory");
#pragma unroll
        for (int k = 0; k < QW; ++k) {
            if (k >= nq) break;
            const int32_t *row = rows + (size_t)k * row_stride;
            const int cm = (m0 + k) / BS;
            for (int e0 = 0; e0 < T; e0 += kWaveSize) {
                const int e = e0 + lane;
                const int t = e < T ? __builtin_nontemporal_load(&row[e]) : -1;
                const int d = t - lo;
                if (t >= 0 && t <= cm && t < NB && d >= 0 && d < kMapBlocks) {
                    const unsigned bits = (1u << k) << (8 * (d & 3));
                    asm volatile("ds_or_b32 %0, %1" ::"v"(base + (unsigned)(d & ~3)), "v"(bits) : "memory");
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        cb = lo - 4 * kWaveSize;
        word = 0;
        nz = 0;
    }
    __device__ __forceinline__ int next(unsigned &active) {
        for (;;) {
            if (nz) {
                const int l = __builtin_ctzll(nz);
                const unsigned w = (unsigned)__builtin_amdgcn_readlane((int)word, l);
                const int bi = __builtin_ctz(w) >> 3;
                active = (w >> (8 * bi)) & 0xffu;
                if (lane == l) word &= ~(0xffu << (8 * bi));
                nz = __ballot(word != 0u);
                return cb + 4 * l + bi;
            }
            cb += 4 * kWaveSize;
            if (cb >= lim) {
                active = 0;
                return kDone;
            }
            if (cb >= lo + kMapBlocks) {  // next window
                lo += kMapBlocks;
                build();
                continue;
            }
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                         : "=v"(word)
                         : "v"(base + (unsigned)(cb - lo) + (unsigned)lane * 4u)
                         : "memory");
            nz = __ballot(word != 0u);
        }
    }
};

// Wave-wide reductions over 64 lanes: DPP prefix within each 16-lane row,
// then the four row results.
__device__ __forceinline__ int wave_min(int x) {
    x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x111, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x112, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x114, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(INT_MAX, x, 0x118, 0xf, 0xf, false));
    const int a = __builtin_amdgcn_readlane(x, 15), b = __builtin_amdgcn_readlane(x, 31);
    const int c = __builtin_amdgcn_readlane(x, 47), d = __builtin_amdgcn_readlane(x, 63);
    return min(min(a, b), min(c, d));
}
__device__ __forceinline__ unsigned wave_or(unsigned x) {
    x |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
    x |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
    x |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
    x |= (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
    return (unsigned)(__builtin_amdgcn_readlane((int)x, 15) | __builtin_amdgcn_readlane((int)x, 31) |
                      __builtin_amdgcn_readlane((int)x, 47) | __builtin_amdgcn_readlane((int)x, 63));
}

// Holds all QW*T entries (QW*T <= 128) in two registers per lane: entry
// e = lane + 64*v belongs to query e / T.  Each step takes the smallest
// remaining counted block and retires every entry equal to it, so a block
// repeated within a row, or shared by several rows, is returned once.  An
// entry holds (block << 4) | query (QW <= 8), so the wave-wide minimum is the
// smallest block and the mask of the queries holding it comes from the
// entries themselves: no per-lane query masks to keep live across the loop
// (spilled, their reloads waited on every copy in flight).
template <int QW, int BS>
struct RegMerger {
    static_assert(QW <= 16, "the query index takes 4 bits");
    int e[2];

    __device__ __forceinline__ void init(const Params &p, int b, int g, int m0, int nq, int lane, void *) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int ent = lane + 64 * v;
            const int qi = ent / p.T;
            const bool slot = ent < QW * p.T && qi < nq;
            const int m = m0 + (slot ? qi : 0);
            const int32_t *row = p.idx + ((size_t)(b * (size_t)p.M + m) * p.G + g) * p.T;
            const int t = slot ? __builtin_nontemporal_load(&row[ent - qi * p.T]) : -1;
            const bool ok = t >= 0 && t <= m / BS && t < p.NB;  // NB < 2^27: (t << 4) fits
            e[v] = ok ? (t << 4) | qi : INT_MAX;
        }
    }
    __device__ __forceinline__ int next(unsigned &active) {
        const int x = wave_min(min(e[0], e[1]));
        active = 0;
        if (x == INT_MAX) return kDone;
        const int t = x >> 4;
        const bool h0 = (e[0] >> 4) == t, h1 = (e[1] >> 4) == t;
        active = wave_or((h0 ? 1u << (e[0] & 15) : 0u) | (h1 ? 1u << (e[1] & 15) : 0u));
        e[0] = h0 ? INT_MAX : e[0];
        e[1] = h1 ? INT_MAX : e[1];
        return t;
    }
};

// s_waitcnt immediate for "at most n vector-memory ops outstanding"
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Workgroup barrier for LDS traffic between wavefronts: waits for this
// wavefront's own LDS operations, then s_barrier.  Unlike __syncthreads() it
// does not wait for outstanding global loads, so copies already issued stay
// in flight across it.  The memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Score and accumulate steps shared by the selection and dense kernels.

__device__ __forceinline__ float4v mfma_16x16x32(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}


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

// Element-type-generic steps: BF16 selects bfloat16 operands (MFMA bf16,
// round-to-nearest-even packing), else fp16.
template <bool BF16>
__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                        c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ half4 pack4(float4v v) {
    if constexpr (BF16) {
        bf16x4 r;
        r[0] = (__bf16)v[0];
        r[1] = (__bf16)v[1];
        r[2] = (__bf16)v[2];
        r[3] = (__bf16)v[3];
        return __builtin_bit_cast(half4, r);
    } else {
        return to_half4(v);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum over the four lanes l%16 + 16*j of an MFMA result (one column)
// with the gfx950 row-swap permutes, which stay in VALU: permlane16_swap with
// both operands x leaves rows (0, 0, 2, 2) in the first result and (1, 1, 3,
// 3) in the second, permlane32_swap the low and the high half likewise.
__device__ __forceinline__ float col_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// S^T = K Q^T of one 16-column tile over a staged sub-block: lane l holds
// keys 16*kt + 4*(l/16) + i of column l%16.
template <int SBS, int D, bool BF16>
__device__ __forceinline__ void qk_tile(const half8 (&kf)[SBS / 16][D / 32], const half8 (&qf)[D / 32],
                                        float4v (&s)[SBS / 16]) {
#pragma unroll
    for (int kt = 0; kt < SBS / 16; ++kt) {
        s[kt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) s[kt] = mfma16<BF16>(kf[kt][c], qf[c], s[kt]);
    }
}

// Scores of one gathered block folded into the running softmax state: the
// running max, the rescale factor of the accumulator and the block's
// probabilities P^T (fp16), all in the log2 domain (x * log2(e) / sqrt(D)).
// s holds S^T from qk_tile (keys key0 + 16*kt + 4*q4 + i) and is overwritten.
//
// causal: the block reaches past the smallest packed query or past N (or,
//   for a sliding window, before some column's first visible key), so keys
//   outside the column's visible range [lo, lim] are masked to -inf (the
//   caller forms lo and lim once; lim = min(its query, N - 1) for causal
//   attention, lo = INT_MIN when there is no lower bound).
// col_mask: some packed query did not select this block; for those columns
//   (col_on false) the running state is left unchanged and P is zero.
// The running max is only raised when a block's max exceeds it by more than
// kLazyMax (P then stays below 2^kLazyMax, well inside fp16), so most blocks
// need no rescale of the accumulator (alpha == 1 exactly).  That is tested
// first, lane by lane, against each column's running max: when no lane's
// scaled scores exceed it by more than kLazyMax (a wave-uniform test), P
// follows with the running max as it stands and no reduction over a column.
// Otherwise -- and on a column's first block, where the running max is -inf
// -- the step takes each column's block max over its four lanes.  Both ways
// give the same P wherever the running max is kept.
constexpr float kLazyMax = 8.0f;

// The lanes whose column belongs to a query set in tbits (bit q: query q of
// a 16-column tile, columns q*gs .. q*gs+gs-1 of each 16-lane row), as a
// wave-wide mask built on the scalar unit.
template <int PACK>
__device__ __forceinline__ uint64_t col_lanes(unsigned tbits, int gs) {
    const unsigned g = (1u << gs) - 1u;
    unsigned m16 = 0;
#pragma unroll
    for (int q = 0; q < PACK; ++q)
        if ((tbits >> q) & 1u) m16 |= g << (q * gs);
    const uint64_t m32 = (uint64_t)(m16 | (m16 << 16));
    return m32 | (m32 << 32);
}

// Per lane: if1 where the lane's bit of mask is set, else if0 (one
// v_cndmask with the mask in scalar registers).
__device__ __forceinline__ float select_lanes(uint64_t mask, float if0, float if1) {
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if0), "v"(if1), "s"(mask));
    return r;
}

// LO: keys below lo are masked too (a window's left edge); without it lo is
// ignored and the test is against lim alone, relative to the lane's first
// key, so that nothing per score is computed outside the masked branch.
// SMASK: the columns taking part are the lanes set in on_lanes (a scalar
// mask) instead of those with col_on (col_mask and col_on are then unused).
template <int KT, bool BF16 = false, bool LO = true, bool SMASK = false>
__device__ __forceinline__ void softmax_tile(float4v (&s)[KT], int key0, bool causal, bool col_mask, bool col_on,
                                             int lo, int lim, float scale_log2, float &m_run, float &l_run,
                                             float &alpha, half4 (&pf)[KT], int q4, uint64_t on_lanes = 0) {
    if (causal) {
        if constexpr (LO) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + kt * 16 + q4 * 4 + i;
                    if (key > lim || key < lo) s[kt][i] = -INFINITY;
                }
        } else {
            const int hi_rel = lim - (key0 + q4 * 4);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kt * 16 + i > hi_rel) s[kt][i] = -INFINITY;
        }
    }
    const bool off = col_mask && !col_on;
    // if_off for a column left out of this block, else if_on.
    auto pick = [&](float if_off, float if_on) -> float {
        if constexpr (SMASK)
            return select_lanes(on_lanes, if_off, if_on);
        else
            return off ? if_off : if_on;
    };
    {
        const float m_keep = pick(INFINITY, m_run);
        float x[KT][4];
        float xmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[kt][i] = __builtin_fmaf(s[kt][i], scale_log2, -m_keep);
            xmax = fmaxf(xmax, fmaxf(fmaxf(x[kt][0], x[kt][1]), fmaxf(x[kt][2], x[kt][3])));
        }
        // Two ballots of plain compares (one of the combined condition makes
        // the compiler round-trip it through a vector register).
        if (!(__builtin_amdgcn_ballot_w64(xmax > kLazyMax) | __builtin_amdgcn_ballot_w64(m_keep == -INFINITY))) {
            float psum;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                float4v pv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = fast_exp2(x[kt][i]);
                    psum = (kt == 0 && i == 0) ? pv[i] : psum + pv[i];
                }
                pf[kt] = pack4<BF16>(pv);
            }
            alpha = 1.f;
            l_run += psum;
            return;
        }
    }
    // Row max of the raw scores (the scale is positive), then over the 4
    // lanes (l, l^16, l^32, l^48) that share a column.
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) mloc = fmaxf(mloc, fmaxf(fmaxf(s[kt][0], s[kt][1]), fmaxf(s[kt][2], s[kt][3])));
    mloc = col_max(mloc);
    const float m_blk = mloc * scale_log2;
    const float m_new = pick(m_run, (m_blk > m_run + kLazyMax) ? m_blk : m_run);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_use);
    m_run = m_new;
    // A column left out of this block gets P = exp2(-inf) = 0.
    const float m_exp = pick(INFINITY, m_use);
    float psum;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        float4v pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = fast_exp2(__builtin_fmaf(s[kt][i], scale_log2, -m_exp));
            psum = (kt == 0 && i == 0) ? pv[i] : psum + pv[i];
        }
        pf[kt] = pack4<BF16>(pv);
    }
    l_run = l_run * alpha + psum;  // per-lane partial; lanes are summed at the end
}

// qk_tile and softmax_tile in one step.
template <int BS, int D, bool BF16 = false, bool LO = true, bool SMASK = false>
__device__ __forceinline__ void score_block(const half8 (&kf)[BS / 16][D / 32], const half8 (&qf)[D / 32],
                                            int key0, bool causal, bool col_mask, bool col_on, int lo, int lim,
                                            float scale_log2, float &m_run, float &l_run,
                                            float &alpha, half4 (&pf)[BS / 16], int q4, uint64_t on_lanes = 0) {
    float4v s[BS / 16];
    qk_tile<BS, D, BF16>(kf, qf, s);
    softmax_tile<BS / 16, BF16, LO, SMASK>(s, key0, causal, col_mask, col_on, lo, lim, scale_log2, m_run, l_run,
                                           alpha, pf, q4, on_lanes);
}

// O^T = alpha * O^T + V^T * P^T over 32-key chunks.  acc[c][hh] holds O^T rows
// d = 32*c + 8*(l/16) + 4*hh + i for head l%16.  The B operand is P^T straight
// from the score layout; the A operand V^T comes from the transposing reads.
template <int BS, int D, bool BF16 = false>
__device__ __forceinline__ void accumulate_block(const half4 (&vt)[BS / 32][D / 32][2][2],
                                                 const half4 (&pf)[BS / 16], float alpha,
                                                 float4v (&acc)[D / 32][2]) {
    constexpr int DC = D / 32;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // wave-uniform: some column rescales
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            acc[c][0] *= alpha;
            acc[c][1] *= alpha;
        }
    }
#pragma unroll
    for (int kc = 0; kc < BS / 32; ++kc) {
        const half8 bp = cat8(pf[2 * kc], pf[2 * kc + 1]);
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                acc[c][hh] = mfma16<BF16>(cat8(vt[kc][c][hh][0], vt[kc][c][hh][1]), bp, acc[c][hh]);
    }
}

// The queries of wavefront slot ws: m0 .. m0 + nq - 1 of one (b, g).  Slots
// are numbered (b, g)-major, so a contiguous slot range walks consecutive
// queries of few groups.
struct Slot {
    int b, g, m0, nq;
};
__device__ __forceinline__ Slot decode_slot(const Params &p, int ws, int qw) {
    Slot s;
    const int bg = ws / p.wslots_per_bg;
    s.m0 = (ws - bg * p.wslots_per_bg) * qw;
    s.nq = min(qw, p.M - s.m0);
    s.g = bg % p.G;
    s.b = bg / p.G;
    return s;
}

// Wavefront slot of wavefront `wave` of this workgroup, or -1.  Workgroup
// blockIdx.x belongs to generation p.gen + blockIdx.x / wg_per_gen; within a
// generation, XCD w % nxcd runs the next gen_step slots of its contiguous
// range, so one generation fills every workgroup slot of every CU.
template <int WAVES>
__device__ __forceinline__ int wave_slot(const Params &p, int wave) {
    const int gen = p.gen + (int)blockIdx.x / p.wg_per_gen;
    const int w = (int)blockIdx.x - (gen - p.gen) * p.wg_per_gen;
    const int loc = gen * p.gen_step + (w / p.nxcd) * WAVES + wave;
    const int ws = (w % p.nxcd) * p.per_xcd + loc;
    return (loc >= p.per_xcd || ws >= p.wslots) ? -1 : ws;
}

// Persistent launch.  One workgroup per workgroup slot of the device instead
// of one launch per generation: the workgroups of XCD x (w % nxcd == x, as
// the dispatcher deals them) run one generation of slots per step.  At every
// step they meet at a barrier of their XCD, so that its wavefronts start
// together and sweep key space in step, as a generation launch makes them;
// the last workgroup to arrive claims the step's generation -- the next one
// of the XCD's own range or, once that range is used up, the next one of
// another range -- and publishes it.  XCDs then advance independently, and
// one whose range runs fast takes generations over from slow ones, where a
// generation launch makes every XCD wait for the slowest.
//
// 32-bit words at p.sched, cleared by sched_clear_kernel before the launch:
//   taken[r]      word 32 * r: generations of range r claimed so far
//   arrive[x][s]  word 32 * nxcd + x * steps_max + s: workgroups of XCD x that
//                 reached step s
//   claim[x][s]   word 32 * nxcd + (nxcd + x) * steps_max + s: the generation
//                 of step s (kSchedValid | r << 20 | j), kSchedFinished, or
//                 kSchedEmpty / kSchedClaiming while it is not yet known
// Every wait is bounded.  A workgroup that waits at the barrier for more than
// kAlignSpin polls claims the step itself; whoever claims a step, each of its
// slots runs once, with the same code, so workgroups that are not all
// resident at once cost time, never correctness.  The atomics are
// device-scope: the ranges are claimed across XCDs.
constexpr unsigned kSchedEmpty = 0, kSchedClaiming = 1, kSchedFinished = 2, kSchedValid = 0x80000000u;
constexpr int kAlignSpin = 400;     // about 0.5 ms of polls
constexpr int kClaimSpin = 1 << 20;  // a claim in progress ends after at most nxcd atomics

__device__ __forceinline__ unsigned sched_add(unsigned *a) {
    return __hip_atomic_fetch_add(a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned sched_load(unsigned *a) {
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The generation of step s for XCD x, as seen by one lane (lane 0 of
// wavefront 0 of a workgroup: the code runs with that lane alone active).
// Returns kSchedFinished or kSchedValid | r << 20 | j.
__device__ __forceinline__ unsigned sched_step(const Params &p, int x, int s) {
    unsigned *arrive = p.sched + 32 * p.nxcd + x * p.steps_max + s;
    unsigned *claim = p.sched + 32 * p.nxcd + (p.nxcd + x) * p.steps_max + s;
    const unsigned wgs = (unsigned)(p.wg_per_gen / p.nxcd);
    if (sched_add(arrive) + 1 < wgs) {  // not the last to arrive: wait for the claim
#pragma unroll 1
        for (int it = 0; it < kAlignSpin; ++it) {
            const unsigned v = sched_load(claim);
            if (v >= kSchedFinished) return v;
            __builtin_amdgcn_s_sleep(8);
        }
    }
    unsigned prev = kSchedEmpty;
    __hip_atomic_compare_exchange_strong(claim, &prev, kSchedClaiming, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    if (prev == kSchedEmpty) {  // this workgroup claims the step
        unsigned res = kSchedFinished;
#pragma unroll 1
        for (int d = 0; d < p.nxcd; ++d) {
            const int r = (x + d) % p.nxcd;
            const unsigned j = sched_add(p.sched + 32 * r);
            if (j < (unsigned)p.gens) {
                res = kSchedValid | ((unsigned)r << 20) | j;
                break;
            }
        }
        __hip_atomic_store(claim, res, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return res;
    }
    if (prev >= kSchedFinished) return prev;
#pragma unroll 1
    for (int it = 0; it < kClaimSpin; ++it) {  // another workgroup is claiming
        const unsigned v = sched_load(claim);
        if (v >= kSchedFinished) return v;
        __builtin_amdgcn_s_sleep(2);
    }
    return kSchedFinished;  // not reached: the claimer stores after at most nxcd atomics
}

// The persistent loop of one workgroup: run(ws) for its wavefront's slot of
// each generation the XCD is given.  One lane of the workgroup takes part in
// the schedule; the wavefronts wait for it at the workgroup barrier.
template <int WAVES, class Run>
__device__ __forceinline__ void run_persistent(const Params &p, int wave, int lane, Run &&run) {
    __shared__ unsigned step_claim;
    const int x = (int)blockIdx.x % p.nxcd;
    const int i = ((int)blockIdx.x / p.nxcd) * WAVES + wave;
    for (int s = 0; s < p.steps_max; ++s) {
        __syncthreads();  // every wavefront of the workgroup is done with step s - 1
        if (wave == 0 && lane == 0) step_claim = sched_step(p, x, s);
        __syncthreads();
        const unsigned v = __builtin_amdgcn_readfirstlane(step_claim);
        if (v == kSchedFinished) return;
        const int r = (int)((v >> 20) & 0x7ffu), j = (int)(v & 0xfffffu);
        const int loc = j * p.gen_step + i;
        const int ws = r * p.per_xcd + loc;
        if (r < p.nxcd && loc < p.per_xcd && ws < p.wslots) run(ws);
    }
}

__global__ void sched_clear_kernel(unsigned *w, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) w[i] = 0u;
}

// Buffer descriptors of K and V for (b, g): the range runs from the group's
// first row to the end of the tensor.  b and g are wave-uniform; reading them
// through readfirstlane keeps the descriptors in scalar registers (without
// it the compiler may place them in vector registers and wrap every copy in a
// loop over distinct descriptor values).
template <int SBS, int D>
__device__ __forceinline__ void init_stage(Stage<SBS, D> &st, const Params &p, int b, int g, int lane) {
    b = __builtin_amdgcn_readfirstlane(b);
    g = __builtin_amdgcn_readfirstlane(g);
    const _Float16 *Kg = p.K + ((size_t)b * p.N * p.G + g) * D;
    const _Float16 *Vg = p.V + ((size_t)b * p.N * p.G + g) * D;
    const size_t kv_elems = (size_t)p.B * p.N * p.G * D;
    const size_t first = ((size_t)b * p.N * p.G + g) * D;
    const size_t bytes = (kv_elems - first) * 2;
    st.init(Kg, Vg, (unsigned)(bytes < 0xFFFFFFFFu ? bytes : 0xFFFFFFFFu), p.G * D, p.N, lane);
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Compute units and XCDs of the current device, cached per device (the first
// call on a device asks the runtime).  The launch plans deal workgroup w to
// XCD w % nxcd, the order in which the hardware spreads a grid over the XCDs
// of a device that is not partitioned; an XCD count the runtime does not give,
// or one that does not divide the CUs evenly, falls back to nxcd = 1 (one
// contiguous range of work: correct everywhere, without the L2 locality).  A
// failed CU query falls back to 256.
struct Topology {
    int cus, nxcd, l2;  // l2: bytes of one XCD's L2 (the device attribute reports it per XCD)
};
Topology device_topology() {
    static std::atomic<int> cached_cus[64], cached_xcd[64], cached_l2[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    Topology t{cached_cus[dev].load(std::memory_order_relaxed), cached_xcd[dev].load(std::memory_order_relaxed),
               cached_l2[dev].load(std::memory_order_relaxed)};
    if (t.cus <= 0 || t.nxcd <= 0 || t.l2 <= 0) {
        if (hipDeviceGetAttribute(&t.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || t.cus <= 0)
            t.cus = 256;
        if (hipDeviceGetAttribute(&t.nxcd, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || t.nxcd < 1 ||
            t.nxcd > 64 || t.cus % t.nxcd != 0)
            t.nxcd = 1;
        if (hipDeviceGetAttribute(&t.l2, hipDeviceAttributeL2CacheSize, dev) != hipSuccess || t.l2 <= 0)
            t.l2 = 4 << 20;
        cached_cus[dev].store(t.cus, std::memory_order_relaxed);
        cached_xcd[dev].store(t.nxcd, std::memory_order_relaxed);
        cached_l2[dev].store(t.l2, std::memory_order_relaxed);
    }
    return t;
}


// Host-side argument checks shared by the entry points: sizes, supported
// configurations and index ranges.  Fills the size fields of p and the
// queries per 16-column tile (pack).  Makes no HIP call.  Returns an
// NSA_SEL_* status.
int check_sizes(int B, int M, int N, int H, int G, int D, int block_size, int T, Params &p) {
    if (B < 1 || M < 1 || N < 1 || H < 1 || G < 1 || D < 1 || block_size < 1 || T < 1)
        return NSA_SEL_ERR_SHAPE;
    if (H % G != 0) return NSA_SEL_ERR_SHAPE;
    const int gs = H / G;
    if ((D != 64 && D != 128) || (block_size != 32 && block_size != 64) || gs > 16)
        return NSA_SEL_ERR_UNSUPPORTED;
    // Unit ids, slot ids and per-(b, g) element offsets use int.
    if ((int64_t)B * M * G > INT_MAX || (int64_t)N * G * D > INT_MAX) return NSA_SEL_ERR_RANGE;
    p.B = B; p.M = M; p.N = N; p.H = H; p.G = G; p.T = T; p.gs = gs;
    p.NB = (N + block_size - 1) / block_size;
    // Queries per tile: as many whole groups of gs heads as fit 16 columns,
    // rounded down to 1, 2 or 4.
    p.pack = (16 / gs) >= 4 ? 4 : (16 / gs) >= 2 ? 2 : 1;
    p.scale_log2 = kLog2e / sqrtf((float)D);
    p.gen = 0;
    p.gen_step = 0;
    p.wg_per_gen = 1;
    p.nxcd = 1;
    p.l2_bytes = 0;
    p.sched = nullptr;
    p.sched_cap = 0;
    p.gens = 0;
    p.steps_max = 0;
    return NSA_SEL_OK;
}

// Tiles per wavefront (mode) and the slot layout, for a device with `cus`
// compute units.  Measured on MI355X: up to two tiles, while the index rows
// of the wavefront's queries fit in two registers per lane (else one tile
// with streamed rows), and fewer while the grid would give a CU less than 8
// wavefront slots.  Two tiles keep a wavefront within 256 registers, so two
// wavefronts share each SIMD.
// max_mode caps the tiles per wavefront.
void plan_slots(Params &p, const Topology &tp, int max_mode = 2) {
    const int cus = tp.cus;
    p.nxcd = tp.nxcd;
    p.l2_bytes = tp.l2;
    int mode = 0;
    for (int nt = max_mode; nt >= 1; nt /= 2) {
        if ((int64_t)p.pack * nt * p.T <= 128) {
            mode = nt;
            break;
        }
    }
    while (mode > 1 && (int64_t)p.B * p.G * ((p.M + p.pack * mode - 1) / (p.pack * mode)) < 8LL * cus) mode /= 2;
    const int qw = p.pack * (mode > 0 ? mode : 1);
    const int64_t wslots_per_bg = ((int64_t)p.M + qw - 1) / qw;
    const int64_t wslots = (int64_t)p.B * p.G * wslots_per_bg;
    p.mode = mode;
    p.wslots_per_bg = (int)wslots_per_bg;
    p.wslots = (int)wslots;
    p.per_xcd = (int)((wslots + p.nxcd - 1) / p.nxcd);
}

// Queries per wavefront slot of a planned launch.
int slot_queries(const Params &p) { return p.pack * (p.mode > 0 ? p.mode : 1); }

// Schedule words of a persistent launch planned in p.
int64_t sched_words(const Params &p) { return 32 * (int64_t)p.nxcd + 2 * (int64_t)p.nxcd * p.steps_max; }

// Upper bound of sched_words for p after plan_slots on a device with `cus`
// compute units, whatever the kernel's occupancy: a generation holds at
// least one wavefront per CU.
int64_t sched_words_bound(const Params &p, int cus) {
    const int64_t per_gen = cus / p.nxcd > 0 ? cus / p.nxcd : 1;
    const int64_t gens = (p.per_xcd + per_gen - 1) / per_gen;
    return 32 * (int64_t)p.nxcd + 2 * (int64_t)p.nxcd * (p.nxcd * gens + 1);
}

// Workgroups of `kernel` (`threads` threads, static LDS only) that one CU holds
// at once, from the HIP occupancy calculator, cached per device in `cache`;
// 0 when unknown.
int resident_workgroups(std::atomic<int> (&cache)[64], const void *kernel, int threads) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Launch chain, generic over a kernel family: f.launch<BS, SPLIT, D, PACK,
// MODE>(grid, block, stream, params) queues one generation (or, from
// p.gen, as many as the grid holds), f.launch_persist<...>(...) the
// persistent kernel, and f.resident<...>() gives how many of the persistent
// kernel's workgroups one CU holds (0: unknown).
//
// Generations are queued in order on the stream.  Every generation starts all
// its workgroups together and ends before the next starts, so the slots
// resident on an XCD sweep key space in step and share its L2.  With a
// schedule buffer (p.sched) the persistent kernel keeps that step per XCD
// instead (see run_persistent).
template <class F, int BS, int SPLIT, int D, int PACK, int MODE>
hipError_t launch_generations(const F &f, Params p, int cus, hipStream_t stream) {
    // One generation fills every workgroup slot of every CU: the staging
    // buffers (K and V, one sub-block each per wavefront, plus the block map
    // of MODE 0) set how many workgroups fit the CU's 160 KiB of LDS.
    constexpr int WAVES = waves_per_wg(BS / SPLIT);
    constexpr int lds_per_wg = (2 * Stage<BS / SPLIT, D>::HALVES * 2 + (MODE == 0 ? kMapBlocks : 0)) * WAVES;
    constexpr int by_lds = 160 * 1024 / lds_per_wg;
    constexpr int wg_per_cu = by_lds < 4 ? (by_lds > 0 ? by_lds : 1) : 4;
    const int wg_per_xcd = (cus / p.nxcd > 0 ? cus / p.nxcd : 1) * wg_per_cu;
    p.gen_step = wg_per_xcd * WAVES;
    p.wg_per_gen = wg_per_xcd * p.nxcd;
    const int gens = (p.per_xcd + p.gen_step - 1) / p.gen_step;
    // One launch per generation keeps the wavefronts resident on an XCD
    // sweeping one group's K/V together, which is what its L2 hits come
    // from.  When one (b, g)'s K and V fit an XCD's L2 that sweep buys
    // nothing, and a single launch carrying every generation lets the next
    // generation's workgroups fill the tail of the previous one.
    const bool one_launch = (int64_t)p.N * D * 2 * 2 <= (int64_t)p.l2_bytes;
    if constexpr (F::kPersistent) {
    if (p.sched && !one_launch) {
        // One workgroup per slot that is resident at once: a barrier of the
        // XCD waits for all of them.
        const int occ = f.template resident<BS, SPLIT, D, PACK, MODE>();
        const int per_cu = occ > 0 && occ < wg_per_cu ? occ : wg_per_cu;
        Params q = p;
        const int wxcd = (cus / q.nxcd > 0 ? cus / q.nxcd : 1) * per_cu;
        q.gen_step = wxcd * WAVES;
        q.wg_per_gen = wxcd * q.nxcd;
        q.gens = (q.per_xcd + q.gen_step - 1) / q.gen_step;
        q.steps_max = q.nxcd * q.gens + 1;
        q.gen = 0;
        if (q.gens < (1 << 20) && sched_words(q) <= q.sched_cap) {
            const int n = (int)sched_words(q);
            hipLaunchKernelGGL(sched_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, q.sched, n);
            f.template launch_persist<BS, SPLIT, D, PACK, MODE>(dim3(q.wg_per_gen), dim3(kWaveSize * WAVES), stream,
                                                                q);
            return hipGetLastError();
        }
    }
    }
    const int per_launch = one_launch ? gens : 1;
    for (int g = 0; g < gens; g += per_launch) {
        p.gen = g;
        f.template launch<BS, SPLIT, D, PACK, MODE>(dim3(p.wg_per_gen * per_launch), dim3(kWaveSize * WAVES), stream,
                                                    p);
    }
    return hipGetLastError();
}

// 64-key blocks are always staged as two 32-key halves.
template <class F, int BS, int D, int PACK>
hipError_t launch_mode(const F &f, const Params &p, int cus, hipStream_t stream) {
    constexpr int SPLIT = BS / 32;
    switch (p.mode) {
        case 2: return launch_generations<F, BS, SPLIT, D, PACK, 2>(f, p, cus, stream);
        case 1: return launch_generations<F, BS, SPLIT, D, PACK, 1>(f, p, cus, stream);
        default: return launch_generations<F, BS, SPLIT, D, PACK, 0>(f, p, cus, stream);
    }
}

template <class F, int BS, int D>
hipError_t launch_pack(const F &f, const Params &p, int cus, hipStream_t stream) {
    if (p.pack == 4) return launch_mode<F, BS, D, 4>(f, p, cus, stream);
    if (p.pack == 2) return launch_mode<F, BS, D, 2>(f, p, cus, stream);
    return launch_mode<F, BS, D, 1>(f, p, cus, stream);
}

template <class F>
hipError_t launch_all(const F &f, const Params &p, int block_size, int D, int cus, hipStream_t stream) {
    if (block_size == 64)
        return (D == 128) ? launch_pack<F, 64, 128>(f, p, cus, stream) : launch_pack<F, 64, 64>(f, p, cus, stream);
    return (D == 128) ? launch_pack<F, 32, 128>(f, p, cus, stream) : launch_pack<F, 32, 64>(f, p, cus, stream);
}

}  // namespace
