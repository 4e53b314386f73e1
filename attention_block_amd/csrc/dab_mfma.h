// Matrix-core row panels for batches of 8 or more (bf16, gfx950, wave64).
//
// A panel is TILES tiles of 16 weight rows (W stored [N, K], one output
// feature per row) against 16 * NG sequences, all of K, in one workgroup of
// four waves, with v_mfma_f32_16x16x32_bf16.  K goes through in stages of
// 512 values:
//   - every weight row of the stage is one 1 KB wave-wide load (lane l: 16
//     bytes at k + 8l), so the weight stream reads whole contiguous kilobytes
//     of each row, as the VALU panels do; the matrix-core operand layout
//     (16 rows x 64 bytes per wave-wide load) measured ~30% slower to stream;
//   - the batch operand of the stage (16 * NG rows of 512 values, bf16;
//     x .* norm_w with the sums of x^2 taken on the way where NORM) is
//     loaded once per workgroup, not once per wave and tile;
//   - both go to LDS, rows 1040 bytes apart (so that the 16 rows an operand
//     read touches start 4 banks apart), and each wave takes every fourth
//     32-value step of the stage, reading its A and B fragments from LDS;
//   - the loads of the next kMfmaPrefetch stages are in flight (in
//     registers) while a stage is computed.
// The waves' partial tiles are summed in wave order through LDS by the
// caller, after run() (MfmaLds::red aliases the stage buffers).
#pragma once

#include "dab_device.h"

namespace dab {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ inline bf16x8 as_bf16x8(const u32x4& v) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = __builtin_bit_cast(__bf16, (uint16_t)(v[i] & 0xffffu));
        r[2 * i + 1] = __builtin_bit_cast(__bf16, (uint16_t)(v[i] >> 16));
    }
    return r;
}

// ---------------------------------------------------------------------------
// direct loads into LDS (global_load_lds_dwordx4) and their waits
// ---------------------------------------------------------------------------
//
// Issued from inline asm: the compiler's builtin for them makes it wait for
// every load in flight (vmcnt(0)) before any LDS read it cannot prove
// disjoint.  The kernels that use them count their own loads: wait_vm<N>
// leaves the N most recent in flight.

template <int N>
__device__ inline void wait_vm() {
    // s_waitcnt vmcnt(N), expcnt and lgkmcnt left alone
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) for an n the compiler folds to a constant (an unrolled loop's count).
__device__ inline void wait_vm_n(int n) {
    switch (n) {
#define DAB_WAIT_CASE(N) case N: wait_vm<N>(); break;
        DAB_WAIT_CASE(0) DAB_WAIT_CASE(1) DAB_WAIT_CASE(2) DAB_WAIT_CASE(3) DAB_WAIT_CASE(4) DAB_WAIT_CASE(5)
        DAB_WAIT_CASE(6) DAB_WAIT_CASE(7) DAB_WAIT_CASE(8) DAB_WAIT_CASE(9) DAB_WAIT_CASE(10) DAB_WAIT_CASE(11)
        DAB_WAIT_CASE(12) DAB_WAIT_CASE(13) DAB_WAIT_CASE(14) DAB_WAIT_CASE(15) DAB_WAIT_CASE(16)
        DAB_WAIT_CASE(17) DAB_WAIT_CASE(18) DAB_WAIT_CASE(19) DAB_WAIT_CASE(20) DAB_WAIT_CASE(21)
        DAB_WAIT_CASE(22) DAB_WAIT_CASE(23) DAB_WAIT_CASE(24)
#undef DAB_WAIT_CASE
        default: wait_vm<0>(); break;
    }
}

__device__ inline void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0): this wave's LDS reads done
    asm volatile("s_barrier" ::: "memory");
}

// 16 bytes per lane from src into LDS at byte lds + 16 * lane (lds wave-uniform).  M0 holds the LDS
// address; no other instruction of the kernels here uses M0 (no dynamic register indexing, no message
// or GDS instructions), so setting it in the asm is safe.  The load has no register result.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_load16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Four 16-bit values of a transposing LDS read (ds_read_b64_tr_b16): in each
// 16-lane group, lane i receives element i % 4 of the 8 bytes addressed by
// lanes 4j + i / 4 of its group, j = 0..3.
__device__ inline v4i16 read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)((__attribute__((address_space(3))) char*)(p)));
}

constexpr int kMfmaThreads = 256;                   // four waves
// K values per stage: kMfmaSub 1 KB loads per weight row (1024 measured no faster for the 8B layer at
// batch 16 on MI355X, and slower for its FFN)
constexpr int kMfmaStageK = 512;
constexpr int kMfmaSub = kMfmaStageK / 512;
// stages whose loads are in flight ahead of the one computed (3 and 4 measured slower: 8B layer, batch 16,
// QKV 22.5 -> 23.3 -> 24.3 us; its FFN 88 -> 93 -> 122 us)
constexpr int kMfmaPrefetch = 2;
constexpr int kMfmaRowLds = kMfmaStageK + 8;        // bf16 per LDS row (+16 bytes: rows start 4 banks apart)

template <int TILES, int NG>
struct MfmaStage {
    uint16_t w[16 * TILES][kMfmaRowLds];   // the stage's weight rows
    uint16_t x[16 * NG][kMfmaRowLds];      // the stage's batch operand
};

template <int TILES, int NG>
struct MfmaReduce {
    float c[4][TILES][NG][16][17];         // per-wave partial tiles [wave][tile][group][row][sequence]
    float ss[16 * NG];                     // NORM: sums of x^2 per sequence
};

template <int TILES, int NG>
union MfmaLds {
    MfmaStage<TILES, NG> st;
    MfmaReduce<TILES, NG> red;
};

template <int TILES, int NG, bool NORM>
struct MfmaCore {
    static constexpr int ROWS = 16 * TILES;
    static constexpr int RPW = ROWS / 4;     // weight rows each wave loads per stage: wave + 4r
    static constexpr int XPT = 4 * NG;       // batch rows each thread loads per stage: wave + 4i
    static constexpr int WL = RPW * kMfmaSub, XL = XPT * kMfmaSub;   // 16-byte loads per thread and stage
    f32x4 acc[TILES][NG];
    float ssq[XPT];                          // NORM: sums of x^2 of this thread's batch rows (its k values)

    // rows[r]: weight row wave + 4r of the panel; xrows[i]: batch row wave + 4i
    // (nullptr past the batch: zeros); nw: norm_w in LDS (NORM).  Returns with
    // the stage buffers free (after a barrier).
    __device__ void run(const uint16_t* const (&rows)[RPW], const uint16_t* const (&xrows)[XPT],
                        const uint16_t* nw, int K, MfmaStage<TILES, NG>& st) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[tl][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < XPT; ++i) ssq[i] = 0.f;
        const int nst = (K + kMfmaStageK - 1) / kMfmaStageK;

        auto issue_w = [&](u32x4 (&wr)[WL], int s) {
#pragma unroll
            for (int j = 0; j < kMfmaSub; ++j) {
                const int k = s * kMfmaStageK + 512 * j + 8 * lane;
#pragma unroll
                for (int r = 0; r < RPW; ++r)
                    wr[j * RPW + r] = k < K ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows[r] + k))
                                            : u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto issue_x = [&](u32x4 (&xr)[XL], int s) {
#pragma unroll
            for (int j = 0; j < kMfmaSub; ++j) {
                const int k = s * kMfmaStageK + 512 * j + 8 * lane;
#pragma unroll
                for (int i = 0; i < XPT; ++i)
                    xr[j * XPT + i] = k < K && xrows[i] ? *reinterpret_cast<const u32x4*>(xrows[i] + k)
                                                        : u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto store_w = [&](const u32x4 (&wr)[WL]) {
#pragma unroll
            for (int j = 0; j < kMfmaSub; ++j)
#pragma unroll
                for (int r = 0; r < RPW; ++r)
                    *reinterpret_cast<u32x4*>(&st.w[wave + 4 * r][512 * j + 8 * lane]) = wr[j * RPW + r];
        };
        auto store_x = [&](const u32x4 (&xr)[XL], int s) {
#pragma unroll
            for (int j = 0; j < kMfmaSub; ++j) {
                const int kl = 512 * j + 8 * lane, k = s * kMfmaStageK + kl;
#pragma unroll
                for (int i = 0; i < XPT; ++i) {
                    u32x4 v = xr[j * XPT + i];
                    if constexpr (NORM) {
                        if (k < K) {
                            const u32x4 w8 = *reinterpret_cast<const u32x4*>(nw + k);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float x0 = __uint_as_float(v[e] << 16), x1 = __uint_as_float(v[e] & 0xffff0000u);
                                ssq[i] = fmaf(x0, x0, ssq[i]);
                                ssq[i] = fmaf(x1, x1, ssq[i]);
                                v[e] = pack_bf16x2(x0 * __uint_as_float(w8[e] << 16),
                                                   x1 * __uint_as_float(w8[e] & 0xffff0000u));
                            }
                        }
                    }
                    *reinterpret_cast<u32x4*>(&st.x[wave + 4 * i][kl]) = v;
                }
            }
        };
        auto compute = [&]() {
            const int m = lane & 15, kg = lane >> 4;
#pragma unroll
            for (int q = 0; q < kMfmaStageK / 32 / 4; ++q) {
                const int kk = 32 * (wave + 4 * q) + 8 * kg;      // step wave + 4q of the stage
                bf16x8 bfr[NG];
#pragma unroll
                for (int g = 0; g < NG; ++g) bfr[g] = as_bf16x8(*reinterpret_cast<const u32x4*>(&st.x[16 * g + m][kk]));
#pragma unroll
                for (int tl = 0; tl < TILES; ++tl) {
                    const bf16x8 afr = as_bf16x8(*reinterpret_cast<const u32x4*>(&st.w[16 * tl + m][kk]));
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        acc[tl][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[g], acc[tl][g], 0, 0, 0);
                }
            }
        };

        // a ring of kMfmaPrefetch register sets: stages s + 1 .. s + kMfmaPrefetch in flight while
        // stage s is computed (the ring is unrolled, so every set stays in registers)
        u32x4 wr[kMfmaPrefetch][WL], xr[kMfmaPrefetch][XL];
#pragma unroll
        for (int p = 0; p < kMfmaPrefetch; ++p)
            if (p < nst) {
                issue_w(wr[p], p);
                issue_x(xr[p], p);
            }
        for (int s0 = 0; s0 < nst; s0 += kMfmaPrefetch) {
#pragma unroll
            for (int p = 0; p < kMfmaPrefetch; ++p) {
                if (s0 + p < nst) {
                    __syncthreads();                   // the previous stage is computed: LDS free
                    store_w(wr[p]);
                    store_x(xr[p], s0 + p);
                    if (s0 + p + kMfmaPrefetch < nst) {
                        issue_w(wr[p], s0 + p + kMfmaPrefetch);
                        issue_x(xr[p], s0 + p + kMfmaPrefetch);
                    }
                    __syncthreads();
                    compute();
                }
            }
        }
        __syncthreads();
    }

    // Partial tiles (and, NORM, the sums of x^2 per sequence) to `red`; a
    // barrier follows, then every wave's partials are readable.
    __device__ void publish_partials(MfmaReduce<TILES, NG>& red) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int n = lane & 15, kg = lane >> 4;
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j) red.c[wave][tl][g][4 * kg + j][n] = acc[tl][g][j];
        if constexpr (NORM) {
#pragma unroll
            for (int i = 0; i < XPT; ++i) {
                const float s = wave_sum(ssq[i]);
                if (lane == 0) red.ss[wave + 4 * i] = s;
            }
        }
        __syncthreads();
    }
};

// Sum over the four waves, in wave order, of output (tile, row r, sequence
// 16 g + n) of the panel.
template <int TILES, int NG>
__device__ inline float mfma_sum(const MfmaReduce<TILES, NG>& red, int tile, int g, int r, int n) {
    return red.c[0][tile][g][r][n] + red.c[1][tile][g][r][n] + red.c[2][tile][g][r][n] + red.c[3][tile][g][r][n];
}


// ---------------------------------------------------------------------------
// The resident-operand panel: 16 sequences, K <= kMfmaResMaxK
// ---------------------------------------------------------------------------
//
// Where the batch operand of 16 sequences fits in LDS whole (16 x K bf16,
// 131 KB at K = 4096), a workgroup of eight waves stages it once, then each
// wave streams its eighth of K of the panel's weight rows straight into the
// matrix-core operand layout (lane i: row i % 16 of a tile, 16 bytes at
// 8 (i / 16) of each 32-value step), kMfmaResSteps steps requested at once,
// with the batch fragments read from LDS: no barrier in the stream and no
// batch-operand loads from memory after the start.  (8B layer, batch 16, on
// MI355X: QKV projection 18.7 us, output projection 10.4 us; with the batch
// operand staged stage by stage as in MfmaCore 22.5 and 13.2; with all 16
// steps of a wave requested at once 20.4 and 10.9.)
// The waves' partial tiles are summed in wave order through LDS.

constexpr int kMfmaResWaves = 8;
constexpr int kMfmaResThreads = 64 * kMfmaResWaves;
constexpr int kMfmaResSteps = 8;                   // steps of 32 per wave requested at once
constexpr int kMfmaResMaxK = 4096;

template <int TILES>
struct MfmaResLds {
    union {
        uint16_t x[16][kMfmaResMaxK + 8];                  // the batch operand (rows 4 banks apart)
        float c[kMfmaResWaves][TILES][16][17];             // per-wave partial tiles, after the stream
    };
    float ss[16];                                          // NORM: sums of x^2 per sequence
};

template <int TILES, bool NORM>
struct MfmaResident {
    f32x4 acc[TILES];

    // rows[tile]: this lane's weight row of each tile (tile row lane % 16); xrow(n): batch row n (nullptr
    // past the batch); nw: norm_w in LDS (NORM).  K a multiple of 32 * kMfmaResWaves, at most
    // kMfmaResMaxK.  Ends with the partial tiles in lds.c and the sums of squares in lds.ss, after a
    // barrier.
    template <class XROW>
    __device__ void run(const uint16_t* const (&rows)[TILES], XROW xrow, const uint16_t* nw, int K,
                        MfmaResLds<TILES>& lds) {
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        // 1. the batch operand into LDS: thread t takes sequence t / 32, 16-byte chunks t % 32 + 32 i
        {
            const int n = t >> 5, c0 = t & 31;
            const uint16_t* xr = xrow(n);
            float ssq = 0.f;
            for (int c = c0; c * 8 < K; c += 32 * 8) {
                u32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = (c + 32 * u) * 8;
                    v[u] = xr && k < K ? *reinterpret_cast<const u32x4*>(xr + k) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = (c + 32 * u) * 8;
                    if (k < K) {
                        if constexpr (NORM) {
                            const u32x4 w8 = *reinterpret_cast<const u32x4*>(nw + k);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float x0 = __uint_as_float(v[u][e] << 16), x1 = __uint_as_float(v[u][e] & 0xffff0000u);
                                ssq = fmaf(x0, x0, ssq);
                                ssq = fmaf(x1, x1, ssq);
                                v[u][e] = pack_bf16x2(x0 * __uint_as_float(w8[e] << 16),
                                                      x1 * __uint_as_float(w8[e] & 0xffff0000u));
                            }
                        }
                        *reinterpret_cast<u32x4*>(&lds.x[n][k]) = v[u];
                    }
                }
            }
            if constexpr (NORM) {
#pragma unroll
                for (int off = 16; off > 0; off >>= 1) ssq += __shfl_xor(ssq, off);
                if ((t & 31) == 0) lds.ss[n] = ssq;
            }
        }
        // 2. this wave's steps in groups of kMfmaResSteps, the weight fragments straight from memory,
        // the batch fragments from LDS
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int m = lane & 15, kg = lane >> 4;
        const int nsteps = K / (32 * kMfmaResWaves), k_begin = wave * nsteps * 32;
        u32x4 w[TILES][kMfmaResSteps];
        auto issue = [&](int s0) {
#pragma unroll
            for (int s = 0; s < kMfmaResSteps; ++s) {
                const int k = k_begin + (s0 + s) * 32 + 8 * kg;
#pragma unroll
                for (int tl = 0; tl < TILES; ++tl)
                    w[tl][s] = s0 + s < nsteps ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows[tl] + k))
                                               : u32x4{0u, 0u, 0u, 0u};
            }
        };
        issue(0);
        __syncthreads();                                   // the batch operand is in LDS
        for (int s0 = 0; s0 < nsteps; s0 += kMfmaResSteps) {
#pragma unroll
            for (int s = 0; s < kMfmaResSteps; ++s) {
                if (s0 + s < nsteps) {
                    const bf16x8 bfr =
                        as_bf16x8(*reinterpret_cast<const u32x4*>(&lds.x[m][k_begin + (s0 + s) * 32 + 8 * kg]));
#pragma unroll
                    for (int tl = 0; tl < TILES; ++tl)
                        acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[tl][s]), bfr, acc[tl], 0, 0, 0);
                }
            }
            if (s0 + kMfmaResSteps < nsteps) issue(s0 + kMfmaResSteps);
        }
        // 4. partial tiles to LDS (over the batch operand, which no wave reads any more)
        __syncthreads();
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
            for (int j = 0; j < 4; ++j) lds.c[wave][tl][4 * kg + j][m] = acc[tl][j];
        __syncthreads();
    }
};

template <int TILES>
__device__ inline float mfma_res_sum(const MfmaResLds<TILES>& lds, int tile, int r, int n) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kMfmaResWaves; ++w) s += lds.c[w][tile][r][n];
    return s;
}

// ---------------------------------------------------------------------------
// The streamed panel: 16 or 32 sequences, K a multiple of 1024, at most 4096
// ---------------------------------------------------------------------------
//
// Eight waves; wave w owns K values [w K/8, (w + 1) K/8) of every row of the
// panel.  Its batch fragments for those K values (sequence 16 g + i % 16,
// 8 values at 8 (i / 16) of each 32-value step), and with the RMSNorm its
// norm_w fragments, are loaded once into registers, so no LDS holds the
// batch operand and no barrier stages it.  The weight rows go through LDS by
// direct loads (global_load_lds_dwordx4): a window is 128 K values (256
// bytes) of a tile's 16 rows, four loads of 4 rows x 256 bytes, each row's
// 16-byte pieces XOR-swizzled by the row (piece c of row r at c ^ r) so that
// the operand reads (16 rows, one piece each) hit distinct banks.  Each wave
// keeps mfma_str_ring windows in flight in a ring of its own, waits for the
// oldest with s_waitcnt vmcnt, reads its operands, runs its four steps and
// requests the next window into the freed slot: no barrier in the stream.
// The direct loads use the compiler's builtin, so its own waits for the
// batch fragments (requested first) count them and wait for nothing else;
// the ring is read from inline asm (the four reads and their wait in one
// block), so the compiler sees no LDS read that could alias a load in flight
// and adds no wait for every load before it.
// The waves' partial tiles are summed in wave order through LDS.

constexpr int kMfmaStrWaves = 8;
constexpr int kMfmaStrThreads = 64 * kMfmaStrWaves;
constexpr int kMfmaStrWin = 128;                   // K values of a window
// Windows in flight per wave: two (8B layer, batch 16, on MI355X: QKV projection 14.3, 14.9, 15.2 and
// 15.4 us with one, two, three and four; output projection 9.4, 9.0, 9.7 and 10.1 us; a read probe of the
// same pattern without the matrix work: 10.5 us with two, 13.6 with four).  The batch and norm_w
// fragments are requested before the stream's first loads (after them measured no faster).
template <int NG> constexpr int mfma_str_ring() { return 2; }
// K = 1024 NWIN: at most 4096 with two tiles or the RMSNorm (a window's batch fragments serve every
// tile, so they stay in registers for the panel; norm_w is one direct load per wave), 16384 with one
// tile (each window's fragments are dead after its four steps)
constexpr int kMfmaStrMaxK = 4096;
constexpr int kMfmaStrMaxK1 = 16384;

template <int TILES, int NG>
struct MfmaStrLds {
    union {
        u32x4 ring[kMfmaStrWaves][mfma_str_ring<NG>()][256];   // per wave: windows of 16 rows x 256 bytes
        float c[kMfmaStrWaves][TILES][NG][16][17];         // partial tiles, after the stream
    };
    float ss[kMfmaStrWaves][16 * NG];                      // NORM: per-wave sums of x^2
    u32x4 nw[kMfmaStrWaves][64];                           // NORM: each wave's norm_w values
};

// Four 16-byte LDS reads (byte addresses) and their wait, in one block.
__device__ inline void lds_read4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, u32x4& r0, u32x4& r1, u32x4& r2,
                                 u32x4& r3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

// HALF2: the second tile is half used (its rows 0-3 and 8-11; 24-row panels): its other rows are never
// loaded, and what the MFMA makes of them (whatever the slot held) is never read.
template <int TILES, int NG, bool NORM, int NWIN, bool HALF2 = false>
struct MfmaStream {
    static_assert(NWIN >= 1 && NWIN * kMfmaStrWin * kMfmaStrWaves <= (TILES == 1 && !NORM ? kMfmaStrMaxK1 : kMfmaStrMaxK),
                  "K = 1024 NWIN");
    static_assert(!HALF2 || TILES == 2, "a half-used second tile");
    static constexpr int RING = mfma_str_ring<NG>();
    f32x4 acc[TILES][NG];

    // rowp(tile, r): weight row r of a tile; xrow(n): batch row n of the workgroup (nullptr past the
    // batch: zeros); norm_w: the RMSNorm weights (NORM).  K = 1024 NWIN (every loop and wait static).
    // Ends with the partial tiles in lds.c and the per-wave sums of x^2 in lds.ss, after a barrier.
    // trace: profiling builds only, this workgroup's timestamp slots (stage ends at 4 and 5), or null.
    template <class ROWP, class XROW>
    __device__ void run(ROWP rowp, XROW xrow, const uint16_t* norm_w, int K, MfmaStrLds<TILES, NG>& lds,
                        unsigned long long* trace = nullptr) {
        const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
        const int m = lane & 15, kg = lane >> 4;
        (void)K;
        constexpr int ks = NWIN * kMfmaStrWin, nsteps = ks / 32, nwin = NWIN, nw_all = TILES * NWIN;
        const int k0 = wave * ks;                                 // this wave's K values
        // 1. this wave's batch fragments (raw) and norm_w fragments, four steps at a time, each group
        // requested just before the weight window that first uses them (all of them at the start, the
        // panel's first window waited ~4 us for them: every workgroup reads the same batch rows); rows
        // past the batch read a valid address and are zeroed after
        const uint16_t* w00 = rowp(0, 0);
        u32x4 xf[NG][nsteps];
        bool xlive[NG];
        // NORM: the wave's norm_w values reach its LDS by one direct load with the first window (lane i:
        // values 8 (i mod ks/8) ..) and are read from there (a load per step and lane read the same 16
        // bytes 16 times over, and the loads a CU issues are what bound this panel)
        const uint16_t* xb[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint16_t* xr = xrow(16 * g + m);
            xlive[g] = xr != nullptr;
            xb[g] = xr ? xr + k0 + 8 * kg : w00;
        }
        // the batch (and norm_w) fragments of window w of the first tile: its four steps
        auto load_aux = [&](int w) {
#pragma unroll
            for (int s = 4 * w; s < 4 * w + 4; ++s) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    xf[g][s] = *reinterpret_cast<const u32x4*>(xb[g] + (xlive[g] ? 32 * s : 0));
            }
        };
        // loads requested per window: its batch fragments (first tile only) and its four weight loads
        auto count = [&](int w) { return (w < nwin ? 4 * NG : 0) + (HALF2 && w >= nwin ? 2 : 4); };
        // 2. the first windows of weight rows in flight: window j is tile j / nwin, K values
        // k0 + 128 (j % nwin) ..; load q of a window takes rows 4q .. 4q + 3, lane i row 4q + i / 16 and
        // piece (i % 16) ^ row, so that the piece lands at (i % 16) = piece ^ row
        const uint16_t* src[TILES][4];
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 4 * q + (lane >> 4);
                src[tl][q] = rowp(tl, r) + k0 + 8 * ((lane & 15) ^ r);
            }
        // The wait counts below assume the loads go out in program order: the batch fragments of a
        // window, then its four weight loads; scheduling barriers keep the compiler from moving loads
        // across a window's weight loads.
        auto issue = [&](int j) {
            const int tj = j / nwin, kw = j - tj * nwin;
            u32x4* dst = &lds.ring[wave][j % RING][0];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (HALF2 && tj == 1 && (q & 1)) continue;   // rows 4-7 and 12-15 of a half-used tile
                const uint16_t* sp = src[0][q];
#pragma unroll
                for (int tl = 1; tl < TILES; ++tl)
                    if (tj == tl) sp = src[tl][q];
                __builtin_amdgcn_global_load_lds(sp + kMfmaStrWin * kw,
                                                 (__attribute__((address_space(3))) void*)(
                                                     (__attribute__((address_space(3))) char*)(dst + 64 * q)),
                                                 16, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int j = 0; j < RING; ++j)
            if (j < nw_all) {
                if (j < nwin) load_aux(j);
                if (NORM && j == 0)
                    __builtin_amdgcn_global_load_lds(norm_w + k0 + 8 * (lane % (ks / 8)),
                                                     (__attribute__((address_space(3))) void*)(
                                                         (__attribute__((address_space(3))) char*)(&lds.nw[wave][0])),
                                                     16, 0, 0);
                issue(j);
            }
        const uint32_t nw0 = lds_address(&lds.nw[wave][0]);
        // nothing below moves above the stream's first loads
        __builtin_amdgcn_sched_barrier(0);
        float ssq[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) ssq[g] = 0.f;
#ifdef DAB_TRACE
        if (trace && t == 0) trace[4] = __builtin_amdgcn_s_memrealtime();
#endif
        // 4. the windows: wait for the oldest, read its operands, four steps, request the next into its slot
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[tl][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint32_t ring0 = lds_address(&lds.ring[wave][0][0]);
        uint32_t rd[4];                                          // this lane's operand pieces in a slot
#pragma unroll
        for (int s = 0; s < 4; ++s) rd[s] = 16u * (uint32_t)((m >> 2) * 64 + (m & 3) * 16 + (((4 * s + kg) ^ m) & 15));
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl) {
#pragma unroll
            for (int kw = 0; kw < NWIN; ++kw) {
                {
                    const int j = tl * nwin + kw;
                    // this window's loads (and every older one) are in: the windows requested after it
                    // may still be in flight
                    int later = 0;
#pragma unroll
                    for (int w = j + 1; w < j + RING; ++w)
                        if (w < nw_all) later += count(w);
                    wait_vm_n(later);
                    __builtin_amdgcn_sched_barrier(0);  // nothing that uses this window moves above the wait
                    const uint32_t slot = ring0 + (uint32_t)(j % RING) * 4096u;
                    u32x4 w[4];
                    lds_read4(slot + rd[0], slot + rd[1], slot + rd[2], slot + rd[3], w[0], w[1], w[2], w[3]);
                    // first tile: the window's batch steps are zeroed past the batch and, NORM, become
                    // x .* norm_w rounded to bf16 with the sums of x^2 taken on the way (here, after the
                    // wait above, so that the compiler's own wait for these fragments does not wait for
                    // the whole stream)
                    if (tl == 0) {
#pragma unroll
                        for (int s = 4 * kw; s < 4 * kw + 4; ++s)
#pragma unroll
                            for (int g = 0; g < NG; ++g)
                                if (!xlive[g]) xf[g][s] = u32x4{0u, 0u, 0u, 0u};
                    }
                    if constexpr (NORM) {
                        if (tl == 0) {
                            u32x4 nfw[4];                     // norm_w of the window's steps (piece 4 s + kg)
                            lds_read4(nw0 + 16u * (16 * kw + kg), nw0 + 16u * (16 * kw + 4 + kg),
                                      nw0 + 16u * (16 * kw + 8 + kg), nw0 + 16u * (16 * kw + 12 + kg), nfw[0], nfw[1],
                                      nfw[2], nfw[3]);
#pragma unroll
                            for (int s = 4 * kw; s < 4 * kw + 4; ++s) {
                                const u32x4 nf = nfw[s - 4 * kw];
#pragma unroll
                                for (int g = 0; g < NG; ++g)
#pragma unroll
                                    for (int e = 0; e < 4; ++e) {
                                        const float x0 = __uint_as_float(xf[g][s][e] << 16);
                                        const float x1 = __uint_as_float(xf[g][s][e] & 0xffff0000u);
                                        ssq[g] = fmaf(x0, x0, ssq[g]);
                                        ssq[g] = fmaf(x1, x1, ssq[g]);
                                        xf[g][s][e] = pack_bf16x2(x0 * __uint_as_float(nf[e] << 16),
                                                                  x1 * __uint_as_float(nf[e] & 0xffff0000u));
                                    }
                            }
                        }
                    }
                    if (j + RING < nw_all) {            // into the slot just read (its reads are done)
                        if (j + RING < nwin) load_aux(j + RING);
                        issue(j + RING);
                    }
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int g = 0; g < NG; ++g)
                            acc[tl][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[s]), as_bf16x8(xf[g][4 * kw + s]),
                                                                                  acc[tl][g], 0, 0, 0);
                }
            }
        }
        // 5. partial tiles and sums of x^2 to LDS (over the ring, which no wave reads any more)
#ifdef DAB_TRACE
        if (trace && t == 0) trace[5] = __builtin_amdgcn_s_memrealtime();
#endif
        __syncthreads();
#pragma unroll
        for (int tl = 0; tl < TILES; ++tl)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j) lds.c[wave][tl][g][4 * kg + j][m] = acc[tl][g][j];
        if constexpr (NORM) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                float v = ssq[g];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (lane < 16) lds.ss[wave][16 * g + lane] = v;
            }
        }
        __syncthreads();
    }
};

template <int TILES, int NG>
__device__ inline float mfma_str_sum(const MfmaStrLds<TILES, NG>& lds, int tile, int g, int r, int n) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kMfmaStrWaves; ++w) s += lds.c[w][tile][g][r][n];
    return s;
}

template <int TILES, int NG>
__device__ inline float mfma_str_ssq(const MfmaStrLds<TILES, NG>& lds, int sq) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kMfmaStrWaves; ++w) s += lds.ss[w][sq];
    return s;
}

}  // namespace dev
}  // namespace dab
