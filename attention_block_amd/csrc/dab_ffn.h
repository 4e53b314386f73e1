// The FFN half of the decoder layer (gfx950, wave64): two row-panel GEMVs.
//
//   gate/up panel  wave w of panel i takes row n = 4i + w of W_gate and of
//                  W_up (a PanelDot pair of rows, like a RoPE pair of the
//                  QKV panel), against x .* norm_w staged in LDS; RMSNorm is
//                  applied as a scale after the sums, r = (mean x^2 + eps)^-1/2,
//                  then m[n] = silu(r g) * (r u) goes to the workspace.
//   down panel     two rows of W_down per wave against m staged in LDS;
//                  out = h + m . W_down[n], rounded to the storage type.
//                  (Two rows: with m in fp32 a workgroup takes 4 bytes of
//                  LDS per intermediate feature, 44 KB at F = 11008, so
//                  three fit on a CU, and 512 workgroups of 8 rows all hold
//                  a slot from the start where 1024 of 4 rows needed a
//                  second, partial round: 19.5 against 21.8 us for the 7B
//                  layer's 90 MB.)
//
// The operator-fusion page, section 1, places a second RMS norm and the FFN
// after the attention block's residual; the gated SiLU form is the one of
// the LLaMA architecture that page takes as its example.
#pragma once

#include "dab_gemv.h"

namespace dab {
namespace dev {

template <int NB>
struct FfnShared {
    float ss[NB][4];
};

// Gate/up panel `panel` for batch rows [bgi * NB, +NB).  xs: NB x H floats of LDS.
// WAIT (the overlapped layer): h is written by the output projection's
// panels of the same launch; the panel streams its weights, waits for its
// sequences' ready counts, then reads h with device-coherent loads.  Each thread takes
// the same elements in the same order either way, so the results are
// bit-identical.
template <typename T, int NB, bool EXACT, bool WAIT = false>
__device__ void ffn_gate_up_panel(const FfnArgs& a, int panel, int bgi, float* xs, FfnShared<NB>& sm) {
    constexpr int N = W16<T>::N;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int H = a.H;
    const int n = panel * 4 + wave;
    const T* const rows[2] = {static_cast<const T*>(a.w_gate) + (size_t)n * H,
                              static_cast<const T*>(a.w_up) + (size_t)n * H};
    const T* hid = static_cast<const T*>(a.hidden);
    const T* nw = static_cast<const T*>(a.norm_w);
    const int b0 = bgi * NB;

    // 1. this thread's first input vectors, then the weight stream (a
    // wave's loads complete in issue order)
    W16<T> xr[kStageAhead][NB], wr[kStageAhead];
    if constexpr (!WAIT) {
#pragma unroll
        for (int i = 0; i < kStageAhead; ++i) {
            const int k = (i * 256 + t) * N;
            if (k < H) {
                wr[i].load_cached(nw + k);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (b0 + j < a.B) xr[i][j].load_cached(hid + (size_t)(b0 + j) * H + k);
                    else xr[i][j].zero();
                }
            }
        }
    }
    PanelDot<T, 2, NB, EXACT> dot;
    dot.issue(rows, 0, H, lane);
    DAB_TRACE_POINT(a, 1);
    if constexpr (WAIT) {
        if (t < NB && b0 + t < a.B)
            wait_at_least<8>(&a.hand[h_flag_at(b0 + t, panel % kHCopies)], h_subs(a.h_panels), a.flags);
        __syncthreads();
        DAB_TRACE_POINT(a, 4);
    }

    // 2. h .* norm_w into LDS, and the sum of h^2 per sequence
    float ss[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) ss[j] = 0.f;
    auto stage = [&](int k, const W16<T>& wv, const W16<T> (&xv)[NB]) {
        float wn[N];
        wv.unpack(wn);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float x[N];
            xv[j].unpack(x);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                ss[j] = fmaf(x[i], x[i], ss[j]);
                x[i] *= wn[i];
            }
#pragma unroll
            for (int i = 0; i < N / 4; ++i)
                *reinterpret_cast<f32x4*>(xs + (size_t)j * H + k + 4 * i) =
                    f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
        }
    };
    if constexpr (WAIT) {
        // rounds of kHRound vectors per thread, every load of a round issued
        // before any is used (h from the coherence point, norm_w as usual)
        constexpr int kHRound = 4;
        for (int k0 = 0; k0 < H; k0 += kHRound * 256 * N) {
            W16<T> hv[kHRound][NB], nv[kHRound];
#pragma unroll
            for (int i = 0; i < kHRound; ++i) {
                const int k = k0 + (i * 256 + t) * N;
                if (k < H) {
                    nv[i].load_cached(nw + k);
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        if (b0 + j < a.B) hv[i][j].fetch(hid + (size_t)(b0 + j) * H + k);
                        else hv[i][j].zero();
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < kHRound; ++i) {
                const int k = k0 + (i * 256 + t) * N;
                if (k < H) stage(k, nv[i], hv[i]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kStageAhead; ++i) {
            const int k = (i * 256 + t) * N;
            if (k < H) stage(k, wr[i], xr[i]);
        }
        for (int k = (kStageAhead * 256 + t) * N; k < H; k += 256 * N) {
            W16<T> wv, xv[NB];
            wv.load_cached(nw + k);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (b0 + j < a.B) xv[j].load_cached(hid + (size_t)(b0 + j) * H + k);
                else xv[j].zero();
            }
            stage(k, wv, xv);
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const float s = wave_sum(ss[j]);
        if (lane == 0) sm.ss[j][wave] = s;
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 2);

    // 3. both rows against every staged sequence
    dot.run(rows, xs, H, lane);

    // 4. lane j finishes sequence b0 + j
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (lane == j) {
            g = dot.acc[0][j];
            u = dot.acc[1][j];
        }
    const int bb = b0 + lane;
    if (lane < NB && bb < a.B) {
        const float* s = sm.ss[lane];
        const float r = 1.0f / sqrtf((s[0] + s[1] + s[2] + s[3]) / (float)H + a.eps);
        g *= r;
        u *= r;
        a.m[(size_t)bb * a.F + n] = g / (1.0f + expf(-g)) * u;
    }
}

// The down panel's dot product for bf16 rows of NBLK K-blocks (F above 4096,
// up to 16384): block b + 1 is requested before block b is used, so each
// wave keeps a block in flight while it computes, where PanelDot waits out a
// round trip per block (7B layer, F 11008: down panel 19.4 -> 17.4 us).  Every load is unconditional (addresses past K are
// clamped into the row), so the compiler counts the loads in flight and
// waits only for the block it is about to use; the elements past K are
// skipped at use, in the last block.  The sums are PanelDot's, in its order.
template <int RW, int NB, int NBLK>
struct DownDot2 {
    using T = uint16_t;
    static constexpr int N = W16<T>::N;
    static constexpr int KB = 64 * kPanelVecs * N;
    W16<T> w[2][RW][kPanelVecs];
    float acc[RW][NB];

    template <int BUF>
    __device__ void issue(const T* const (&rows)[RW], int k0, int K, int lane) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int v = 0; v < kPanelVecs; ++v) {
                const int k = k0 + (v * 64 + lane) * N;
                w[BUF][r][v].load(rows[r] + (k < K ? k : K - N));
            }
    }

    template <int BUF, bool LAST>
    __device__ void accumulate(const float* xs, int k0, int K, int lane) {
#pragma unroll
        for (int v = 0; v < kPanelVecs; ++v) {
            const int k = k0 + (v * 64 + lane) * N;
            if (LAST && k >= K) continue;
            float wf[RW][N];
#pragma unroll
            for (int r = 0; r < RW; ++r) w[BUF][r][v].unpack(wf[r]);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float xv[N];
#pragma unroll
                for (int i = 0; i < N / 4; ++i) {
                    const f32x4 x4 = *reinterpret_cast<const f32x4*>(xs + (size_t)j * K + k + 4 * i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) xv[4 * i + e] = x4[e];
                }
#pragma unroll
                for (int r = 0; r < RW; ++r)
#pragma unroll
                    for (int e = 0; e < N; ++e) acc[r][j] = fmaf(wf[r][e], xv[e], acc[r][j]);
            }
        }
    }

    template <int B>
    __device__ void step(const T* const (&rows)[RW], const float* xs, int K, int lane) {
        if constexpr (B + 1 < NBLK) issue<(B + 1) & 1>(rows, (B + 1) * KB, K, lane);
        // the next block's requests all go out before this block's
        // arithmetic (left to itself the compiler reuses each register as
        // its value is consumed: 7B down panel 17.8 against 17.4 us)
        __builtin_amdgcn_sched_barrier(0);
        accumulate<B & 1, B + 1 == NBLK>(xs, B * KB, K, lane);
    }

    // Block 0 must already be issued (issue<0>(rows, 0, K, lane)).  Every
    // lane ends with every sum.
    __device__ void run(const T* const (&rows)[RW], const float* xs, int K, int lane) {
        static_assert(NBLK >= 2 && NBLK <= 4, "two to four K-blocks");
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[r][j] = 0.f;
        step<0>(rows, xs, K, lane);
        step<1>(rows, xs, K, lane);
        if constexpr (NBLK > 2) step<2>(rows, xs, K, lane);
        if constexpr (NBLK > 3) step<3>(rows, xs, K, lane);
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[r][j] = wave_sum(acc[r][j]);
    }
};

// The down panel's dot product: DownDot2 for bf16 rows of NBLK = 2..4
// blocks, PanelDot otherwise (NBLK = 0).
template <typename T, int RW, int NB, bool EXACT, int NBLK, bool DB = (NBLK >= 2)>
struct DownDot {
    PanelDot<T, RW, NB, EXACT> d;
    __device__ void issue0(const T* const (&rows)[RW], int K, int lane) { d.issue(rows, 0, K, lane); }
    __device__ void run(const T* const (&rows)[RW], const float* xs, int K, int lane) { d.run(rows, xs, K, lane); }
    __device__ float sum(int r, int j) const { return d.acc[r][j]; }
};
template <typename T, int RW, int NB, bool EXACT, int NBLK>
struct DownDot<T, RW, NB, EXACT, NBLK, true> {
    static_assert(sizeof(T) == 2, "the double-buffered down panel is built for bf16");
    DownDot2<RW, NB, NBLK> d;
    __device__ void issue0(const T* const (&rows)[RW], int K, int lane) { d.template issue<0>(rows, 0, K, lane); }
    __device__ void run(const T* const (&rows)[RW], const float* xs, int K, int lane) { d.run(rows, xs, K, lane); }
    __device__ float sum(int r, int j) const { return d.acc[r][j]; }
};

// Down panel `panel` (RW rows per wave) for batch rows [bgi * NB, +NB).
// xs: NB x F floats of LDS.  NBLK: see DownDot.
template <typename T, int RW, int NB, bool EXACT, int NBLK = 0>
__device__ void ffn_down_panel(const FfnArgs& a, int panel, int bgi, float* xs) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int K = a.F, H = a.H;
    const int row0 = (panel * 4 + wave) * RW;
    const T* rows[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) rows[r] = static_cast<const T*>(a.w_down) + (size_t)(row0 + r) * K;
    const int b0 = bgi * NB;
    // lane j's residual inputs, requested first so they are in by the end
    const bool mine = lane < NB && b0 + lane < a.B;
    float xres[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r)
        xres[r] = mine ? to_f32(static_cast<const T*>(a.hidden)[(size_t)(b0 + lane) * H + row0 + r]) : 0.f;

    // 1. this thread's first m vectors, then the weight stream
    constexpr int SA = 2 * kStageAhead;               // fp32 vectors: 4 floats each
    f32x4 xr[SA][NB];
#pragma unroll
    for (int i = 0; i < SA; ++i) {
        const int k = (i * 256 + t) * 4;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            xr[i][j] = k < K && b0 + j < a.B ? *reinterpret_cast<const f32x4*>(a.m + (size_t)(b0 + j) * K + k)
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    DownDot<T, RW, NB, EXACT, NBLK> dot;
    dot.issue0(rows, K, lane);
    DAB_TRACE_POINT(a, 1);

    // 2. m into LDS (zeros for padding rows of the batch group)
#pragma unroll
    for (int i = 0; i < SA; ++i) {
        const int k = (i * 256 + t) * 4;
        if (k < K) {
#pragma unroll
            for (int j = 0; j < NB; ++j) *reinterpret_cast<f32x4*>(xs + (size_t)j * K + k) = xr[i][j];
        }
    }
    for (int k = (SA * 256 + t) * 4; k < K; k += 1024) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
            *reinterpret_cast<f32x4*>(xs + (size_t)j * K + k) =
                b0 + j < a.B ? *reinterpret_cast<const f32x4*>(a.m + (size_t)(b0 + j) * K + k)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 2);

    // 3. the rows against every staged sequence
    dot.run(rows, xs, K, lane);

    // 4. lane j finishes sequence b0 + j: residual, rounding to storage
    float y[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) y[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (lane == j) {
#pragma unroll
            for (int r = 0; r < RW; ++r) y[r] = dot.sum(r, j);
        }
    if (!mine) return;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const size_t i = (size_t)(b0 + lane) * H + row0 + r;
        static_cast<T*>(a.out)[i] = from_f32<T>(xres[r] + y[r]);
        if (a.dbg_y) a.dbg_y[i] = y[r];
    }
}

// MFMA panels (bf16, batch >= 8): the matrix-core row panel of dab_mfma.h
// for 16 or 32 sequences per workgroup.
//   GATE_UP  tile 0: rows 16p .. 16p+15 of W_gate, tile 1: the same rows of
//            W_up; the batch operand is h .* norm_w rounded to bf16 (norm_w
//            from LDS), with the sums of h^2 taken on the way; m = silu(r g)(r u)
//            goes to the workspace rounded to bf16.
//   down     TILES tiles of 16 rows of W_down against m (bf16); out = h + y.
template <bool GATE_UP, int TILES, int NG>
__device__ void ffn_mfma_panel(const FfnArgs& a, int panel, int bgi, MfmaLds<TILES, NG>& lds, const uint16_t* nw_lds) {
    using Core = MfmaCore<TILES, NG, GATE_UP>;
    constexpr int ROWS = GATE_UP ? 16 : 16 * TILES, NS = 16 * NG;
    const int t = threadIdx.x, wave = t >> 6;
    const int K = GATE_UP ? a.H : a.F;
    const uint16_t* rows[Core::RPW];
#pragma unroll
    for (int r = 0; r < Core::RPW; ++r) {
        const int pr = wave + 4 * r, tile = pr >> 4, m = pr & 15;
        if constexpr (GATE_UP)
            rows[r] = static_cast<const uint16_t*>(tile == 0 ? a.w_gate : a.w_up) + (size_t)(panel * 16 + m) * K;
        else
            rows[r] = static_cast<const uint16_t*>(a.w_down) + (size_t)(panel * ROWS + pr) * K;
    }
    const uint16_t* xrows[Core::XPT];
#pragma unroll
    for (int i = 0; i < Core::XPT; ++i) {
        const int b = bgi * NS + wave + 4 * i;
        xrows[i] = b < a.B ? (GATE_UP ? static_cast<const uint16_t*>(a.hidden) : a.m16) + (size_t)b * K : nullptr;
    }
    Core core;
    DAB_TRACE_POINT(a, 1);
    core.run(rows, xrows, nw_lds, K, lds.st);
    core.publish_partials(lds.red);
    DAB_TRACE_POINT(a, 2);
    const MfmaReduce<TILES, NG>& red = lds.red;
    if constexpr (GATE_UP) {
        for (int idx = t; idx < 16 * NS; idx += kMfmaThreads) {
            const int r = idx / NS, sq = idx % NS, g = sq >> 4, n = sq & 15;
            const int bb = bgi * NS + sq;
            if (bb >= a.B) continue;
            const float rs = 1.0f / sqrtf(red.ss[sq] / (float)a.H + a.eps);
            const float gt = mfma_sum(red, 0, g, r, n) * rs, up = mfma_sum(red, 1, g, r, n) * rs;
            a.m16[(size_t)bb * a.F + panel * 16 + r] = from_f32<uint16_t>(gt / (1.0f + expf(-gt)) * up);
        }
    } else {
        for (int idx = t; idx < ROWS * NS; idx += kMfmaThreads) {
            const int row = idx / NS, sq = idx % NS, g = sq >> 4, n = sq & 15;
            const int bb = bgi * NS + sq;
            if (bb >= a.B) continue;
            const float y = mfma_sum(red, row >> 4, g, row & 15, n);
            const size_t i = (size_t)bb * a.H + panel * ROWS + row;
            static_cast<uint16_t*>(a.out)[i] =
                from_f32<uint16_t>(to_f32(static_cast<const uint16_t*>(a.hidden)[i]) + y);
            if (a.dbg_y) a.dbg_y[i] = y;
        }
    }
}

// Gate/up on the streamed panel (dab_mfma.h MfmaStream, H = 1024 NWIN), T
// mixed tiles per panel: tile j holds features f0 + 8j .. f0 + 8j + 7, their
// W_gate rows at tile rows 0-7 and their W_up rows at 8-15, so that the gate
// and up sums of a feature are rows r and r + 8 of one tile (as a RoPE pair
// in the QKV panel); 16 or 32 sequences; the finish is the staged panel's.
template <int T, int NG, int NWIN>
__device__ void ffn_str_gate_up(const FfnArgs& a, int panel, int bgi, MfmaStrLds<T, NG>& lds) {
    constexpr int NS = 16 * NG;
    const int t = threadIdx.x, K = a.H, f0 = panel * 8 * T;
    MfmaStream<T, NG, true, NWIN> core;
    DAB_TRACE_POINT(a, 1);
    core.run([&](int tl, int r) {
                 return static_cast<const uint16_t*>(r < 8 ? a.w_gate : a.w_up) + (size_t)(f0 + 8 * tl + (r & 7)) * K;
             },
             [&](int n) {
                 const int b = bgi * NS + n;
                 return b < a.B ? static_cast<const uint16_t*>(a.hidden) + (size_t)b * K : nullptr;
             },
             static_cast<const uint16_t*>(a.norm_w), K, lds);
    DAB_TRACE_POINT(a, 2);
    for (int idx = t; idx < T * 8 * NS; idx += kMfmaStrThreads) {
        const int f = idx / NS, sq = idx % NS, g = sq >> 4, n = sq & 15, tl = f >> 3, r = f & 7;
        const int bb = bgi * NS + sq;
        if (bb >= a.B) continue;
        const float rs = 1.0f / sqrtf(mfma_str_ssq(lds, sq) / (float)a.H + a.eps);
        const float gt = mfma_str_sum(lds, tl, g, r, n) * rs, up = mfma_str_sum(lds, tl, g, r + 8, n) * rs;
        a.m16[(size_t)bb * a.F + f0 + f] = from_f32<uint16_t>(gt / (1.0f + expf(-gt)) * up);
    }
}

// Down projection on the streamed panel (one tile of 16 rows of W_down, K = F
// = 1024 NWIN, 16 or 32 sequences against m in bf16); out = h + y.
template <int NG, int NWIN>
__device__ void ffn_str_down(const FfnArgs& a, int panel, int bgi, MfmaStrLds<1, NG>& lds) {
    constexpr int NS = 16 * NG;
    const int t = threadIdx.x, K = a.F;
    MfmaStream<1, NG, false, NWIN> core;
    DAB_TRACE_POINT(a, 1);
    core.run([&](int, int r) { return static_cast<const uint16_t*>(a.w_down) + (size_t)(panel * 16 + r) * K; },
             [&](int n) {
                 const int b = bgi * NS + n;
                 return b < a.B ? a.m16 + (size_t)b * K : nullptr;
             },
             nullptr, K, lds);
    DAB_TRACE_POINT(a, 2);
    for (int idx = t; idx < 16 * NS; idx += kMfmaStrThreads) {
        const int row = idx / NS, sq = idx % NS, g = sq >> 4, n = sq & 15;
        const int bb = bgi * NS + sq;
        if (bb >= a.B) continue;
        const float y = mfma_str_sum(lds, 0, g, row, n);
        const size_t i = (size_t)bb * a.H + panel * 16 + row;
        static_cast<uint16_t*>(a.out)[i] = from_f32<uint16_t>(to_f32(static_cast<const uint16_t*>(a.hidden)[i]) + y);
        if (a.dbg_y) a.dbg_y[i] = y;
    }
}

}  // namespace dev
}  // namespace dab
