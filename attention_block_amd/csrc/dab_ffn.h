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
template <typename T, int NB, bool EXACT>
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
    PanelDot<T, 2, NB, EXACT> dot;
    dot.issue(rows, 0, H, lane);
    DAB_TRACE_POINT(a, 1);

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

// Down panel `panel` (RW rows per wave) for batch rows [bgi * NB, +NB).
// xs: NB x F floats of LDS.
template <typename T, int RW, int NB, bool EXACT>
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
    PanelDot<T, RW, NB, EXACT> dot;
    dot.issue(rows, 0, K, lane);
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
            for (int r = 0; r < RW; ++r) y[r] = dot.acc[r][j];
        }
    if (!mine) return;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const size_t i = (size_t)(b0 + lane) * H + row0 + r;
        static_cast<T*>(a.out)[i] = from_f32<T>(xres[r] + y[r]);
        if (a.dbg_y) a.dbg_y[i] = y[r];
    }
}

// MFMA panels (bf16, batch >= 8): 16 sequences per workgroup, kMfmaWaves
// waves splitting K, v_mfma_f32_16x16x32_bf16 tiles of 16 rows x 16
// sequences (the layout of the attention block's MFMA panels).
//   GATE_UP  tile 0: rows 16p .. 16p+15 of W_gate, tile 1: the same rows of
//            W_up; the B operand is h .* norm_w rounded to bf16 (norm_w from
//            LDS), with the sums of h^2 taken on the way; m = silu(r g)(r u)
//            goes to the workspace rounded to bf16.
//   down     TILES tiles of 16 rows of W_down against m (bf16); out = h + y.
template <bool GATE_UP, int TILES>
__device__ void ffn_mfma_panel(const FfnArgs& a, int panel, int bgi, MfmaShared& sm, const uint16_t* nw_lds) {
    constexpr int ROWS = 16 * TILES;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int K = GATE_UP ? a.H : a.F;
    const int m = lane & 15, kg = lane >> 4;
    const int row0 = GATE_UP ? panel * 16 + m : panel * ROWS + m;
    const uint16_t* W0 = static_cast<const uint16_t*>(GATE_UP ? a.w_gate : a.w_down) + (size_t)row0 * K + kg * 8;
    const uint16_t* W1 = GATE_UP ? static_cast<const uint16_t*>(a.w_up) + (size_t)row0 * K + kg * 8
                                 : W0 + (size_t)16 * K;
    // this lane's sequence (tile column m)
    const int b = bgi * 16 + m;
    const bool live = b < a.B;
    const uint16_t* X = (GATE_UP ? static_cast<const uint16_t*>(a.hidden) : a.m16) + (size_t)(live ? b : 0) * K + kg * 8;

    const int nsteps = K / (32 * kMfmaWaves), k_begin = wave * nsteps * 32;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    float ssq = 0.f;
    for (int s0 = 0; s0 < nsteps; s0 += kMfmaSteps) {
        u32x4 w0[kMfmaSteps], w1[kMfmaSteps], x[kMfmaSteps];
#pragma unroll
        for (int s = 0; s < kMfmaSteps; ++s) {
            const int k = k_begin + (s0 + s) * 32;
            const bool in = s0 + s < nsteps;
            w0[s] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W0 + k)) : u32x4{0u, 0u, 0u, 0u};
            if constexpr (GATE_UP || TILES == 2)
                w1[s] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W1 + k)) : u32x4{0u, 0u, 0u, 0u};
            x[s] = in && live ? *reinterpret_cast<const u32x4*>(X + k) : u32x4{0u, 0u, 0u, 0u};
        }
        if (s0 == 0) DAB_TRACE_POINT(a, 1);
#pragma unroll
        for (int s = 0; s < kMfmaSteps; ++s) {
            if (s0 + s >= nsteps) break;
            bf16x8 bv;
            if constexpr (GATE_UP) {
                const int k = k_begin + (s0 + s) * 32 + kg * 8;
                const u32x4 nw = *reinterpret_cast<const u32x4*>(nw_lds + k);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = __uint_as_float(x[s][i] << 16), x1 = __uint_as_float(x[s][i] & 0xffff0000u);
                    ssq = fmaf(x0, x0, ssq);
                    ssq = fmaf(x1, x1, ssq);
                    bv[2 * i] = (__bf16)(x0 * __uint_as_float(nw[i] << 16));
                    bv[2 * i + 1] = (__bf16)(x1 * __uint_as_float(nw[i] & 0xffff0000u));
                }
            } else {
                bv = as_bf16x8(x[s]);
            }
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w0[s]), bv, acc0, 0, 0, 0);
            if constexpr (GATE_UP || TILES == 2)
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w1[s]), bv, acc1, 0, 0, 0);
        }
    }

    // partial tiles (and sums of h^2) to LDS, summed in wave order
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sm.c[wave][0][4 * kg + j][m] = acc0[j];
        if constexpr (GATE_UP || TILES == 2) sm.c[wave][1][4 * kg + j][m] = acc1[j];
    }
    if constexpr (GATE_UP) {
        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        if (kg == 0) sm.ss[m][wave] = ssq;
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 2);
    if constexpr (GATE_UP) {
        if (t >= 256) return;                                      // 16 rows x 16 sequences
        const int r = t >> 4, n = t & 15;
        const int bb = bgi * 16 + n;
        if (bb >= a.B) return;
        float g = 0.f, u = 0.f, ss = 0.f;
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) {
            g += sm.c[w][0][r][n];
            u += sm.c[w][1][r][n];
            ss += sm.ss[n][w];
        }
        const float rs = 1.0f / sqrtf(ss / (float)a.H + a.eps);
        g *= rs;
        u *= rs;
        a.m16[(size_t)bb * a.F + panel * 16 + r] = from_f32<uint16_t>(g / (1.0f + expf(-g)) * u);
    } else {
        if (t >= 256 * TILES) return;                              // tiles x 16 rows x 16 sequences
        const int tile = t >> 8, r = (t >> 4) & 15, n = t & 15;
        const int bb = bgi * 16 + n;
        if (bb >= a.B) return;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) y += sm.c[w][tile][r][n];
        const size_t i = (size_t)bb * a.H + panel * ROWS + tile * 16 + r;
        static_cast<uint16_t*>(a.out)[i] = from_f32<uint16_t>(to_f32(static_cast<const uint16_t*>(a.hidden)[i]) + y);
        if (a.dbg_y) a.dbg_y[i] = y;
    }
}

}  // namespace dev
}  // namespace dab
