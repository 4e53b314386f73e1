// Row-panel GEMVs of the decode step (gfx950, wave64).
//
// W is stored [N, K]: one output feature per row, its K weights contiguous
// (the torch.nn.Linear layout).  A workgroup owns 4 waves x RW rows and all
// of K for NB batch rows.  Lane l of a wave reads the 16-byte vectors l,
// l + 64, l + 128, ... of each of its rows, so one wave-wide load covers
// 1 KB of a row and a row of 4096 bf16 weights is 8 loads per lane.  Every
// weight load of the first K-block is issued before anything else; the
// fp32 inputs are staged in LDS meanwhile, and each output is one wave
// reduction.  No partial sum leaves the workgroup: the kernel ends when its
// last weight bytes arrive, with no second pass over partials.
//
//   QKV panel   wave w of panel i takes RoPE pair 4i + w: rows e and e + D/2
//               of one head (q heads, then k heads, then v heads), so both
//               halves of a rotation meet in one wave.  RMSNorm is applied
//               as a scale after the sum, u = r * ((x .* norm_w) . W[n]),
//               r = (mean x^2 + eps)^(-1/2) (the operator-fusion page,
//               section 3, stage 1; the one-shot all-reduce page, section
//               2.2), so the weight stream never waits for the norm.  Then
//               RoPE (rotate-half pairing, angle pos * theta^(-2e/D), formed
//               and reduced to [-pi, pi] in fp64), q and the new k, v to the
//               workspace, k and v appended to the caches (operator-fusion
//               page, section 3, stages 2-3).
//   O panel     rows of W_o; out = x + a . W_o[n] (ClusterFusion page,
//               section 1.1; operator-fusion page, section 1).
#pragma once

#include "dab_device.h"
#include "dab_mfma.h"

namespace dab {
namespace dev {

// 16 bytes of weights: 8 bf16 or 4 fp32, streamed once (nontemporal).
template <typename T> struct W16;

template <> struct W16<uint16_t> {
    static constexpr int N = 8;
    u32x4 r;
    __device__ void load(const uint16_t* p) { r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
    __device__ void load_cached(const uint16_t* p) { r = *reinterpret_cast<const u32x4*>(p); }
    __device__ void fetch(const uint16_t* p) {          // published by another workgroup of the launch
        uint32_t w[4];
        fetch16(p, w);
        r = u32x4{w[0], w[1], w[2], w[3]};
    }
    __device__ void zero() { r = u32x4{0u, 0u, 0u, 0u}; }
    __device__ void unpack(float* f) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(r[i] << 16);
            f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
};

template <> struct W16<float> {
    static constexpr int N = 4;
    f32x4 r;
    __device__ void load(const float* p) { r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)); }
    __device__ void load_cached(const float* p) { r = *reinterpret_cast<const f32x4*>(p); }
    __device__ void fetch(const float* p) {
        uint32_t w[4];
        fetch16(p, w);
        r = f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
    }
    __device__ void zero() { r = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void unpack(float* f) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = r[i];
    }
};

constexpr int kPanelVecs = 8;    // weight vectors per lane, row and K-block

// Work index -> (panel, batch group); false for padding.  The batch groups
// of one panel get work indices 8 apart, so they run on one XCD (blocks are
// dealt to the eight XCDs round-robin) and read the panel through its L2.
__device__ inline bool panel_decode(int nbg, int panels, int idx, int* panel, int* bgi) {
    if (nbg == 1) {
        *panel = idx;
        *bgi = 0;
        return idx < panels;
    }
    const int lo = idx & 7, rest = idx >> 3;
    *bgi = rest % nbg;
    *panel = (rest / nbg) * 8 + lo;
    return *panel < panels;
}

// RW rows of W against NB fp32 input rows staged in LDS (xs, row stride K).
// EXACT: K is a whole number of K-blocks, so every lane's every vector is in
// range and the loads go out with no bounds checks (and no branches, which
// would make the compiler wait for every load at the first use).
template <typename T, int RW, int NB, bool EXACT>
struct PanelDot {
    static constexpr int N = W16<T>::N;
    static constexpr int KB = 64 * kPanelVecs * N;   // K per block: 4096 bf16, 2048 fp32
    W16<T> w[RW][kPanelVecs];
    float acc[RW][NB];

    __device__ void issue(const T* const (&rows)[RW], int k0, int K, int lane) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int v = 0; v < kPanelVecs; ++v) {
                const int k = k0 + (v * 64 + lane) * N;
                if (EXACT || k < K) w[r][v].load(rows[r] + k);
                else w[r][v].zero();
            }
    }

    __device__ void accumulate(const float* xs, int k0, int K, int lane) {
#pragma unroll
        for (int v = 0; v < kPanelVecs; ++v) {
            const int k = k0 + (v * 64 + lane) * N;
            if (EXACT || k < K) {
                float wf[RW][N];
#pragma unroll
                for (int r = 0; r < RW; ++r) w[r][v].unpack(wf[r]);
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
    }

    // The whole dot product: block 0 must already be issued.  Every lane
    // ends with every sum.
    __device__ void run(const T* const (&rows)[RW], const float* xs, int K, int lane) {
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[r][j] = 0.f;
        for (int k0 = 0; k0 < K; k0 += KB) {
            if (k0 > 0) issue(rows, k0, K, lane);
            accumulate(xs, k0, K, lane);
        }
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[r][j] = wave_sum(acc[r][j]);
    }
};

// Staging of NB input rows of K values into LDS as fp32.  The first SI
// vectors of every thread are loaded into registers before the weight
// stream is issued (one round trip to L2 in front of the weights instead of
// one behind them: a wave's loads complete in issue order); the rest, for
// large K only, are loaded afterwards.
constexpr int kStageAhead = 2;

template <typename T, int NB>
struct QkvShared {
    float ss[NB][4];
};

// How a QKV panel hands its results on.
enum QkvMode {
    kQkvPlain = 0,     // a kernel of its own: plain stores, and it re-arms the ready counts of the
                       // attention + projection launch that follows
    kQkvSignalGroup,   // attention in the same launch: device-coherent stores, then the panel count of its
                       // (batch group, head) goes up
    kQkvSignalSeq,     // the whole step in one launch: device-coherent stores, then the panel count of
                       // (sequence, head) goes up for each of its valid sequences; no re-arming here
};

// Lane work of a QKV panel for sequence bb: RMS scale, RoPE, q and the new
// k, v out, the cache append.  ss: the four waves' sums of x^2.
template <typename T, int MODE>
__device__ void qkv_finish(const StepArgs& a, int panel, int wave, int bb, int hd, int e, int row0, float u0,
                           float u1, const float* ss) {
    constexpr bool SIGNAL = MODE != kQkvPlain;
    const int H = a.H, D = a.D, half = D >> 1;
    // re-arm the ready counts of this sequence for the attention kernel that
    // follows (it runs after this kernel completes)
    if (MODE != kQkvSignalSeq && panel == 0 && wave == 0)
        for (int i = 0; i < kReadyCopies; ++i) set_counter(&a.seq_ready[(bb * kReadyCopies + i) * kReadyStride], 0);
    const float sum_sq = ss[0] + ss[1] + ss[2] + ss[3];
    const float r = 1.0f / sqrtf(sum_sq / (float)H + a.eps);
    u0 *= r;
    u1 *= r;
    int p;
    const bool ok = pos_valid(a, bb, &p);
    if (!ok && panel == 0 && wave == 0) __hip_atomic_fetch_or(a.flags, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (hd < a.nq + a.nkv) {
        // q and k rows rotate: angle pos * theta^(-2e/D) in fp64, reduced to
        // [-pi, pi] (fp32 would lose ~1e-3 rad at pos 16K), sin/cos in fp32
        const double ang = (double)p * exp2(-(2.0 * e / D) * a.log2_theta);
        const double two_pi = 6.283185307179586;
        float sn, cs;
        sincosf((float)(ang - two_pi * rint(ang / two_pi)), &sn, &cs);
        const float v0 = u0 * cs - u1 * sn;
        const float v1 = u1 * cs + u0 * sn;
        u0 = v0;
        u1 = v1;
    }
    auto out = [&](float* dst, float v) {
        if constexpr (SIGNAL) publish(dst, v);
        else *dst = v;
    };
    if (hd < a.nq) {
        float* q = a.q + (size_t)bb * a.n_q + row0;
        out(q, u0);
        out(q + half, u1);
    } else {
        const int kvrow = row0 - a.n_q;                  // in [0, 2 nkv D)
        const int is_v = kvrow >= a.nkv * D;
        const int col = is_v ? kvrow - a.nkv * D : kvrow;
        float* kn = a.kv_new + ((size_t)bb * 2 + is_v) * a.nkv * D + col;
        out(kn, u0);
        out(kn + half, u1);
        if (ok) {
            T* dst = static_cast<T*>(is_v ? a.v_cache : a.k_cache) + ((size_t)bb * a.cap + p) * a.nkv * D + col;
            dst[0] = from_f32<T>(u0);
            dst[half] = from_f32<T>(u1);
        }
    }
}

// QKV panel `panel` for batch rows [bgi * NB, +NB).  xs: NB x H floats of LDS.
// MODE (QkvMode) kQkvSignal*: attention runs in the same launch; q and the
// new k, v are stored device-coherently and, once the whole panel's stores
// are acknowledged, the panel counts of its head go up.
template <typename T, int NB, bool EXACT, int MODE>
__device__ void qkv_panel(const StepArgs& a, int panel, int bgi, float* xs, QkvShared<T, NB>& sm) {
    constexpr int N = W16<T>::N;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int H = a.H, D = a.D, half = D >> 1;
    const int pr = panel * 4 + wave;                 // this wave's RoPE pair
    const int hd = pr / half, e = pr - hd * half;    // head (q, then k, then v heads), dim
    const int row0 = hd * D + e;
    const T* W = static_cast<const T*>(a.w_qkv);
    const T* const rows[2] = {W + (size_t)row0 * H, W + (size_t)(row0 + half) * H};
    const T* hid = static_cast<const T*>(a.hidden);
    const T* nw = static_cast<const T*>(a.norm_w);
    const int b0 = bgi * NB;

    // 1. this thread's first input vectors, then the weight stream
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

    // 2. x .* norm_w into LDS, and sum of x^2 per sequence
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
    float u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
        if (lane == j) {
            u0 = dot.acc[0][j];
            u1 = dot.acc[1][j];
        }
    const int bb = b0 + lane;
    if (lane < NB && bb < a.B) qkv_finish<T, MODE>(a, panel, wave, bb, hd, e, row0, u0, u1, sm.ss[lane]);
    if constexpr (MODE == kQkvSignalGroup) {
        drain_and_sync();
        if (t == 0) bump(&a.head_cnt[bgi * (a.nq + 2 * a.nkv) + hd]);
    } else if constexpr (MODE == kQkvSignalSeq) {
        // one count per valid sequence (a sequence with a bad position has no
        // attention, so nothing would re-arm its counts)
        drain_and_sync();
        int p;
        if (t < NB && b0 + t < a.B && pos_valid(a, b0 + t, &p))
            add_counter(&a.head_cnt[(b0 + t) * (a.nq + 2 * a.nkv) + hd]);
    }
}

// O panel `panel` (RW rows per wave) for batch rows [bgi * NB, +NB).
// xs: NB x n_q floats of LDS.  WAIT: the attention output is produced in the
// same launch; the weight stream goes out first, then the workgroup waits
// until every kv group of its sequences is merged and reads the attention
// output device-coherently.  REARM (with WAIT; the whole step in one
// launch): past its wait, the panel counts itself as a reader of its copy of
// each sequence's ready count; the last reader of a copy re-arms it, and
// panel 0 re-arms the sequences' QKV panel counts (every attention chunk of
// those sequences, the only readers, has finished: the merges they fed are
// done).
//
// PUBLISH (the overlapped layer, RW = 2): h goes out with device-coherent
// stores (a lane's two rows are adjacent, one 4- or 8-byte store), then every
// sequence of the group counts the panel at its sub-counter; the panel that
// completes a sub-counter re-arms it and adds one to each of the sequence's
// ready counts, which the FFN panels of the same launch poll.
template <typename T, int RW, int NB, bool EXACT, bool WAIT, bool REARM = false, bool PUBLISH = false>
__device__ void oproj_panel(const StepArgs& a, int panel, int bgi, float* xs) {
    static_assert(!PUBLISH || RW == 2, "published rows go out in pairs");
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int K = a.n_q, H = a.H;
    const int row0 = (panel * 4 + wave) * RW;
    const T* W = static_cast<const T*>(a.w_o);
    const T* rows[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) rows[r] = W + (size_t)(row0 + r) * K;
    const int b0 = bgi * NB;
    // sequences of this group with an attention output (valid position)
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        int p;
        if (b0 + j < a.B && pos_valid(a, b0 + j, &p)) valid |= 1u << j;
    }
    // lane j's residual inputs, requested first so they are in by the end
    const bool mine = lane < NB && ((valid >> lane) & 1u);
    float xres[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r)
        xres[r] = mine ? to_f32(static_cast<const T*>(a.hidden)[(size_t)(b0 + lane) * H + row0 + r]) : 0.f;

    PanelDot<T, RW, NB, EXACT> dot;
    const int copy = WAIT ? panel % a.ready_copies : 0;   // this panel's copy of the ready counts
    int readers_before[NB];                               // REARM: readers of the copy before this one
#pragma unroll
    for (int j = 0; j < NB; ++j) readers_before[j] = -1;
    if constexpr (WAIT) {
        // 1. the weight stream, then the wait for the attention output
        dot.issue(rows, 0, K, lane);
        DAB_TRACE_POINT(a, 1);
        if (t == 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if ((valid >> j) & 1u)
                    wait_at_least<8>(&a.seq_ready[((b0 + j) * kReadyCopies + copy) * kReadyStride], a.nkv, a.flags);
            if constexpr (REARM) {
                // the replies return while the attention output is read below
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    readers_before[j] = ((valid >> j) & 1u)
                        ? bump(&a.ready_done[((b0 + j) * kReadyCopies + copy) * kReadyStride]) : -1;
            }
        }
        __syncthreads();
        if constexpr (REARM) {
            if (panel == 0) {
                const int nheads = a.nq + 2 * a.nkv;
                for (int j = 0; j < NB; ++j)
                    if ((valid >> j) & 1u)
                        for (int i = t; i < nheads; i += 256) set_counter(&a.head_cnt[(b0 + j) * nheads + i], 0);
            }
        }
        // 2. attention outputs into LDS (zeros for sequences without one):
        // every load of a round issued before any is used, so the round
        // costs one trip to the memory-side cache
        constexpr int PR = 8;                         // 8-byte loads per thread and round
        for (int k0 = 0; k0 < K; k0 += 2 * 256 * PR) {
            float v[NB][PR][2];
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < PR; ++i) {
                    const int k = k0 + 2 * (i * 256 + t);
                    if (k < K && ((valid >> j) & 1u)) {
                        fetch2(a.a + (size_t)(b0 + j) * K + k, v[j][i]);
                    } else {
                        v[j][i][0] = 0.f;
                        v[j][i][1] = 0.f;
                    }
                }
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int i = 0; i < PR; ++i) {
                    const int k = k0 + 2 * (i * 256 + t);
                    if (k < K) {
                        xs[(size_t)j * K + k] = v[j][i][0];
                        xs[(size_t)j * K + k + 1] = v[j][i][1];
                    }
                }
        }
    } else {
        // 1. this thread's first attention-output vectors, then the weight stream
        constexpr int SA = 2 * kStageAhead;           // fp32 vectors: 4 floats each
        f32x4 xr[SA][NB];
#pragma unroll
        for (int i = 0; i < SA; ++i) {
            const int k = (i * 256 + t) * 4;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                xr[i][j] = (k < K && ((valid >> j) & 1u))
                               ? *reinterpret_cast<const f32x4*>(a.a + (size_t)(b0 + j) * K + k)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        dot.issue(rows, 0, K, lane);
        DAB_TRACE_POINT(a, 1);

        // 2. attention outputs into LDS (zeros for sequences without one)
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
                    ((valid >> j) & 1u) ? *reinterpret_cast<const f32x4*>(a.a + (size_t)(b0 + j) * K + k)
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __syncthreads();
    DAB_TRACE_POINT(a, 2);
    if constexpr (WAIT && REARM) {
        if (t == 0) {
            // readers of this copy: the panels p with p % ready_copies == copy
            const int readers = (a.oproj.panels - copy + a.ready_copies - 1) / a.ready_copies;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (readers_before[j] == readers - 1) {
                    set_counter(&a.seq_ready[((b0 + j) * kReadyCopies + copy) * kReadyStride], 0);
                    set_counter(&a.ready_done[((b0 + j) * kReadyCopies + copy) * kReadyStride], 0);
                }
        }
    }

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
    if constexpr (PUBLISH) {
        if (mine) {
            const size_t i = (size_t)(b0 + lane) * H + row0;
            publish_pair(static_cast<T*>(a.out) + i, from_f32<T>(xres[0] + y[0]), from_f32<T>(xres[1] + y[1]));
            if (a.dbg_y) {
                a.dbg_y[i] = y[0];
                a.dbg_y[i + 1] = y[1];
            }
        }
        drain_and_sync();
        DAB_TRACE_POINT(a, 4);
        if (wave == 0) {
            bool done = false;
            if (lane < NB && b0 + lane < a.B) {
                const int b = b0 + lane, sub = panel % kHSub;
                const int per_sub = (a.oproj.panels - sub + kHSub - 1) / kHSub;
                if (bump(&a.hand[h_sub_at(b, sub)]) == per_sub - 1) {
                    set_counter(&a.hand[h_sub_at(b, sub)], 0);
                    done = true;
                }
            }
            uint64_t last = __ballot(done);
            while (last) {
                const int b = b0 + __builtin_ctzll(last);
                last &= last - 1;
                static_assert(kHCopies == 64, "one ready count per lane");
                add_counter(&a.hand[h_flag_at(b, lane)]);
            }
        }
        return;
    }
    if (!mine) return;
    const int bb = b0 + lane;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const size_t i = (size_t)bb * H + row0 + r;
        static_cast<T*>(a.out)[i] = from_f32<T>(xres[r] + y[r]);
        if (a.dbg_y) a.dbg_y[i] = y[r];
    }
}

// ---------------------------------------------------------------------------
// MFMA panels (bf16, batch >= 8)
// ---------------------------------------------------------------------------
//
// The matrix-core row panel of dab_mfma.h for the QKV projection (each tile
// 8 RoPE pairs of one head: rows e and e + D/2 at tile rows r and r + 8, so
// that each rotation stays in a tile; the batch operand x .* norm_w, RMSNorm
// applied as a scale after the sum, then the lane work of the VALU panel) and
// for the output projection (the batch operand the bf16 copy of the attention
// output; the residual added after the sum).

// The rows of a panel: tile row (tile, m) -> a row of W (QKV: 8 RoPE pairs of
// one head per tile, rows e and e + D/2 at tile rows r and r + 8).
struct MfmaRows {
    int hd = 0, e0 = 0;
    __device__ MfmaRows(const StepArgs& a, bool qkv, int panel, int tiles) {
        if (qkv) {
            const int pr0 = panel * 8 * tiles;             // first RoPE pair of the panel
            hd = pr0 / (a.D >> 1);
            e0 = pr0 - hd * (a.D >> 1);
        }
    }
    __device__ int qkv_row(const StepArgs& a, int tile, int m) const {
        return hd * a.D + e0 + tile * 8 + (m & 7) + (m >= 8 ? a.D >> 1 : 0);
    }
};

// The lane work after the sums: sum(tile, g, r, n) is output row r of the
// tile for sequence 16 g + n of the workgroup, ssq(sq) the sum of x^2 of
// sequence sq (QKV).
template <bool QKV, int TILES, int NG, int THREADS, class SUM, class SSQ>
__device__ void mfma_finish(const StepArgs& a, int panel, int bgi, const MfmaRows& mr, SUM sum, SSQ ssq) {
    constexpr int ROWS = 16 * TILES, NS = 16 * NG;
    const int t = threadIdx.x, D = a.D;
    if constexpr (QKV) {
        // thread (tile, pair r, sequence) finishes pair (r, r + 8) of one sequence
        for (int idx = t; idx < TILES * 8 * NS; idx += THREADS) {
            const int tile = idx / (8 * NS), r = (idx / NS) % 8, sq = idx % NS, g = sq >> 4, n = sq & 15;
            const int bb = bgi * NS + sq;
            if (bb >= a.B) continue;
            const float ss[4] = {ssq(sq), 0.f, 0.f, 0.f};
            const int e = mr.e0 + tile * 8 + r;
            qkv_finish<uint16_t, kQkvPlain>(a, panel, tile * 8 + r, bb, mr.hd, e, mr.hd * D + e, sum(tile, g, r, n),
                                            sum(tile, g, r + 8, n), ss);
        }
    } else {
        for (int idx = t; idx < ROWS * NS; idx += THREADS) {
            const int row = idx / NS, sq = idx % NS, g = sq >> 4, n = sq & 15;
            const int bb = bgi * NS + sq;
            int pp;
            if (bb >= a.B || !pos_valid(a, bb, &pp)) continue;
            const float y = sum(row >> 4, g, row & 15, n);
            const size_t i = (size_t)bb * a.H + panel * ROWS + row;
            static_cast<uint16_t*>(a.out)[i] = from_f32<uint16_t>(to_f32(static_cast<const uint16_t*>(a.hidden)[i]) + y);
            if (a.dbg_y) a.dbg_y[i] = y;
        }
    }
}

// The batch row of sequence b for a panel (QKV: the hidden row; output
// projection: the bf16 attention output, for sequences with a valid position).
template <bool QKV>
__device__ inline const uint16_t* mfma_xrow(const StepArgs& a, int b) {
    int p;
    const bool live = b < a.B && (QKV || pos_valid(a, b, &p));
    const int K = QKV ? a.H : a.n_q;
    return live ? (QKV ? static_cast<const uint16_t*>(a.hidden) : a.a16) + (size_t)b * K : nullptr;
}

// Staged panel (dab_mfma.h MfmaCore): 256 threads, any K, 16 or 32 sequences.
// nw_lds: QKV only, H bf16 values of norm_w (staged by the caller).
template <bool QKV, int TILES, int NG>
__device__ void mfma_panel(const StepArgs& a, int panel, int bgi, MfmaLds<TILES, NG>& lds, const uint16_t* nw_lds) {
    using Core = MfmaCore<TILES, NG, QKV>;
    constexpr int ROWS = 16 * TILES, NS = 16 * NG;
    const int wave = threadIdx.x >> 6;
    const int K = QKV ? a.H : a.n_q;
    const uint16_t* W = static_cast<const uint16_t*>(QKV ? a.w_qkv : a.w_o);
    const MfmaRows mr(a, QKV, panel, TILES);
    const uint16_t* rows[Core::RPW];
#pragma unroll
    for (int r = 0; r < Core::RPW; ++r) {
        const int pr = wave + 4 * r;
        rows[r] = W + (size_t)(QKV ? mr.qkv_row(a, pr >> 4, pr & 15) : panel * ROWS + pr) * K;
    }
    const uint16_t* xrows[Core::XPT];
#pragma unroll
    for (int i = 0; i < Core::XPT; ++i) xrows[i] = mfma_xrow<QKV>(a, bgi * NS + wave + 4 * i);
    Core core;
    DAB_TRACE_POINT(a, 1);
    core.run(rows, xrows, nw_lds, K, lds.st);
    core.publish_partials(lds.red);
    DAB_TRACE_POINT(a, 2);
    const MfmaReduce<TILES, NG>& red = lds.red;
    mfma_finish<QKV, TILES, NG, kMfmaThreads>(
        a, panel, bgi, mr, [&](int tl, int g, int r, int n) { return mfma_sum(red, tl, g, r, n); },
        [&](int sq) { return red.ss[sq]; });
}

// Resident-operand panel (dab_mfma.h MfmaResident): 512 threads, 16
// sequences, K a multiple of 256 and at most kMfmaResMaxK.
template <bool QKV, int TILES>
__device__ void mfma_res_panel(const StepArgs& a, int panel, int bgi, MfmaResLds<TILES>& lds, const uint16_t* nw_lds) {
    const int m = threadIdx.x & 15;
    const int K = QKV ? a.H : a.n_q;
    const uint16_t* W = static_cast<const uint16_t*>(QKV ? a.w_qkv : a.w_o);
    const MfmaRows mr(a, QKV, panel, TILES);
    const uint16_t* rows[TILES];
#pragma unroll
    for (int tl = 0; tl < TILES; ++tl)
        rows[tl] = W + (size_t)(QKV ? mr.qkv_row(a, tl, m) : panel * 16 * TILES + tl * 16 + m) * K;
    MfmaResident<TILES, QKV> core;
    DAB_TRACE_POINT(a, 1);
    core.run(rows, [&](int n) { return mfma_xrow<QKV>(a, bgi * 16 + n); }, nw_lds, K, lds);
    DAB_TRACE_POINT(a, 2);
    mfma_finish<QKV, TILES, 1, kMfmaResThreads>(
        a, panel, bgi, mr, [&](int tl, int, int r, int n) { return mfma_res_sum(lds, tl, r, n); },
        [&](int sq) { return lds.ss[sq]; });
}

// Streamed panel (dab_mfma.h MfmaStream): 512 threads, 16 or 32 sequences,
// K = 1024 NWIN.
template <bool QKV, int TILES, int NG, int NWIN>
__device__ void mfma_str_panel(const StepArgs& a, int panel, int bgi, MfmaStrLds<TILES, NG>& lds) {
    constexpr int NS = 16 * NG;
    const int K = QKV ? a.H : a.n_q;
    const uint16_t* W = static_cast<const uint16_t*>(QKV ? a.w_qkv : a.w_o);
    const MfmaRows mr(a, QKV, panel, TILES);
    MfmaStream<TILES, NG, QKV, NWIN> core;
    DAB_TRACE_POINT(a, 1);
    core.run([&](int tl, int r) { return W + (size_t)(QKV ? mr.qkv_row(a, tl, r) : panel * 16 * TILES + tl * 16 + r) * K; },
             [&](int n) { return mfma_xrow<QKV>(a, bgi * NS + n); }, static_cast<const uint16_t*>(a.norm_w), K, lds,
#ifdef DAB_TRACE
             a.trace ? a.trace + (size_t)(a.trace_base + blockIdx.x) * 8 : nullptr
#else
             nullptr
#endif
    );
    DAB_TRACE_POINT(a, 2);
    mfma_finish<QKV, TILES, NG, kMfmaStrThreads>(
        a, panel, bgi, mr, [&](int tl, int g, int r, int n) { return mfma_str_sum(lds, tl, g, r, n); },
        [&](int sq) { return mfma_str_ssq(lds, sq); });
}

// QKV projection in 24-row panels on the streamed panel: three half tiles
// of 4 RoPE pairs each (rows e .. e+3 and e+D/2 .. e+D/2+3 of one head),
// half tiles A and B in tile 0 (A at tile rows 0-3 and 8-11, B at 4-7 and
// 12-15), C in tile 1 (rows 0-3 and 8-11; the rest unused), so that pair
// (r, r + 8) of a tile stays one rotation.  A panel's half tiles may belong
// to different heads.  (The 6144 rows of the 8B GQA layer make 256 such
// panels, one per CU, against 192 of 32 rows.)
struct QkvHalfTiles {
    int hd[3], e0[3];
    __device__ QkvHalfTiles(const StepArgs& a, int panel) {
        const int per_head = a.D >> 3;                    // half tiles per head
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int ht = panel * 3 + i;
            hd[i] = ht / per_head;
            e0[i] = (ht - hd[i] * per_head) * 4;
        }
    }
    // half tile of tile row m of tile tl (the unused rows of tile 1 map to C's)
    __device__ int which(int tl, int m) const { return tl == 0 ? (m >> 2) & 1 : 2; }
    __device__ int row(const StepArgs& a, int tl, int m) const {
        const int i = which(tl, m);
        return hd[i] * a.D + e0[i] + (m & 3) + (m >= 8 ? a.D >> 1 : 0);
    }
};

template <int NG, int NWIN>
__device__ void mfma_str_qkv24(const StepArgs& a, int panel, int bgi, MfmaStrLds<2, NG>& lds) {
    constexpr int NS = 16 * NG;
    const int t = threadIdx.x, K = a.H, D = a.D;
    const uint16_t* W = static_cast<const uint16_t*>(a.w_qkv);
    const QkvHalfTiles ht(a, panel);
    MfmaStream<2, NG, true, NWIN, true> core;
    DAB_TRACE_POINT(a, 1);
    core.run([&](int tl, int r) { return W + (size_t)ht.row(a, tl, r) * K; },
             [&](int n) { return mfma_xrow<true>(a, bgi * NS + n); }, static_cast<const uint16_t*>(a.norm_w), K, lds,
#ifdef DAB_TRACE
             a.trace ? a.trace + (size_t)(a.trace_base + blockIdx.x) * 8 : nullptr
#else
             nullptr
#endif
    );
    DAB_TRACE_POINT(a, 2);
    // thread (pair slot, sequence): slots 0-7 are tile 0's pairs (A, then B), 8-11 tile 1's (C)
    for (int idx = t; idx < 12 * NS; idx += kMfmaStrThreads) {
        const int ps = idx / NS, sq = idx % NS, g = sq >> 4, n = sq & 15;
        const int bb = bgi * NS + sq;
        if (bb >= a.B) continue;
        const int tl = ps >> 3, r = ps & 7, i = ht.which(tl, r);
        const float ss[4] = {mfma_str_ssq(lds, sq), 0.f, 0.f, 0.f};
        const int e = ht.e0[i] + (r & 3);
        qkv_finish<uint16_t, kQkvPlain>(a, panel, ps, bb, ht.hd[i], e, ht.hd[i] * D + e, mfma_str_sum(lds, tl, g, r, n),
                                        mfma_str_sum(lds, tl, g, r + 8, n), ss);
    }
}

}  // namespace dev
}  // namespace dab
