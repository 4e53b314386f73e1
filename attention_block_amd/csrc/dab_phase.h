// The kernels of the step and their launchers, templated on the storage
// type; each storage type is instantiated in a translation unit of its own.
//   phased schedule    QKV, attention, output projection: three kernels.
//   attn_oproj         QKV, then attention and output projection in one
//                      launch: the projection's workgroups follow every
//                      attention chunk in the grid, stream their rows of W_o
//                      while the last chunks and merges finish, and wait on
//                      per-sequence ready flags.
//   qkv_attn           QKV and attention in one launch: the attention chunks
//                      follow every QKV panel in the grid, load their K/V
//                      rows while the projection finishes, and wait on
//                      per-(batch group, head) panel counters; then the
//                      output projection.
// In a one-launch kernel a workgroup only waits on lower-numbered ones that
// never wait themselves, and each XCD dispatches its workgroups in index
// order, so every wait ends.
#pragma once

#include <hip/hip_ext.h>

#include "dab_gemv.h"

namespace dab {
namespace dev {

// Launch `kernel(a...)` on `s`; with events, through hipExtLaunchKernel,
// which records them at the kernel's own start and end.
template <typename K, typename... A>
inline hipError_t dab_launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const LaunchEvents& ev,
                             A... a) {
    void* args[] = {static_cast<void*>(&a)...};
    const void* f = reinterpret_cast<const void*>(kernel);
    if (ev.start || ev.stop) return hipExtLaunchKernel(f, grid, block, args, lds, s, ev.start, ev.stop, 0);
    return hipLaunchKernel(f, grid, block, args, lds, s);
}

// Attention work index -> (sequence, kv head, chunk); kv head fastest, so
// concurrent items read neighbouring rows of one token range.
__device__ inline void attn_decode(const StepArgs& a, int i, int* b, int* g, int* c) {
    *g = i % a.nkv;
    const int rest = i / a.nkv;
    *c = rest % a.maxc;
    *b = rest / a.maxc;
}

template <typename T, int NB, bool EXACT>
__global__ __launch_bounds__(256) void qkv_kernel(StepArgs a) {
    extern __shared__ f32x4 xs_raw[];
    __shared__ QkvShared<T, NB> sm;
    DAB_TRACE_POINT(a, 0);
    publish_seq_chunks(a);
    int panel, bgi;
    if (panel_decode(a.qkv.nbg, a.qkv.panels, blockIdx.x, &panel, &bgi))
        qkv_panel<T, NB, EXACT, kQkvPlain>(a, panel, bgi, reinterpret_cast<float*>(xs_raw), sm);
    DAB_TRACE_POINT(a, 3);
}

template <typename T, int NB, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && G == 1 && NB == 1 ? 4 : 1)))
void qkv_attn_kernel(StepArgs a) {
    extern __shared__ f32x4 lds_raw[];   // the QKV panel's staged inputs, or attention scratch
    __shared__ QkvShared<T, NB> qsm;
    __shared__ int s_flag;
    DAB_TRACE_POINT(a, 0);
    if ((int)blockIdx.x < a.qkv.items) {
        int panel, bgi;
        if (panel_decode(a.qkv.nbg, a.qkv.panels, blockIdx.x, &panel, &bgi))
            qkv_panel<T, NB, true, kQkvSignalGroup>(a, panel, bgi, reinterpret_cast<float*>(lds_raw), qsm);
    } else {
        int b, g, c;
        attn_decode(a, blockIdx.x - a.qkv.items, &b, &g, &c);
        attn_item<T, D, G, false, true>(a, b, g, c, *reinterpret_cast<AttnShared<D, G>*>(lds_raw), &s_flag);
    }
    DAB_TRACE_POINT(a, 3);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_kernel(StepArgs a) {
    __shared__ AttnShared<D, G> sm;
    __shared__ int s_flag;
    int b, g, c;
    DAB_TRACE_POINT(a, 0);
    attn_decode(a, blockIdx.x, &b, &g, &c);
    attn_item<T, D, G, false, false>(a, b, g, c, sm, &s_flag);
    DAB_TRACE_POINT(a, 3);
}

// Four waves per SIMD, as the attention kernel alone gets: all 1024 chunks of
// a 7B-sized step resident at once.
template <typename T, int D, int G, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && G == 1 && NB == 1 ? 4 : 1))) void attn_oproj_kernel(StepArgs a) {
    extern __shared__ f32x4 lds_raw[];   // attention scratch, or the projection's staged inputs
    __shared__ int s_flag;
    DAB_TRACE_POINT(a, 0);
    if ((int)blockIdx.x < a.attn_items) {
        int b, g, c;
        attn_decode(a, blockIdx.x, &b, &g, &c);
        attn_item<T, D, G, true, false>(a, b, g, c, *reinterpret_cast<AttnShared<D, G>*>(lds_raw), &s_flag);
    } else {
        int panel, bgi;
        if (panel_decode(a.oproj.nbg, a.oproj.panels, blockIdx.x - a.attn_items, &panel, &bgi))
            oproj_panel<T, 2, NB, true, true>(a, panel, bgi, reinterpret_cast<float*>(lds_raw));
    }
    DAB_TRACE_POINT(a, 3);
}

// The whole step in one launch, its workgroups in dependency order: the QKV
// panels (q heads, then k, then v heads), the attention chunks, the output
// projection's panels.  A chunk waits for the q panels of its group's query
// heads, the chunk with the new token also for the group's k and v panels
// before that token; a projection panel streams its rows of W_o from the
// moment it has a slot and waits for its sequences' attention output.
// Every wait is on lower-numbered workgroups, which never wait on higher
// ones, and each XCD dispatches its workgroups in index order, so every wait
// ends.  The counters are re-armed inside the launch by their last readers
// (see oproj_panel), so consecutive calls need no clearing in between.
template <typename T, int NB, int D, int G, bool EXACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && G == 1 && NB == 1 ? 4 : 1)))
void fused_kernel(StepArgs a) {
    extern __shared__ f32x4 lds_raw[];   // the QKV panel's staged inputs, attention scratch, or the projection's
    __shared__ QkvShared<T, NB> qsm;
    __shared__ int s_flag;
    DAB_TRACE_POINT(a, 0);
    const int i = blockIdx.x;
    if (i < a.qkv.items) {
        qkv_panel<T, NB, EXACT, kQkvSignalSeq>(a, i, 0, reinterpret_cast<float*>(lds_raw), qsm);
    } else if (i < a.qkv.items + a.attn_items) {
        int b, g, c;
        attn_decode(a, i - a.qkv.items, &b, &g, &c);
        attn_item<T, D, G, true, true>(a, b, g, c, *reinterpret_cast<AttnShared<D, G>*>(lds_raw), &s_flag);
    } else {
        int panel, bgi;
        if (panel_decode(a.oproj.nbg, a.oproj.panels, i - a.qkv.items - a.attn_items, &panel, &bgi))
            oproj_panel<T, 2, NB, true, true, true>(a, panel, bgi, reinterpret_cast<float*>(lds_raw));
    }
    DAB_TRACE_POINT(a, 3);
}

// Log-sum-exp merge of the chunk partials of one (sequence, q head), after
// the attention kernel (phased schedule, split merge).  The arithmetic and
// its order are those of the merge inside the attention kernel (thread
// (part, d) sums chunks part, part + PARTS, ... in order; maxima and sums by
// wave reductions, the waves in order), so the bits are the same; only the
// loads differ: plain loads after the kernel boundary, up to 32
// chunks per thread requested at once.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(StepArgs a) {
    constexpr int PARTS = 256 / D, R = 32;
    __shared__ float w[kMaxChunks], cl[kMaxChunks], red[4], acc[PARTS][D];
    DAB_TRACE_POINT(a, 0);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = blockIdx.x / a.nq, h = blockIdx.x - b * a.nq;
    int2 pre;
    if (a.seq_chunk) pre = reinterpret_cast<const int2*>(a.seq_chunk)[b];
    int p;
    if (!pos_valid(a, b, &p)) return;
    const int nchunk = seq_chunk_of(a, b, p, a.seq_chunk ? &pre : nullptr).n;
    const size_t pbase = ((size_t)b * a.nq + h) * a.maxc;     // chunk cc: pbase + cc
    const int d = t % D, part = t / D;
    float v0[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int cc = part + q * PARTS;
        v0[q] = cc < nchunk ? a.attn_o[(pbase + cc) * D + d] : 0.f;
    }
    for (int cc = t; cc < nchunk; cc += 256) {
        w[cc] = a.attn_ml[(pbase + cc) * 2];
        cl[cc] = a.attn_ml[(pbase + cc) * 2 + 1];
    }
    __syncthreads();
    float v = kNegInf;
    for (int cc = t; cc < nchunk; cc += 256) v = fmaxf(v, w[cc]);
    const float mx = wave_max(v);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float ls = 0.f;
    for (int cc = t; cc < nchunk; cc += 256) {
        const float wt = __builtin_amdgcn_exp2f(w[cc] - M);       // every chunk has a token: m finite
        ls += wt * cl[cc];
        w[cc] = wt;
    }
    const float lsum = wave_sum(ls);
    __syncthreads();                     // weights visible, red read by everyone
    if (lane == 0) red[wave] = lsum;
    float s = 0.f;
    for (int q0 = 0; part + q0 * PARTS < nchunk; q0 += R) {
        float vq[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int cc = part + (q0 + q) * PARTS;
            vq[q] = q0 == 0 ? v0[q] : (cc < nchunk ? a.attn_o[(pbase + cc) * D + d] : 0.f);
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int cc = part + (q0 + q) * PARTS;
            if (cc < nchunk) s += w[cc] * vq[q];
        }
    }
    acc[part][d] = s;
    __syncthreads();
    if (t < D) {
        const float L = red[0] + red[1] + red[2] + red[3];
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < PARTS; ++q) tot += acc[q][t];
        const size_t ai = (size_t)b * a.n_q + (size_t)h * D + t;
        a.a[ai] = tot / L;
        if constexpr (sizeof(T) == 2) a.a16[ai] = from_f32<uint16_t>(tot / L);   // input of the MFMA projection
    }
    DAB_TRACE_POINT(a, 3);
}

template <typename T, int RW, int NB, bool EXACT>
__global__ __launch_bounds__(256) void oproj_kernel(StepArgs a) {
    extern __shared__ f32x4 xs_raw[];
    DAB_TRACE_POINT(a, 0);
    // re-arm the panel counters of a one-launch QKV + attention that ran before
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < a.qkv.nbg * (a.nq + 2 * a.nkv); i += 256) set_counter(&a.head_cnt[i], 0);
    int panel, bgi;
    if (panel_decode(a.oproj.nbg, a.oproj.panels, blockIdx.x, &panel, &bgi))
        oproj_panel<T, RW, NB, EXACT, false>(a, panel, bgi, reinterpret_cast<float*>(xs_raw));
    DAB_TRACE_POINT(a, 3);
}

// MFMA panels of the phased schedule (bf16, batch >= 8)
template <bool QKV>
__device__ inline void mfma_prologue(const StepArgs& a, u32x4* nw_raw, int threads) {
    if constexpr (QKV) {
        publish_seq_chunks(a);
        for (int k = threadIdx.x * 8; k < a.H; k += threads * 8)
            nw_raw[k / 8] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.norm_w) + k);
        __syncthreads();
    } else {
        // re-arm the panel counters of a one-launch QKV + attention that ran before
        if (blockIdx.x == 0)
            for (int i = threadIdx.x; i < a.qkv.nbg * (a.nq + 2 * a.nkv); i += threads) set_counter(&a.head_cnt[i], 0);
    }
}

template <bool QKV, int TILES, int NG>
__global__ __launch_bounds__(kMfmaThreads) void mfma_panel_kernel(StepArgs a) {
    __shared__ MfmaLds<TILES, NG> lds;
    extern __shared__ u32x4 nw_raw[];    // QKV: norm_w, H bf16 values
    DAB_TRACE_POINT(a, 0);
    mfma_prologue<QKV>(a, nw_raw, kMfmaThreads);
    const PanelPlanDev& g = QKV ? a.qkv : a.oproj;
    int panel, bgi;
    if (panel_decode(g.nbg, g.panels, blockIdx.x, &panel, &bgi))
        mfma_panel<QKV, TILES, NG>(a, panel, bgi, lds, reinterpret_cast<const uint16_t*>(nw_raw));
    DAB_TRACE_POINT(a, 3);
}

template <bool QKV, int TILES>
__global__ __launch_bounds__(kMfmaResThreads) void mfma_res_kernel(StepArgs a) {
    __shared__ MfmaResLds<TILES> lds;
    extern __shared__ u32x4 nw_raw[];    // QKV: norm_w, H bf16 values
    DAB_TRACE_POINT(a, 0);
    mfma_prologue<QKV>(a, nw_raw, kMfmaResThreads);
    const PanelPlanDev& g = QKV ? a.qkv : a.oproj;
    int panel, bgi;
    if (panel_decode(g.nbg, g.panels, blockIdx.x, &panel, &bgi))
        mfma_res_panel<QKV, TILES>(a, panel, bgi, lds, reinterpret_cast<const uint16_t*>(nw_raw));
    DAB_TRACE_POINT(a, 3);
}

template <bool QKV, int TILES, int NG, int NWIN>
__global__ __launch_bounds__(kMfmaStrThreads) void mfma_str_kernel(StepArgs a) {
    __shared__ MfmaStrLds<TILES, NG> lds;
    DAB_TRACE_POINT(a, 0);
    if constexpr (!QKV) mfma_prologue<false>(a, nullptr, kMfmaStrThreads);
    else publish_seq_chunks(a);
    const PanelPlanDev& g = QKV ? a.qkv : a.oproj;
    int panel, bgi;
    if (panel_decode(g.nbg, g.panels, blockIdx.x, &panel, &bgi))
        mfma_str_panel<QKV, TILES, NG, NWIN>(a, panel, bgi, lds);
    DAB_TRACE_POINT(a, 3);
}

template <int NG, int NWIN>
__global__ __launch_bounds__(kMfmaStrThreads) void mfma_str_qkv24_kernel(StepArgs a) {
    __shared__ MfmaStrLds<2, NG> lds;
    DAB_TRACE_POINT(a, 0);
    publish_seq_chunks(a);
    int panel, bgi;
    if (panel_decode(a.qkv.nbg, a.qkv.panels, blockIdx.x, &panel, &bgi)) mfma_str_qkv24<NG, NWIN>(a, panel, bgi, lds);
    DAB_TRACE_POINT(a, 3);
}

// The streamed panel applies to 16 or 32 sequences per workgroup and K of
// 1024, 2048 or 4096.
inline bool mfma_streamed(const PanelPlan& g) {
    return (g.nb == 16 || g.nb == 32) && (g.K == 1024 || g.K == 2048 || g.K == 4096);
}

template <bool QKV, int NWIN>
void launch_mfma_str(const StepArgs& a, const PanelPlan& g, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(g.grid), block(kMfmaStrThreads);
    if (QKV && g.rows == 24) {
        if (g.nb == 32) dab_launch((mfma_str_qkv24_kernel<2, NWIN>), grid, block, 0, s, ev, a);
        else dab_launch((mfma_str_qkv24_kernel<1, NWIN>), grid, block, 0, s, ev, a);
        return;
    }
    const int key = (g.rows == 32 ? 2 : 0) + (g.nb == 32 ? 1 : 0);
    switch (key) {
        case 0: dab_launch((mfma_str_kernel<QKV, 1, 1, NWIN>), grid, block, 0, s, ev, a); break;
        case 1: dab_launch((mfma_str_kernel<QKV, 1, 2, NWIN>), grid, block, 0, s, ev, a); break;
        case 2: dab_launch((mfma_str_kernel<QKV, 2, 1, NWIN>), grid, block, 0, s, ev, a); break;
        default: dab_launch((mfma_str_kernel<QKV, 2, 2, NWIN>), grid, block, 0, s, ev, a); break;
    }
}

// The resident-operand panel applies to 16 sequences per workgroup and K a
// multiple of 256 of at most kMfmaResMaxK.
inline bool mfma_resident(const PanelPlan& g) {
    return g.nb == 16 && g.K <= kMfmaResMaxK && g.K % (32 * kMfmaResWaves) == 0;
}

template <typename T, bool QKV>
hipError_t launch_mfma(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    if constexpr (sizeof(T) != 2) {
        return hipErrorInvalidValue;               // planned for bf16 only
    } else {
        const PanelPlan& g = QKV ? p.qkv : p.oproj;
        const size_t lds = QKV ? (size_t)p.H * 2 : 0;
        const dim3 grid(g.grid);
        if (mfma_streamed(g)) {
            if (g.K == 4096) launch_mfma_str<QKV, 4>(a, g, s, ev);
            else if (g.K == 2048) launch_mfma_str<QKV, 2>(a, g, s, ev);
            else launch_mfma_str<QKV, 1>(a, g, s, ev);
            return hipGetLastError();
        }
        if (mfma_resident(g)) {
            if (g.rows == 32) dab_launch((mfma_res_kernel<QKV, 2>), grid, dim3(kMfmaResThreads), lds, s, ev, a);
            else dab_launch((mfma_res_kernel<QKV, 1>), grid, dim3(kMfmaResThreads), lds, s, ev, a);
            return hipGetLastError();
        }
        const dim3 block(kMfmaThreads);
        const int key = (g.rows == 32 ? 2 : 0) + (g.nb == 32 ? 1 : 0);
        switch (key) {
            case 0: dab_launch((mfma_panel_kernel<QKV, 1, 1>), grid, block, lds, s, ev, a); break;
            case 1: dab_launch((mfma_panel_kernel<QKV, 1, 2>), grid, block, lds, s, ev, a); break;
            case 2: dab_launch((mfma_panel_kernel<QKV, 2, 1>), grid, block, lds, s, ev, a); break;
            default: dab_launch((mfma_panel_kernel<QKV, 2, 2>), grid, block, lds, s, ev, a); break;
        }
        return hipGetLastError();
    }
}

// K is a whole number of PanelDot K-blocks (4096 bf16 or 2048 fp32 values)
template <typename T>
inline bool exact_blocks(int K) { return K % PanelDot<T, 1, 1, true>::KB == 0; }

template <typename T, bool EXACT>
hipError_t launch_qkv_e(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(p.qkv.grid), block(kThreads);
    const size_t lds = p.qkv.lds;
    switch (p.qkv.nb) {
        case 1: dab_launch((qkv_kernel<T, 1, EXACT>), grid, block, lds, s, ev, a); break;
        case 2: dab_launch((qkv_kernel<T, 2, EXACT>), grid, block, lds, s, ev, a); break;
        case 4: dab_launch((qkv_kernel<T, 4, EXACT>), grid, block, lds, s, ev, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_qkv(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    if (p.qkv.mfma) return launch_mfma<T, true>(a, p, s, ev);
    return exact_blocks<T>(a.H) ? launch_qkv_e<T, true>(a, p, s, ev) : launch_qkv_e<T, false>(a, p, s, ev);
}

template <typename T, int RW, bool EXACT>
hipError_t launch_oproj_e(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(p.oproj.grid), block(kThreads);
    const size_t lds = p.oproj.lds;
    switch (p.oproj.nb) {
        case 1: dab_launch((oproj_kernel<T, RW, 1, EXACT>), grid, block, lds, s, ev, a); break;
        case 2: dab_launch((oproj_kernel<T, RW, 2, EXACT>), grid, block, lds, s, ev, a); break;
        case 4: dab_launch((oproj_kernel<T, RW, 4, EXACT>), grid, block, lds, s, ev, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int RW>
hipError_t launch_oproj_rw(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    return exact_blocks<T>(a.n_q) ? launch_oproj_e<T, RW, true>(a, p, s, ev) : launch_oproj_e<T, RW, false>(a, p, s, ev);
}

template <typename T>
hipError_t launch_oproj(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    if (p.oproj.mfma) return launch_mfma<T, false>(a, p, s, ev);
    switch (p.oproj.rows_per_wave) {
        case 1: return launch_oproj_rw<T, 1>(a, p, s, ev);
        case 2: return launch_oproj_rw<T, 2>(a, p, s, ev);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t launch_attn_d(const StepArgs& a, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(a.attn_items), block(kThreads);
    switch (a.G) {
#define DAB_G(NG) case NG: dab_launch((attn_kernel<T, D, NG>), grid, block, 0, s, ev, a); break;
        DAB_G(1) DAB_G(2) DAB_G(3) DAB_G(4) DAB_G(5) DAB_G(6) DAB_G(7) DAB_G(8)
#undef DAB_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_attn_oproj_g(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(p.attn_grid + p.oproj.grid), block(kThreads);
    const size_t lds = p.oproj.lds > sizeof(AttnShared<D, G>) ? p.oproj.lds : sizeof(AttnShared<D, G>);
    switch (p.oproj.nb) {
        case 1: dab_launch((attn_oproj_kernel<T, D, G, 1>), grid, block, lds, s, ev, a); break;
        case 2: dab_launch((attn_oproj_kernel<T, D, G, 2>), grid, block, lds, s, ev, a); break;
        case 4: dab_launch((attn_oproj_kernel<T, D, G, 4>), grid, block, lds, s, ev, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Shapes the one-launch attention + projection is instantiated for: whole
// K-blocks in the projection, two rows per wave, groups of 1, 2, 4 or 8.
template <typename T>
inline bool attn_oproj_supported(const Plan& p) {
    return exact_blocks<T>(p.n_q) && p.oproj.rows_per_wave == 2 && (p.G == 1 || p.G == 2 || p.G == 4 || p.G == 8);
}

template <typename T, int D>
hipError_t launch_attn_oproj_d(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    switch (p.G) {
        case 1: return launch_attn_oproj_g<T, D, 1>(a, p, s, ev);
        case 2: return launch_attn_oproj_g<T, D, 2>(a, p, s, ev);
        case 4: return launch_attn_oproj_g<T, D, 4>(a, p, s, ev);
        case 8: return launch_attn_oproj_g<T, D, 8>(a, p, s, ev);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int NB, int D>
hipError_t launch_qkv_attn_nd(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(p.qkv.grid + p.attn_grid), block(kThreads);
    size_t lds = p.qkv.lds;
    switch (p.G) {
#define DAB_G(NG)                                                                                           \
        case NG:                                                                                            \
            if (sizeof(AttnShared<D, NG>) > lds) lds = sizeof(AttnShared<D, NG>);                             \
            dab_launch((qkv_attn_kernel<T, NB, D, NG>), grid, block, lds, s, ev, a);                    \
            break;
        DAB_G(1) DAB_G(2) DAB_G(4) DAB_G(8)
#undef DAB_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int NB>
hipError_t launch_qkv_attn_n(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    return a.D == 128 ? launch_qkv_attn_nd<T, NB, 128>(a, p, s, ev) : launch_qkv_attn_nd<T, NB, 64>(a, p, s, ev);
}

template <typename T>
hipError_t launch_qkv_attn(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    if (!exact_blocks<T>(a.H)) return hipErrorInvalidValue;
    switch (p.qkv.nb) {
        case 1: return launch_qkv_attn_n<T, 1>(a, p, s, ev);
        case 2: return launch_qkv_attn_n<T, 2>(a, p, s, ev);
        case 4: return launch_qkv_attn_n<T, 4>(a, p, s, ev);
        default: return hipErrorInvalidValue;
    }
}

// Workgroups of the phased schedule's attention kernel one CU holds at once
// (0 if the runtime cannot say).
template <typename T, int D>
int attn_resident_d(int G) {
    const void* f = nullptr;
    switch (G) {
#define DAB_G(NG) case NG: f = reinterpret_cast<const void*>(attn_kernel<T, D, NG>); break;
        DAB_G(1) DAB_G(2) DAB_G(3) DAB_G(4) DAB_G(5) DAB_G(6) DAB_G(7) DAB_G(8)
#undef DAB_G
        default: return 0;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kThreads, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

template <typename T>
int attn_resident(int D, int G) {
    return D == 128 ? attn_resident_d<T, 128>(G) : D == 64 ? attn_resident_d<T, 64>(G) : 0;
}

template <typename T, int NB, int D>
hipError_t launch_fused_nd(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(p.qkv.grid + p.attn_grid + p.oproj.grid), block(kThreads);
    size_t lds = p.qkv.lds > p.oproj.lds ? p.qkv.lds : p.oproj.lds;
    switch (p.G) {
#define DAB_G(NG)                                                                                           \
        case NG:                                                                                            \
            if (sizeof(AttnShared<D, NG>) > lds) lds = sizeof(AttnShared<D, NG>);                             \
            if (exact_blocks<T>(p.H))                                                                       \
                dab_launch((fused_kernel<T, NB, D, NG, true>), grid, block, lds, s, ev, a);                 \
            else                                                                                            \
                dab_launch((fused_kernel<T, NB, D, NG, false>), grid, block, lds, s, ev, a);                \
            break;
        DAB_G(1) DAB_G(2) DAB_G(4) DAB_G(8)
#undef DAB_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int NB>
hipError_t launch_fused_n(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    return a.D == 128 ? launch_fused_nd<T, NB, 128>(a, p, s, ev) : launch_fused_nd<T, NB, 64>(a, p, s, ev);
}

// The whole step in one launch: built for groups of 1, 2, 4, 8, an output
// projection of whole K-blocks with two rows per wave, and one batch group
// of the same size in both projections.
template <typename T>
hipError_t launch_fused(const StepArgs& a, const Plan& p, hipStream_t s, const LaunchEvents& ev) {
    if (!exact_blocks<T>(p.n_q) || p.oproj.rows_per_wave != 2 || p.qkv.mfma || p.oproj.mfma ||
        p.qkv.nb != p.oproj.nb || p.qkv.nbg != 1)
        return hipErrorInvalidValue;
    switch (p.qkv.nb) {
        case 1: return launch_fused_n<T, 1>(a, p, s, ev);
        case 2: return launch_fused_n<T, 2>(a, p, s, ev);
        case 4: return launch_fused_n<T, 4>(a, p, s, ev);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_phase_t(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev) {
    if (p.schedule == DAB_SCHEDULE_FUSED) return launch_fused<T>(a, p, s, ev);
    if (p.schedule == DAB_SCHEDULE_QKV_ATTN) return phase == 0 ? launch_qkv_attn<T>(a, p, s, ev) : launch_oproj<T>(a, p, s, ev);
    if (phase == 0) return launch_qkv<T>(a, p, s, ev);
    if (p.schedule == DAB_SCHEDULE_ATTN_OPROJ) {
        if (!attn_oproj_supported<T>(p)) return hipErrorInvalidValue;
        return a.D == 128 ? launch_attn_oproj_d<T, 128>(a, p, s, ev) : launch_attn_oproj_d<T, 64>(a, p, s, ev);
    }
    if (phase == 1) return a.D == 128 ? launch_attn_d<T, 128>(a, s, ev) : launch_attn_d<T, 64>(a, s, ev);
    if (phase == 2 && p.split_merge) {
        const dim3 grid(p.B * p.nq), block(kThreads);
        if (a.D == 128) dab_launch((merge_kernel<T, 128>), grid, block, 0, s, ev, a);
        else dab_launch((merge_kernel<T, 64>), grid, block, 0, s, ev, a);
        return hipGetLastError();
    }
    return launch_oproj<T>(a, p, s, ev);
}

}  // namespace dev
}  // namespace dab
