// The three kernels of the phased schedule (QKV, attention, output
// projection) and their launchers, templated on the storage type; each
// storage type is instantiated in a translation unit of its own.
#pragma once

#include "dab_gemv.h"

namespace dab {
namespace dev {

template <typename T, int NB, bool EXACT>
__global__ __launch_bounds__(256) void qkv_kernel(StepArgs a) {
    extern __shared__ f32x4 xs_raw[];
    __shared__ QkvShared<T, NB> sm;
    DAB_TRACE_POINT(a, 0);
    int panel, bgi;
    if (panel_decode(a.qkv.nbg, a.qkv.panels, blockIdx.x, &panel, &bgi))
        qkv_panel<T, NB, EXACT>(a, panel, bgi, reinterpret_cast<float*>(xs_raw), sm);
    DAB_TRACE_POINT(a, 3);
}

// Attention work index -> (sequence, kv head, chunk); kv head fastest, so
// concurrent items read neighbouring rows of one token range.
__device__ inline void attn_decode(const StepArgs& a, int i, int* b, int* g, int* c) {
    *g = i % a.nkv;
    const int rest = i / a.nkv;
    *c = rest % a.maxc;
    *b = rest / a.maxc;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_kernel(StepArgs a) {
    __shared__ AttnShared<D, G> sm;
    __shared__ int s_flag;
    int b, g, c;
    DAB_TRACE_POINT(a, 0);
    attn_decode(a, blockIdx.x, &b, &g, &c);
    attn_item<T, D, G>(a, b, g, c, sm, &s_flag);
    DAB_TRACE_POINT(a, 3);
}

template <typename T, int RW, int NB, bool EXACT>
__global__ __launch_bounds__(256) void oproj_kernel(StepArgs a) {
    extern __shared__ f32x4 xs_raw[];
    DAB_TRACE_POINT(a, 0);
    int panel, bgi;
    if (panel_decode(a.oproj.nbg, a.oproj.panels, blockIdx.x, &panel, &bgi))
        oproj_panel<T, RW, NB, EXACT>(a, panel, bgi, reinterpret_cast<float*>(xs_raw));
    DAB_TRACE_POINT(a, 3);
}

// K is a whole number of PanelDot K-blocks (4096 bf16 or 2048 fp32 values)
template <typename T>
inline bool exact_blocks(int K) { return K % PanelDot<T, 1, 1, true>::KB == 0; }

template <typename T, bool EXACT>
hipError_t launch_qkv_e(const StepArgs& a, const Plan& p, hipStream_t s) {
    const dim3 grid(p.qkv.grid), block(kThreads);
    const size_t lds = p.qkv.lds;
    switch (p.qkv.nb) {
        case 1: hipLaunchKernelGGL((qkv_kernel<T, 1, EXACT>), grid, block, lds, s, a); break;
        case 2: hipLaunchKernelGGL((qkv_kernel<T, 2, EXACT>), grid, block, lds, s, a); break;
        case 4: hipLaunchKernelGGL((qkv_kernel<T, 4, EXACT>), grid, block, lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_qkv(const StepArgs& a, const Plan& p, hipStream_t s) {
    return exact_blocks<T>(a.H) ? launch_qkv_e<T, true>(a, p, s) : launch_qkv_e<T, false>(a, p, s);
}

template <typename T, int RW, bool EXACT>
hipError_t launch_oproj_e(const StepArgs& a, const Plan& p, hipStream_t s) {
    const dim3 grid(p.oproj.grid), block(kThreads);
    const size_t lds = p.oproj.lds;
    switch (p.oproj.nb) {
        case 1: hipLaunchKernelGGL((oproj_kernel<T, RW, 1, EXACT>), grid, block, lds, s, a); break;
        case 2: hipLaunchKernelGGL((oproj_kernel<T, RW, 2, EXACT>), grid, block, lds, s, a); break;
        case 4: hipLaunchKernelGGL((oproj_kernel<T, RW, 4, EXACT>), grid, block, lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int RW>
hipError_t launch_oproj_rw(const StepArgs& a, const Plan& p, hipStream_t s) {
    return exact_blocks<T>(a.n_q) ? launch_oproj_e<T, RW, true>(a, p, s) : launch_oproj_e<T, RW, false>(a, p, s);
}

template <typename T>
hipError_t launch_oproj(const StepArgs& a, const Plan& p, hipStream_t s) {
    switch (p.oproj.rows_per_wave) {
        case 1: return launch_oproj_rw<T, 1>(a, p, s);
        case 2: return launch_oproj_rw<T, 2>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t launch_attn_d(const StepArgs& a, hipStream_t s) {
    const dim3 grid(a.attn_items), block(kThreads);
    switch (a.G) {
#define DAB_G(NG) case NG: hipLaunchKernelGGL((attn_kernel<T, D, NG>), grid, block, 0, s, a); break;
        DAB_G(1) DAB_G(2) DAB_G(3) DAB_G(4) DAB_G(5) DAB_G(6) DAB_G(7) DAB_G(8)
#undef DAB_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_phase_t(const StepArgs& a, const Plan& p, int phase, hipStream_t s) {
    switch (phase) {
        case 0: return launch_qkv<T>(a, p, s);
        case 1: return a.D == 128 ? launch_attn_d<T, 128>(a, s) : launch_attn_d<T, 64>(a, s);
        default: return launch_oproj<T>(a, p, s);
    }
}

}  // namespace dev
}  // namespace dab
