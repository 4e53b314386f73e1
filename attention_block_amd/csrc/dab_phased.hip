// One kernel per phase (QKV, attention, output projection), and the
// workspace fill kernel.  Same device functions as the fused kernel, with
// the waits switched off: the stream orders the phases.
#include "dab_fused.h"

namespace dab {
namespace dev {

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <typename T, int BG, bool QKV>
__global__ __launch_bounds__(256) void phased_gemv_kernel(StepArgs a) {
    __shared__ GemvShared<BG> sm;
    __shared__ int s_flag;
    const GemvPlanDev& g = QKV ? a.qkv : a.oproj;
    int tile, bgi;
    DAB_TRACE_POINT(a, 0);
    // K-split-major: concurrent tiles cover whole rows of W (all slabs of a
    // row block), so HBM pages are read whole; slab-major order measured
    // about 1.5x slower for the QKV stream
    if (gemv_decode(g.nbg, g.tiles, blockIdx.x, &tile, &bgi))
        gemv_tile<T, BG, QKV, false>(a, tile % g.slabs, tile / g.slabs, bgi, 0u, sm, &s_flag);
    DAB_TRACE_POINT(a, 3);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void phased_attn_kernel(StepArgs a) {
    __shared__ AttnShared<D, G> sm;
    __shared__ int s_flag;
    int b, g, c;
    DAB_TRACE_POINT(a, 0);
    attn_decode(a, a.nkv, blockIdx.x, &b, &g, &c);
    attn_item<T, D, G, false>(a, b, g, c, 0u, sm, &s_flag);
    DAB_TRACE_POINT(a, 3);
}

template <typename T, bool QKV>
hipError_t launch_gemv_t(const StepArgs& a, hipStream_t s) {
    const dim3 grid((QKV ? a.qkv : a.oproj).items), block(256);
    switch (a.qkv_bg) {
        case 1: hipLaunchKernelGGL((phased_gemv_kernel<T, 1, QKV>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((phased_gemv_kernel<T, 2, QKV>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((phased_gemv_kernel<T, 4, QKV>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((phased_gemv_kernel<T, 8, QKV>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_d(const StepArgs& a, hipStream_t s) {
    const dim3 grid(a.attn_items), block(256);
    switch (a.G) {
#define DAB_G(NG) case NG: hipLaunchKernelGGL((phased_attn_kernel<T, D, NG>), grid, block, 0, s, a); break;
        DAB_G(1) DAB_G(2) DAB_G(3) DAB_G(4) DAB_G(5) DAB_G(6) DAB_G(7) DAB_G(8)
#undef DAB_G
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_phase_t(const StepArgs& a, int phase, hipStream_t s) {
    switch (phase) {
        case 0: return launch_gemv_t<T, true>(a, s);
        case 1: return a.D == 128 ? launch_attn_d<T, 128>(a, s) : launch_attn_d<T, 64>(a, s);
        default: return launch_gemv_t<T, false>(a, s);
    }
}

}  // namespace dev

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(dev::fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

hipError_t launch_phase(const StepArgs& a, bool bf16, int phase, hipStream_t s) {
#ifdef DAB_TRACE
    StepArgs t = a;   // phases trace at the item numbers the fused schedule uses
    t.trace_base = phase == 0 ? 0 : phase == 1 ? a.qkv.items : a.qkv.items + a.attn_items;
    return bf16 ? dev::launch_phase_t<uint16_t>(t, phase, s) : dev::launch_phase_t<float>(t, phase, s);
#else
    return bf16 ? dev::launch_phase_t<uint16_t>(a, phase, s) : dev::launch_phase_t<float>(a, phase, s);
#endif
}

hipError_t launch_fused(const StepArgs& a, bool bf16, hipStream_t s) {
    return bf16 ? launch_fused_bf16(a, s) : launch_fused_f32(a, s);
}

hipError_t launch_two_stage(const StepArgs& a, bool bf16, int stage, hipStream_t s) {
    if (stage == 0) {
#ifdef DAB_TRACE
        StepArgs t = a;
        t.trace_base = 0;
        return bf16 ? launch_stage_qkv_bf16(t, s) : launch_stage_qkv_f32(t, s);
#else
        return bf16 ? launch_stage_qkv_bf16(a, s) : launch_stage_qkv_f32(a, s);
#endif
    }
    StepArgs b = a;   // attention and output tiles: items from the first attention chunk on
    b.item_lo = a.qkv.items;
#ifdef DAB_TRACE
    b.trace_base = b.item_lo;
#endif
    return bf16 ? launch_fused_bf16(b, s) : launch_fused_f32(b, s);
}

}  // namespace dab
