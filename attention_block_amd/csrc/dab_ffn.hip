// Kernels and launchers of the FFN half of the layer (bf16 and fp32 storage).
#include <hip/hip_runtime.h>

#include "dab_ffn.h"
#include "dab_phase.h"

namespace dab {
namespace dev {
namespace {

template <typename T, int NB, bool EXACT>
__global__ __launch_bounds__(256) void ffn_gate_up_kernel(FfnArgs a) {
    extern __shared__ f32x4 xs_raw[];
    __shared__ FfnShared<NB> sm;
    DAB_TRACE_POINT(a, 0);
    int panel, bgi;
    if (panel_decode(a.gu.nbg, a.gu.panels, blockIdx.x, &panel, &bgi))
        ffn_gate_up_panel<T, NB, EXACT>(a, panel, bgi, reinterpret_cast<float*>(xs_raw), sm);
    DAB_TRACE_POINT(a, 3);
}

// NBLK 2..4 (bf16): the double-buffered dot product, held to the 168
// registers that keep three workgroups on a CU, as the LDS does (m of
// 11008 fp32 values: 44 KB each).
template <typename T, int NB, bool EXACT, int NBLK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NBLK >= 2 ? 3 : 1)))
void ffn_down_kernel(FfnArgs a) {
    extern __shared__ f32x4 xs_raw[];
    DAB_TRACE_POINT(a, 0);
    // after the overlapped layer's launch: its gate/up panels are past their
    // waits, so the ready counts of h go back to zero for the next call
    if (a.hand && blockIdx.x == 0)
        for (int i = threadIdx.x; i < a.B * kHCopies; i += blockDim.x)
            set_counter(&a.hand[h_flag_at(i / kHCopies, i % kHCopies)], 0);
    int panel, bgi;
    if (panel_decode(a.down.nbg, a.down.panels, blockIdx.x, &panel, &bgi))
        ffn_down_panel<T, 2, NB, EXACT, NBLK>(a, panel, bgi, reinterpret_cast<float*>(xs_raw));
    DAB_TRACE_POINT(a, 3);
}

template <bool GATE_UP, int TILES, int NG>
__global__ __launch_bounds__(kMfmaThreads) void ffn_mfma_kernel(FfnArgs a) {
    __shared__ MfmaLds<TILES, NG> lds;
    extern __shared__ u32x4 nw_raw[];    // gate/up: norm_w, H bf16 values
    DAB_TRACE_POINT(a, 0);
    if constexpr (GATE_UP) {
        for (int k = threadIdx.x * 8; k < a.H; k += kMfmaThreads * 8)
            nw_raw[k / 8] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.norm_w) + k);
        __syncthreads();
    }
    const PanelPlanDev& g = GATE_UP ? a.gu : a.down;
    int panel, bgi;
    if (panel_decode(g.nbg, g.panels, blockIdx.x, &panel, &bgi))
        ffn_mfma_panel<GATE_UP, TILES, NG>(a, panel, bgi, lds, reinterpret_cast<const uint16_t*>(nw_raw));
    DAB_TRACE_POINT(a, 3);
}

// One workgroup per CU (two, at 128 registers: 8B FFN at batch 16, gate/up 49.4 -> 56.7 us on MI355X).
template <int T, int NG, int NWIN>
__global__ __launch_bounds__(kMfmaStrThreads) void ffn_str_kernel(FfnArgs a) {
    __shared__ MfmaStrLds<T, NG> lds;
    DAB_TRACE_POINT(a, 0);
    int panel, bgi;
    if (panel_decode(a.gu.nbg, a.gu.panels, blockIdx.x, &panel, &bgi)) ffn_str_gate_up<T, NG, NWIN>(a, panel, bgi, lds);
    DAB_TRACE_POINT(a, 3);
}

template <int T, int NWIN>
void launch_ffn_str_t(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(a.gu.items), block(kMfmaStrThreads);
    if (a.gu.nb == 32) dab_launch((ffn_str_kernel<T, 2, NWIN>), grid, block, 0, s, ev, a);
    else dab_launch((ffn_str_kernel<T, 1, NWIN>), grid, block, 0, s, ev, a);
}

template <int NWIN>
void launch_ffn_str(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    switch (a.gu_tiles) {
        case 1: launch_ffn_str_t<1, NWIN>(a, s, ev); break;
        case 2: launch_ffn_str_t<2, NWIN>(a, s, ev); break;
        case 4: launch_ffn_str_t<4, NWIN>(a, s, ev); break;
        case 7: launch_ffn_str_t<7, NWIN>(a, s, ev); break;
        default: launch_ffn_str_t<8, NWIN>(a, s, ev); break;
    }
}

template <int NG, int NWIN>
__global__ __launch_bounds__(kMfmaStrThreads) void ffn_str_down_kernel(FfnArgs a) {
    __shared__ MfmaStrLds<1, NG> lds;
    DAB_TRACE_POINT(a, 0);
    int panel, bgi;
    if (panel_decode(a.down.nbg, a.down.panels, blockIdx.x, &panel, &bgi)) ffn_str_down<NG, NWIN>(a, panel, bgi, lds);
    DAB_TRACE_POINT(a, 3);
}

template <int NWIN>
void launch_ffn_str_down(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(a.down.items), block(kMfmaStrThreads);
    if (a.down.nb == 32) dab_launch((ffn_str_down_kernel<2, NWIN>), grid, block, 0, s, ev, a);
    else dab_launch((ffn_str_down_kernel<1, NWIN>), grid, block, 0, s, ev, a);
}

// The streamed down panel: one tile, F = 1024 NWIN for these NWIN (others take the staged panel).
inline bool ffn_str_down_ok(const FfnArgs& a) {
    const int nw = a.F / 1024;
    return a.down_tiles == 1 && a.F % 1024 == 0 && (nw == 1 || nw == 2 || nw == 4 || nw == 8 || nw == 14);
}

template <typename T, bool GATE_UP>
hipError_t launch_ffn_mfma(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    if constexpr (sizeof(T) != 2) {
        return hipErrorInvalidValue;               // planned for bf16 only
    } else {
        const dim3 block(kMfmaThreads);
        if constexpr (GATE_UP) {
            // the streamed panel where H is 1024, 2048 or 4096
            if (a.gu_tiles > 0) {
                if (a.H == 4096) launch_ffn_str<4>(a, s, ev);
                else if (a.H == 2048) launch_ffn_str<2>(a, s, ev);
                else launch_ffn_str<1>(a, s, ev);
                return hipGetLastError();
            }
            const dim3 grid(a.gu.items);
            const size_t lds = (size_t)a.H * 2;
            if (a.gu.nb == 32) dab_launch((ffn_mfma_kernel<true, 2, 2>), grid, block, lds, s, ev, a);
            else dab_launch((ffn_mfma_kernel<true, 2, 1>), grid, block, lds, s, ev, a);
        } else {
            if (ffn_str_down_ok(a)) {
                switch (a.F / 1024) {
                    case 1: launch_ffn_str_down<1>(a, s, ev); break;
                    case 2: launch_ffn_str_down<2>(a, s, ev); break;
                    case 4: launch_ffn_str_down<4>(a, s, ev); break;
                    case 8: launch_ffn_str_down<8>(a, s, ev); break;
                    default: launch_ffn_str_down<14>(a, s, ev); break;
                }
                return hipGetLastError();
            }
            const dim3 grid(a.down.items);
            const int key = (a.down_tiles == 2 ? 2 : 0) + (a.down.nb == 32 ? 1 : 0);
            switch (key) {
                case 0: dab_launch((ffn_mfma_kernel<false, 1, 1>), grid, block, 0, s, ev, a); break;
                case 1: dab_launch((ffn_mfma_kernel<false, 1, 2>), grid, block, 0, s, ev, a); break;
                case 2: dab_launch((ffn_mfma_kernel<false, 2, 1>), grid, block, 0, s, ev, a); break;
                default: dab_launch((ffn_mfma_kernel<false, 2, 2>), grid, block, 0, s, ev, a); break;
            }
        }
        return hipGetLastError();
    }
}

template <typename T, bool EXACT>
hipError_t launch_gate_up_e(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(a.gu.items), block(kThreads);
    const size_t lds = (size_t)a.gu.nb * a.H * sizeof(float);
    switch (a.gu.nb) {
        case 1: dab_launch((ffn_gate_up_kernel<T, 1, EXACT>), grid, block, lds, s, ev, a); break;
        case 2: dab_launch((ffn_gate_up_kernel<T, 2, EXACT>), grid, block, lds, s, ev, a); break;
        case 4: dab_launch((ffn_gate_up_kernel<T, 4, EXACT>), grid, block, lds, s, ev, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool EXACT, int NBLK>
hipError_t launch_down_n(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    const dim3 grid(a.down.items), block(kThreads);
    const size_t lds = (size_t)a.down.nb * a.F * sizeof(float);
    switch (a.down.nb) {
        case 1: dab_launch((ffn_down_kernel<T, 1, EXACT, NBLK>), grid, block, lds, s, ev, a); break;
        case 2: dab_launch((ffn_down_kernel<T, 2, EXACT, NBLK>), grid, block, lds, s, ev, a); break;
        case 4: dab_launch((ffn_down_kernel<T, 4, EXACT, NBLK>), grid, block, lds, s, ev, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// bf16 rows of 2 to 4 K-blocks (F in (4096, 16384]) on the double-buffered
// dot product, the rest on PanelDot
template <typename T, bool EXACT>
hipError_t launch_down_e(const FfnArgs& a, hipStream_t s, const LaunchEvents& ev) {
    if constexpr (sizeof(T) == 2) {
        const int kb = PanelDot<T, 1, 1, true>::KB, nblk = (a.F + kb - 1) / kb;
        if (nblk == 2) return launch_down_n<T, EXACT, 2>(a, s, ev);
        if (nblk == 3) return launch_down_n<T, EXACT, 3>(a, s, ev);
        if (nblk == 4) return launch_down_n<T, EXACT, 4>(a, s, ev);
    }
    return launch_down_n<T, EXACT, 0>(a, s, ev);
}

template <typename T>
hipError_t launch_ffn_t(const FfnArgs& a, int phase, hipStream_t s, const LaunchEvents& ev) {
    if (a.mfma) return phase == 0 ? launch_ffn_mfma<T, true>(a, s, ev) : launch_ffn_mfma<T, false>(a, s, ev);
    if (phase == 0)
        return exact_blocks<T>(a.H) ? launch_gate_up_e<T, true>(a, s, ev) : launch_gate_up_e<T, false>(a, s, ev);
    if (phase == 1)
        return exact_blocks<T>(a.F) ? launch_down_e<T, true>(a, s, ev) : launch_down_e<T, false>(a, s, ev);
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace dev

hipError_t launch_ffn_phase(const FfnArgs& a, int dtype, int phase, hipStream_t s, const LaunchEvents& ev) {
    return dtype == DAB_BF16 ? dev::launch_ffn_t<uint16_t>(a, phase, s, ev) : dev::launch_ffn_t<float>(a, phase, s, ev);
}

}  // namespace dab
