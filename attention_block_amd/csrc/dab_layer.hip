// The decoder layer with the FFN's weight stream started under the attention
// block's tail: after the QKV kernel, one launch holds the attention chunks,
// the output projection's panels and the FFN gate/up panels, in that order;
// the FFN down kernel follows.  A gate/up panel issues its rows of W_gate and
// W_up as soon as it has a slot and then waits for h, which the projection
// panels publish (see oproj_panel); the kernel boundary between the output
// projection and the FFN, and the FFN's ramp, go away.  The operator-fusion
// page, section 1, places the FFN after the attention block's residual; the
// ClusterFusion page, section 3.3, overlaps a stage's loads with the work
// before it.
//
// Every wait is on lower-numbered workgroups (gate/up panels on projection
// panels, projection panels on attention chunks), which never wait on higher
// ones, and each XCD dispatches its workgroups in index order, so every wait
// ends.
#include <hip/hip_runtime.h>

#include "dab_ffn.h"
#include "dab_phase.h"

namespace dab {
namespace dev {
namespace {

template <typename T, int D, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && NB == 1 ? 4 : 1)))
void layer_attn_ffn_kernel(StepArgs a, FfnArgs f) {
    extern __shared__ f32x4 lds_raw[];
    __shared__ int s_flag;
    __shared__ FfnShared<NB> sm;
    DAB_TRACE_POINT(a, 0);
    const int o0 = a.attn_items, f0 = a.attn_items + a.oproj.items;
    int panel, bgi;
    if ((int)blockIdx.x < o0) {
        int b, g, c;
        attn_decode(a, blockIdx.x, &b, &g, &c);
        attn_item<T, D, 1, true, false>(a, b, g, c, *reinterpret_cast<AttnShared<D, 1>*>(lds_raw), &s_flag);
    } else if ((int)blockIdx.x < f0) {
        if (panel_decode(a.oproj.nbg, a.oproj.panels, blockIdx.x - o0, &panel, &bgi))
            oproj_panel<T, 2, NB, true, true, false, true>(a, panel, bgi, reinterpret_cast<float*>(lds_raw));
    } else {
        if (panel_decode(f.gu.nbg, f.gu.panels, blockIdx.x - f0, &panel, &bgi))
            ffn_gate_up_panel<T, NB, true, true>(f, panel, bgi, reinterpret_cast<float*>(lds_raw), sm);
    }
    DAB_TRACE_POINT(a, 3);
}

template <typename T, int D>
hipError_t launch_layer_d(const StepArgs& a, const FfnArgs& f, const Plan& p, const FfnPlan& fp, hipStream_t s,
                          const LaunchEvents& ev) {
    const dim3 grid(p.attn_grid + p.oproj.grid + fp.gu.grid), block(kThreads);
    size_t lds = sizeof(AttnShared<D, 1>);
    if (p.oproj.lds > lds) lds = p.oproj.lds;
    if (fp.gu.lds > lds) lds = fp.gu.lds;
    switch (p.oproj.nb) {
        case 1: dab_launch((layer_attn_ffn_kernel<T, D, 1>), grid, block, lds, s, ev, a, f); break;
        case 2: dab_launch((layer_attn_ffn_kernel<T, D, 2>), grid, block, lds, s, ev, a, f); break;
        case 4: dab_launch((layer_attn_ffn_kernel<T, D, 4>), grid, block, lds, s, ev, a, f); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_layer_t(const StepArgs& a, const FfnArgs& f, const Plan& p, const FfnPlan& fp, hipStream_t s,
                          const LaunchEvents& ev) {
    return a.D == 128 ? launch_layer_d<T, 128>(a, f, p, fp, s, ev) : launch_layer_d<T, 64>(a, f, p, fp, s, ev);
}

}  // namespace
}  // namespace dev

// One query head per kv head in the one-launch attention + projection
// schedule, the VALU FFN panels, both GEMVs in whole K-blocks with the same
// batch grouping, and head dims 64 or 128.
bool layer_overlap_ok(const Plan& p, const FfnPlan& f) {
    const bool bf16 = p.dtype == DAB_BF16;
    const bool exact = bf16 ? dev::exact_blocks<uint16_t>(p.H) : dev::exact_blocks<float>(p.H);
    return p.schedule == DAB_SCHEDULE_ATTN_OPROJ && p.G == 1 && (p.D == 64 || p.D == 128) && !f.mfma &&
           f.dtype == p.dtype && f.B == p.B && f.H == p.H && exact && p.oproj.rows_per_wave == 2 &&
           f.gu.nb == p.oproj.nb && f.gu.nbg == p.oproj.nbg;
}

hipError_t launch_layer_attn_ffn(const StepArgs& a, const FfnArgs& f, const Plan& p, const FfnPlan& fp, hipStream_t s,
                                 const LaunchEvents& ev) {
    if (!layer_overlap_ok(p, fp) || !a.hand || a.hand != f.hand) return hipErrorInvalidValue;
    return p.dtype == DAB_BF16 ? dev::launch_layer_t<uint16_t>(a, f, p, fp, s, ev)
                               : dev::launch_layer_t<float>(a, f, p, fp, s, ev);
}

}  // namespace dab
