// fp32 storage instantiation of the phase kernels.
#include "dab_phase.h"

namespace dab {
hipError_t launch_phase_f32(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev) {
    return dev::launch_phase_t<float>(a, p, phase, s, ev);
}
int attn_resident_f32(int D, int G) { return dev::attn_resident<float>(D, G); }
}  // namespace dab
