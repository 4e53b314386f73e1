// bf16 storage instantiation of the phase kernels.
#include "dab_phase.h"

namespace dab {
hipError_t launch_phase_bf16(const StepArgs& a, const Plan& p, int phase, hipStream_t s, const LaunchEvents& ev) {
    return dev::launch_phase_t<uint16_t>(a, p, phase, s, ev);
}
int attn_resident_bf16(int D, int G) { return dev::attn_resident<uint16_t>(D, G); }
}  // namespace dab
