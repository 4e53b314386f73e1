// Fused decode step, fp32 storage.
#include "dab_fused.h"

namespace dab {
hipError_t launch_fused_f32(const StepArgs& a, hipStream_t s) { return dev::launch_fused_t<float>(a, s); }
hipError_t launch_stage_qkv_f32(const StepArgs& a, hipStream_t s) { return dev::launch_stage_qkv_t<float>(a, s); }
}  // namespace dab
