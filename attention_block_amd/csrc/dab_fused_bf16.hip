// Fused decode step, bf16 storage.
#include "dab_fused.h"

namespace dab {
hipError_t launch_fused_bf16(const StepArgs& a, hipStream_t s) { return dev::launch_fused_t<uint16_t>(a, s); }
hipError_t launch_stage_qkv_bf16(const StepArgs& a, hipStream_t s) { return dev::launch_stage_qkv_t<uint16_t>(a, s); }
}  // namespace dab
