// Stand-ins for the kernel launchers, for the host-only sanitizer build of the C-ABI's
// validation (tests/test_sanitize_cpu.py): every launch reports an error and touches nothing,
// so calls that pass validation end in TP_ERR_LAUNCH without reaching any device.
#include "../../megatron_tensor_transformer_linear_amd/csrc/common.hpp"

namespace tpk {
hipError_t launch_gemm_bf16(const GemmDesc&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_bf16_split(const GemmDesc&, float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_f32(const GemmDesc&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_attention(const AttnDesc&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_reduce_ln(const ReduceDesc&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace tpk
