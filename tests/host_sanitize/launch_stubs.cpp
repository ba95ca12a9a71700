// Kernel launchers replaced by stubs, so that the host half of the library
// (argument checks, plans, workspace layouts: abi.cpp and plan.cpp) can be
// built by the host compiler alone with AddressSanitizer and
// UndefinedBehaviorSanitizer and driven by the CPU tests. Every stub reports
// that no device is present; the CPU tests never reach a launch.
#include "fa_internal.h"

namespace fa {

hipError_t launch_prefill_f32(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_bf16(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_fp8(const void*, const void*, const void*, const float*, const float*, const float*,
                              void*, float*, int, int, int, int, int, int, float, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attention_bwd(const BwdLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t bwd_scratch(void**) { return hipErrorNoDevice; }
hipError_t device_status_ptr(unsigned**) { return hipErrorNoDevice; }
hipError_t launch_prefill_paged_bf16(const PrefillArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefix_bf16(const PrefillArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_split(const DecodeArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_split_mfma(const DecodeArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_lse_merge(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gather_kv(const void*, int, const int32_t*, int, int, int, int, int, int, int, void*,
                            hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace fa
