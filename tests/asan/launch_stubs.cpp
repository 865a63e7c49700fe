// Kernel launchers replaced by stubs for the host AddressSanitizer build of
// the C front end (mha_api.cpp): argument validation, workspace layout and
// status/error bookkeeping run instrumented on the CPU; a call that got past
// validation reaches a stub and reports "no device" (so does the lookup of
// the allocation-free entry point's device array).
#include "kernels.h"

namespace mha {
hipError_t launch_attention_bf16(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attention_f32(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_linear_bf16(const LinearArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_linear_f32(const LinearArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_add_layernorm_bf16(const AddNormArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_add_layernorm_f32(const AddNormArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_bf16(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_f32(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attention_bwd_bf16(const BwdArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attention_bwd_f32(const BwdArgs&, hipStream_t) { return hipErrorNoDevice; }
mha_status noalloc_scratch(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = 0;
  return report_error(MHA_ERR_HIP, "no device in the host sanitizer build");
}
}  // namespace mha
