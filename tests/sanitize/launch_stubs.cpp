// Host-only stand-ins for the kernel launchers and the HIP calls that the
// C-ABI (kda_abi.cpp) makes after its argument checks, so that the checks can
// be built with the host sanitizers and run without a GPU or the HIP runtime.
// Every stand-in fails: a call that gets past the checks returns KDA_ERR_HIP.
#include "../../gated_delta_rule_55_amd/csrc/kda_internal.h"

namespace kda {

hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_dplr(const PrefillArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_backward(const BackwardArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    return hipErrorNoDevice;
}

}  // namespace kda

extern "C" const char *hipGetErrorString(hipError_t e) {
    return e == hipErrorNoDevice ? "no device (host-only build)" : "hip error (host-only build)";
}
