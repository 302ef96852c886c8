// Launch stubs for the host-only sanitizer build of the C ABI: the argument
// validation, workspace sizing and launch-argument marshalling in path_abi.cpp
// and path_plan.cpp run for real, nothing is sent to a device.
#include <hip/hip_runtime.h>

#include "path_bwd.h"
#include "path_kernels.h"

namespace path {
hipError_t launch_prep(const PrepArgs &, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd(const FwdArgs &, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecodeArgs &, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_produce(const ProduceArgs &, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_cache(const CacheArgs &, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd(const BwdArgs &, bool, hipStream_t) { return hipSuccess; }
size_t decode_scratch_bytes() { return size_t(16) << 20; }
hipError_t decode_scratch(void **) { return hipErrorNoDevice; }  // no device in this build
}  // namespace path
