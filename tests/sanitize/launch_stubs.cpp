// Stand-ins for the kernel launchers and the three HIP runtime calls of the
// host validation layer, for a CPU-only build of api.cpp and paley.cpp under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every launcher reports
// that no device is present, so a call that passes validation returns
// HR_EDEVICE; nothing here touches memory behind the caller's pointers.
#include <hip/hip_runtime_api.h>

#include "../../hadamard_rotation_preprocessing_amd/csrc/plan.h"

namespace hr {
int launch_rotate(const RotPlan&, void*) { return static_cast<int>(hipErrorNoDevice); }
int launch_colrot(const ColArgs&, void*) { return static_cast<int>(hipErrorNoDevice); }
int launch_fast(const FastKey&, const FastArgs&, void*) { return -static_cast<int>(hipErrorNoDevice); }
int launch_kron(const FastKey&, const KronArgs&, void*) { return -static_cast<int>(hipErrorNoDevice); }
int launch_dequant(const DqArgs&, void*) { return static_cast<int>(hipErrorNoDevice); }
int scratch_address(void**) { return static_cast<int>(hipErrorNoDevice); }
}  // namespace hr

extern "C" {
const char* hipGetErrorString(hipError_t) { return "no device (host-only sanitizer build)"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }
}
