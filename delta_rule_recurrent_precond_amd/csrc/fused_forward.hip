// Fused OSDN forward on matrix cores (placeholder until the kernel lands).
#include "device.h"
#include "launch.h"

namespace osdn {

bool fused_supported(int, int, int, int) { return false; }

hipError_t launch_fused_forward(const FusedArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace osdn
