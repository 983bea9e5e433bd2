// MALA fused backward (placeholder until the kernel lands).
#include "mala_internal.h"
namespace mala {
hipError_t launch_bwd(const BwdArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mala
