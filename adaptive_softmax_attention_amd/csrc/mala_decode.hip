// MALA split-KV decode (placeholder until the kernel lands).
#include "mala_internal.h"
namespace mala {
hipError_t launch_decode(const DecodeArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mala
