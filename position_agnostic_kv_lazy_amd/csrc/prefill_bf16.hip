// bf16 MFMA prefill (placeholder until the kernel lands).
#include "launch.hpp"

namespace lazyattn {

hipError_t launch_prefill_bf16(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace lazyattn
