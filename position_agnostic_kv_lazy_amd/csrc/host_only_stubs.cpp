// Kernel launchers for the host-only sanitizer build (build.py --sanitize).
//
// That build compiles the C ABI's host layer (lazy_attn_host.cpp,
// decode_split.cpp, cache_sim.cpp) with AddressSanitizer and
// UndefinedBehaviorSanitizer for CPU-only tests of the argument checks, the
// table packer and validator, the shared-decode planner, the cos/sin tables
// and the cache simulator.  It has no device code: every launcher reports
// that there is no device, as the real library does on a machine without a
// GPU.  Never part of liblazyattn.so.
#include "launch.hpp"

namespace lazyattn {

hipError_t launch_attn_f32(const AttnArgs&, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_bf16(const AttnArgs&, const DecodeSplit&, void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t decode_scratch_ptr(void**) { return hipErrorNoDevice; }
hipError_t launch_decode_shared_bf16(const AttnArgs&, const SharedPlanView&, void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_prefill_bf16(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_store_kv(const void*, const void*, int64_t, const int64_t*, const int32_t*,
                           const float*, int, int, int, bool, bool, void*, void*, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace lazyattn
