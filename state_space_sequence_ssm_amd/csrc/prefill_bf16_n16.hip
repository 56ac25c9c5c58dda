// bf16 prefill instantiations for N = 16, plain core (prefill_pc_impl.hpp).
#include "prefill_pc_launch.hpp"

namespace m3 {
hipError_t launch_prefill_bf16_n16(const PrefillParams& p, bool state_only, hipStream_t s) {
  return pc::launch_n<16, false>(p, state_only, s);
}
}  // namespace m3
