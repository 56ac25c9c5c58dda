// bf16 prefill instantiations for N = 32 (prefill_pc_impl.hpp).
#include "prefill_pc_launch.hpp"

namespace m3 {
hipError_t launch_prefill_bf16_n32(const PrefillParams& p, bool state_only, hipStream_t s) {
  return pc::launch_n<32>(p, state_only, s);
}
}  // namespace m3
