// bf16 prefill instantiations for N = 128 with the prologue (prefill_pc_impl.hpp).
#include "prefill_pc_launch.hpp"

namespace m3 {
hipError_t launch_prefill_bf16_n128_pro(const PrefillParams& p, bool state_only, hipStream_t s) {
  return pc::launch_n<128, true>(p, state_only, s);
}
}  // namespace m3
