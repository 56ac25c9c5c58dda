// bf16 prefill instantiations for N = 32 with the prologue (prefill_pc_impl.hpp).
#include "prefill_pc_launch.hpp"

namespace m3 {
hipError_t launch_prefill_bf16_n32_pro(const PrefillParams& p, bool state_only, hipStream_t s) {
  return pc::launch_n<32, true>(p, state_only, s);
}
}  // namespace m3
