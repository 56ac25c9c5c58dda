// bf16-input instantiations of the fused prefill kernel (prefill_impl.hpp).
#include "prefill_impl.hpp"

namespace m3 {
hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t s) { return prefill_dt<bf16_t>(p, s); }
size_t prefill_lds_bytes_bf16(int N, int P, bool rope) { return lds_n<bf16_t>(N, P, rope); }
}  // namespace m3
