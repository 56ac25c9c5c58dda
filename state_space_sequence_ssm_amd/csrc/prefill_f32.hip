// fp32-input instantiations of the fused prefill kernel (prefill_impl.hpp).
#include "prefill_impl.hpp"

namespace m3 {
hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t s) { return prefill_dt<float>(p, s); }
size_t prefill_lds_bytes_f32(int N, int P, bool rope) { return lds_n<float>(N, P, rope); }
}  // namespace m3
