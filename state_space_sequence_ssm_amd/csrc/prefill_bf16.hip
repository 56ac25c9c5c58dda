// bf16 prefill dispatch: the producer/consumer fused kernel (prefill_pc_impl.hpp),
// instantiated per N in prefill_bf16_n*.hip.
#include "prefill_pc_impl.hpp"

namespace m3 {

hipError_t launch_prefill_bf16_n16(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n32(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n64(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n128(const PrefillParams& p, bool state_only, hipStream_t s);

hipError_t launch_prefill_bf16(const PrefillParams& p, bool state_only, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_prefill_bf16_n16(p, state_only, s);
    case 32: return launch_prefill_bf16_n32(p, state_only, s);
    case 64: return launch_prefill_bf16_n64(p, state_only, s);
    case 128: return launch_prefill_bf16_n128(p, state_only, s);
  }
  return hipErrorInvalidValue;
}

namespace {
template <int N>
size_t lds_pc_n(int P, bool rope) {
  switch (P) {
    case 16: return rope ? pc::PcLayout<N, 16>::kBytesRope : pc::PcLayout<N, 16>::kBytesReal;
    case 32: return rope ? pc::PcLayout<N, 32>::kBytesRope : pc::PcLayout<N, 32>::kBytesReal;
    case 64: return rope ? pc::PcLayout<N, 64>::kBytesRope : pc::PcLayout<N, 64>::kBytesReal;
    case 128: return rope ? pc::PcLayout<N, 128>::kBytesRope : pc::PcLayout<N, 128>::kBytesReal;
  }
  return 0;
}
}  // namespace

size_t prefill_lds_bytes_bf16(int N, int P, bool rope) {
  switch (N) {
    case 16: return lds_pc_n<16>(P, rope);
    case 32: return lds_pc_n<32>(P, rope);
    case 64: return lds_pc_n<64>(P, rope);
    case 128: return lds_pc_n<128>(P, rope);
  }
  return 0;
}

}  // namespace m3
