// bf16 prefill dispatch: the producer/consumer fused kernel (prefill_pc_impl.hpp),
// instantiated per N (and with / without the prologue) in prefill_bf16_n*.hip.
#include "prefill_pc_impl.hpp"

namespace m3 {

hipError_t launch_prefill_bf16_n16(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n32(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n64(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n128(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n16_pro(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n32_pro(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n64_pro(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_bf16_n128_pro(const PrefillParams& p, bool state_only, hipStream_t s);

hipError_t launch_prefill_bf16(const PrefillParams& p, bool state_only, hipStream_t s) {
  // calls that use the prologue run kernels compiled with it; the rest the plain core
  const bool pro = p.pro.bc_norm != 0 || p.pro.dt_softplus != 0 || p.pro.B_bias != nullptr ||
                   p.pro.C_bias != nullptr;
  switch (p.N) {
    case 16: return pro ? launch_prefill_bf16_n16_pro(p, state_only, s) : launch_prefill_bf16_n16(p, state_only, s);
    case 32: return pro ? launch_prefill_bf16_n32_pro(p, state_only, s) : launch_prefill_bf16_n32(p, state_only, s);
    case 64: return pro ? launch_prefill_bf16_n64_pro(p, state_only, s) : launch_prefill_bf16_n64(p, state_only, s);
    case 128:
      return pro ? launch_prefill_bf16_n128_pro(p, state_only, s) : launch_prefill_bf16_n128(p, state_only, s);
  }
  return hipErrorInvalidValue;
}

namespace {
template <int N>
size_t lds_pc_n(int P, int R, bool rope, bool pro) {
  (void)R;
  switch (P) {
    case 16: return pc::PcLayout<N, 16>::bytes(rope, pro);
    case 32: return pc::PcLayout<N, 32>::bytes(rope, pro);
    case 64: return pc::PcLayout<N, 64>::bytes(rope, pro);
    case 128: return pc::PcLayout<N, 128>::bytes(rope, pro);
  }
  return 0;
}
}  // namespace

size_t prefill_lds_bytes_bf16(int N, int P, int R, bool rope, bool pro_bc) {
  switch (N) {
    case 16: return lds_pc_n<16>(P, R, rope, pro_bc);
    case 32: return lds_pc_n<32>(P, R, rope, pro_bc);
    case 64: return lds_pc_n<64>(P, R, rope, pro_bc);
    case 128: return lds_pc_n<128>(P, R, rope, pro_bc);
  }
  return 0;
}

}  // namespace m3
