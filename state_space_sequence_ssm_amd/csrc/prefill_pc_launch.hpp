// Launch helpers of the producer/consumer prefill (one instantiation per
// N, P and log2 R; N is fixed per translation unit to parallelise the build).
#pragma once
#include "prefill_pc_impl.hpp"

namespace m3 {
namespace pc {

// one workgroup per (segment, batch, head)
template <int N, int P, int LGR, bool ROPE, bool SO>
hipError_t launch(const PrefillParams& p, hipStream_t s) {
  using Lt = PcLayout<N, P>;
  const size_t lds = ROPE ? Lt::kBytesRope : Lt::kBytesReal;
  static std::atomic<uint64_t> cleared{0};  // devices this kernel is cleared on
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&prefill_pc_kernel<N, P, LGR, ROPE, SO>), lds, cleared);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_pc_kernel<N, P, LGR, ROPE, SO>), dim3(p.Bt * p.H * p.nseg), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

template <int N, int P, bool ROPE, bool SO>
hipError_t launch_r(const PrefillParams& p, hipStream_t s) {
  switch (p.log2R) {
    case 0: return launch<N, P, 0, ROPE, SO>(p, s);
    case 1: return launch<N, P, 1, ROPE, SO>(p, s);
    case 2: return launch<N, P, 2, ROPE, SO>(p, s);
    case 3: return launch<N, P, 3, ROPE, SO>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int N, int P, bool SO>
hipError_t launch_rr(const PrefillParams& p, hipStream_t s) {
  const bool rope = p.theta != nullptr || p.omega != nullptr;
  return rope ? launch_r<N, P, true, SO>(p, s) : launch_r<N, P, false, SO>(p, s);
}

template <int N, bool SO>
hipError_t launch_p(const PrefillParams& p, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_rr<N, 16, SO>(p, s);
    case 32: return launch_rr<N, 32, SO>(p, s);
    case 64: return launch_rr<N, 64, SO>(p, s);
    case 128: return launch_rr<N, 128, SO>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int N>
hipError_t launch_n(const PrefillParams& p, bool state_only, hipStream_t s) {
  return state_only ? launch_p<N, true>(p, s) : launch_p<N, false>(p, s);
}

}  // namespace pc
}  // namespace m3
