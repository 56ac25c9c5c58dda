// Launch helpers of the producer/consumer prefill (one instantiation per
// N, P, log2 R, RoPE, state-only and prologue; N and the prologue flag are
// fixed per translation unit to parallelise the build).
#pragma once
#include "prefill_pc_impl.hpp"

namespace m3 {
namespace pc {

// one workgroup per (segment, batch, head)
template <int N, int P, int LGR, bool ROPE, bool SO, bool PRO>
hipError_t launch_k(const PrefillParams& p, hipStream_t s) {
  using Lt = PcLayout<N, P>;
  const size_t lds = Lt::bytes(ROPE, PRO && p.pro.bc_norm != 0);
  // cleared once per device for the most this kernel asks for
  constexpr size_t kAllow = Lt::bytes(ROPE, PRO);
  static std::atomic<uint64_t> cleared{0};  // devices this kernel is cleared on
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&prefill_pc_kernel<N, P, LGR, ROPE, SO, PRO>), kAllow,
                           cleared);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_pc_kernel<N, P, LGR, ROPE, SO, PRO>), dim3(p.Bt * p.H * p.nseg), dim3(kThreads), lds,
                     s, p);
  return hipGetLastError();
}

template <int N, int P, bool ROPE, bool SO, bool PRO>
hipError_t launch_r(const PrefillParams& p, hipStream_t s) {
  switch (p.log2R) {
    case 0: return launch_k<N, P, 0, ROPE, SO, PRO>(p, s);
    case 1: return launch_k<N, P, 1, ROPE, SO, PRO>(p, s);
    case 2: return launch_k<N, P, 2, ROPE, SO, PRO>(p, s);
    case 3: return launch_k<N, P, 3, ROPE, SO, PRO>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int N, int P, bool SO, bool PRO>
hipError_t launch_rr(const PrefillParams& p, hipStream_t s) {
  const bool rope = p.theta != nullptr || p.omega != nullptr;
  return rope ? launch_r<N, P, true, SO, PRO>(p, s) : launch_r<N, P, false, SO, PRO>(p, s);
}

template <int N, bool SO, bool PRO>
hipError_t launch_p(const PrefillParams& p, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_rr<N, 16, SO, PRO>(p, s);
    case 32: return launch_rr<N, 32, SO, PRO>(p, s);
    case 64: return launch_rr<N, 64, SO, PRO>(p, s);
    case 128: return launch_rr<N, 128, SO, PRO>(p, s);
  }
  return hipErrorInvalidValue;
}

// All instantiations of one N and one PRO (a translation unit each, so the
// build runs in parallel): PRO when the call uses the prologue.
template <int N, bool PRO>
hipError_t launch_n(const PrefillParams& p, bool state_only, hipStream_t s) {
  return state_only ? launch_p<N, true, PRO>(p, s) : launch_p<N, false, PRO>(p, s);
}

}  // namespace pc
}  // namespace m3
