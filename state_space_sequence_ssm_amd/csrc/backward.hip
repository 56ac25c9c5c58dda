// Backward pass of the chunked prefill: the whole-sequence kernel (one
// workgroup per (batch, head)), the split's joining kernel, the dA reduction
// and the dispatch.  The kernel itself, and the split, are described in
// backward_impl.hpp.
#include "backward_impl.hpp"

namespace m3 {
namespace bw {

__global__ void reduce_dA_kernel(const float* part, float* dA, int Bt, int H) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float s = 0.f;
  for (int b = 0; b < Bt; ++b) s += part[static_cast<size_t>(b) * H + h];
  dA[h] = s;
}

// Joining the two segments of a split walk: token m = cm Q's Delta and
// lambda gradients are the sum of the two segments' parts, and every dtheta
// of segment 0 (and dphi0) adds segment 1's dtheta at token m.  Block x < Bt m
// handles the dtheta row (b, t), x = b m + t; block 0 also the per-unit values.
__global__ __launch_bounds__(256) void split_join_kernel(BackwardParams p) {
  const int J = p.N / 2;
  const int m = p.cm * (kRows >> p.log2R);
  const size_t units = static_cast<size_t>(p.Bt) * p.H;
  if (p.dtheta != nullptr) {
    const int b = static_cast<int>(blockIdx.x) / m, t = static_cast<int>(blockIdx.x) % m;
    float4* row = reinterpret_cast<float4*>(p.dtheta + (static_cast<size_t>(b) * p.L + t) * p.H * J);
    const float4* add = reinterpret_cast<const float4*>(p.sDth + static_cast<size_t>(b) * p.H * J);
    for (int e = threadIdx.x; e < p.H * J / 4; e += blockDim.x) {
      float4 v = row[e];
      const float4 a = add[e];  // the same (h, pair) order as the row
      v.x += a.x;
      v.y += a.y;
      v.z += a.z;
      v.w += a.w;
      row[e] = v;
    }
  }
  if (blockIdx.x == 0) {
    for (size_t u = threadIdx.x; u < units; u += blockDim.x) {
      const size_t b = u / p.H, h = u % p.H;
      const size_t o = (b * p.L + m) * p.H + h;
      p.ddt[o] = p.sTok[u * 2] + p.sTok[(units + u) * 2];
      p.dlam[o] = p.sTok[u * 2 + 1] + p.sTok[(units + u) * 2 + 1];
    }
    if (p.dtheta != nullptr && p.dphi0 != nullptr)
      for (size_t e = threadIdx.x; e < units * J; e += blockDim.x) p.dphi0[e] += p.sDth[e];
  }
}

}  // namespace bw

hipError_t launch_backward(const BackwardParams& p, hipStream_t s) {
  if (p.cm <= 0) return bw::launch_mode<0>(p, s);
  hipError_t e = launch_backward_pre(p, s);
  if (e != hipSuccess) return e;
  e = launch_backward_main(p, s);
  if (e != hipSuccess) return e;
  const int m = p.cm * (bw::kRows >> p.log2R);
  hipLaunchKernelGGL(bw::split_join_kernel, dim3(p.dtheta != nullptr ? p.Bt * m : 1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_backward_dA(const float* part, float* dA, int Bt, int H, hipStream_t s) {
  hipLaunchKernelGGL(bw::reduce_dA_kernel, dim3((H + 255) / 256), dim3(256), 0, s, part, dA, Bt, H);
  return hipGetLastError();
}

size_t backward_lds_bytes(int N, int P, bool rope) {
  switch (N) {
    case 16: return bw::lds_p<16>(P, rope);
    case 32: return bw::lds_p<32>(P, rope);
    case 64: return bw::lds_p<64>(P, rope);
    case 128: return bw::lds_p<128>(P, rope);
  }
  return 0;
}

}  // namespace m3
