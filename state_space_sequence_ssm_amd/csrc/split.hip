// Joining two consecutive segments of a sequence that were walked
// independently, the second from a zero start.
//
// The recurrence ("Znakomstvo s Mamba-3" (chernovdev.ru), sec. 1, displayed
// recurrence) is linear in the state, and the rotation of B by the cumulative
// angle (same page, sec. 2) composes: with Phi_b the angle at the end of the
// first segment, rotating by Phi_b + phi equals rotating by phi and then by
// Phi_b.  So the state after the second segment is
//   h_2 = exp(sum_{t in seg 2} Delta_t A_t) (h_1 + (1 - lambda_t1) Delta_t1 sum_r Btil_1[r] x_1[r]^T)
//         + Rot(Phi_b) h_rel,
// where h_1, Btil_1, x_1, Phi_b are the end state and carry of the first
// segment, t1 the second segment's first token (its beta term reaches back to
// the first segment's last token), h_rel the second segment's end state from
// a zero start with angles counted from zero, and Rot(Phi_b) rotates each pair
// of state rows (2j, 2j+1) the way B is rotated.  The second segment's
// rotated B carry is rotated by Phi_b the same way and its angle carry becomes
// Phi_b + phi_rel; its x carry needs no change.
#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {
namespace {

constexpr int kThreads = 256;

// grid (Bt*H, kParts): part y joins state rows [y N / kParts, (y+1) N / kParts);
// part 0 also handles the B and angle carries
constexpr int kParts = 8;

__global__ __launch_bounds__(kThreads) void split_combine_kernel(CombineParams c) {
  const int bh = blockIdx.x;
  const int part = blockIdx.y;
  const int b = bh / c.H, hh = bh % c.H;
  const int tid = threadIdx.x;
  const size_t units = static_cast<size_t>(c.Bt) * c.H;
  __shared__ float red[kThreads / 64];
  __shared__ float sPhi[64];
  // sum of Delta A over the second segment
  const bool sp = c.dt_softplus != 0;
  const float dtb = sp && c.dt_bias != nullptr ? c.dt_bias[hh] : 0.f;
  float sdt = 0.f;
  for (int t = c.t1 + tid; t < c.t2; t += kThreads) {
    const size_t o = (static_cast<size_t>(b) * c.Lfull + t) * c.H + hh;
    sdt += delta_of(c.dt[o], sp, dtb, true) * (c.A_tok != nullptr ? c.A_tok[o] : 1.f);
  }
  for (int o = 32; o > 0; o >>= 1) sdt += __shfl_xor(sdt, o);
  if ((tid & 63) == 0) red[tid >> 6] = sdt;
  const int J = c.N / 2;
  if (c.phi != nullptr)
    for (int j = tid; j < J; j += kThreads) sPhi[j] = c.phi[static_cast<size_t>(bh) * J + j];
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  const float decay = __expf(c.A_tok != nullptr ? tot : c.A[hh] * tot);
  const size_t o1 = (static_cast<size_t>(b) * c.Lfull + c.t1) * c.H + hh;
  const float coef = (1.f - c.lam[o1]) * delta_of(c.dt[o1], sp, dtb, true);

  float* h1 = c.h + static_cast<size_t>(bh) * c.N * c.P;
  const float* hrel = c.h + (units + bh) * c.N * c.P;
  const float* B1 = c.Bprev + static_cast<size_t>(bh) * c.R * c.N;
  const bf16_t* x1 = static_cast<const bf16_t*>(c.x0) + static_cast<size_t>(bh) * c.R * c.P;
  // state: element (n, p), rows handled in pairs so the rotation stays local
  const int j0 = part * J / kParts, j1 = (part + 1) * J / kParts;
  for (int e = j0 * c.P + tid; e < j1 * c.P; e += kThreads) {
    const int j = e / c.P, p = e % c.P;
    float cs = 1.f, sn = 0.f;
    if (c.phi != nullptr) sincosf(sPhi[j], &sn, &cs);
    float v[2];
    for (int q = 0; q < 2; ++q) {
      const int n = 2 * j + q;
      float u = 0.f;
      for (int r = 0; r < c.R; ++r) u += B1[r * c.N + n] * bf16_to_f32(x1[r * c.P + p].bits);
      v[q] = decay * (h1[static_cast<size_t>(n) * c.P + p] + coef * u);
    }
    const float r0 = hrel[static_cast<size_t>(2 * j) * c.P + p], r1 = hrel[static_cast<size_t>(2 * j + 1) * c.P + p];
    h1[static_cast<size_t>(2 * j) * c.P + p] = v[0] + cs * r0 + sn * r1;
    h1[static_cast<size_t>(2 * j + 1) * c.P + p] = v[1] + cs * r1 - sn * r0;
  }
  if (c.phi != nullptr && part == 0) {
    // second segment's B carry (relative frame) -> absolute; its angle carry
    float* B2 = c.Bprev + (units + bh) * c.R * c.N;
    for (int e = tid; e < c.R * J; e += kThreads) {
      const int r = e / J, j = e % J;
      float sn, cs;
      sincosf(sPhi[j], &sn, &cs);
      const float a0 = B2[r * c.N + 2 * j], a1 = B2[r * c.N + 2 * j + 1];
      B2[r * c.N + 2 * j] = cs * a0 + sn * a1;
      B2[r * c.N + 2 * j + 1] = cs * a1 - sn * a0;
    }
    float* phi2 = c.phi + (units + bh) * J;
    for (int j = tid; j < J; j += kThreads) phi2[j] = wrap_angle(sPhi[j] + phi2[j]);
  }
}

}  // namespace

hipError_t launch_split_combine(const CombineParams& c, hipStream_t s) {
  if (c.N / 2 > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_combine_kernel, dim3(c.Bt * c.H, kParts), dim3(kThreads), 0, s, c);
  return hipGetLastError();
}

}  // namespace m3
