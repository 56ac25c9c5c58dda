// Cumulative rotation angles of the Mamba-3 RoPE trick (gfx950).
//
// "Znakomstvo s Mamba-3" (chernovdev.ru), sec. 2: the complex SSM is a real
// SSM whose B and C are rotated by data-dependent angles aggregated over all
// time steps, i.e. an inclusive prefix sum along the sequence:
//   phi[b, t, h, j] = phi0[b, h, j] + sum_{s <= t} theta[b, s, h, j].
//
// Memory-bound (4 B in, 4 B out per element).  For a fixed batch index the
// (h, j) columns of one token are contiguous, so a workgroup owns 32 columns
// (one 128-byte line per token) and walks the sequence in 256-token segments:
// each thread scans 8 consecutive tokens of one float4 column quad in
// registers, lanes combine their segment totals with a strided wave scan,
// waves combine through LDS, and a per-column carry crosses segments.  The
// next segment's loads are issued before the current one is scanned.
#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {

constexpr int kAngThreads = 256;
constexpr int kAngQuads = 8;                       // float4 columns per block (32 floats)
constexpr int kAngRowGroups = kAngThreads / kAngQuads;  // 32
constexpr int kAngRowsPer = 8;                     // tokens per thread per segment
constexpr int kAngSeg = kAngRowGroups * kAngRowsPer;    // 256 tokens

__global__ __launch_bounds__(kAngThreads) void angles_cumsum_kernel(AnglesParams p) {
  __shared__ f32x4 sTot[4][kAngQuads];
  const int HJ = p.H * p.J;
  const int HJ4 = HJ / 4;
  const int tilesPerB = (HJ4 + kAngQuads - 1) / kAngQuads;
  const int b = blockIdx.x / tilesPerB;
  const int tile = blockIdx.x % tilesPerB;
  const int tid = threadIdx.x;
  const int quad = tid % kAngQuads;
  const int rg = tid / kAngQuads;  // row group 0..31
  const int lane = tid & 63, wave = tid >> 6;
  const int q = tile * kAngQuads + quad;
  const bool colOk = q < HJ4;
  const size_t rowStride = static_cast<size_t>(HJ);
  const f32x4* th = reinterpret_cast<const f32x4*>(p.theta + static_cast<size_t>(b) * p.L * HJ) + q;
  f32x4* ph = reinterpret_cast<f32x4*>(p.phi + static_cast<size_t>(b) * p.L * HJ) + q;
  const size_t rs4 = rowStride / 4;

  f32x4 carry = {0.f, 0.f, 0.f, 0.f};
  if (p.phi0 != nullptr && colOk)
    carry = reinterpret_cast<const f32x4*>(p.phi0 + static_cast<size_t>(b) * HJ)[q];

  f32x4 cur[kAngRowsPer], nxt[kAngRowsPer];
  auto load_seg = [&](int seg, f32x4* dst) {
#pragma unroll
    for (int i = 0; i < kAngRowsPer; ++i) {
      const int t = seg * kAngSeg + rg * kAngRowsPer + i;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (colOk && t < p.L) v = th[static_cast<size_t>(t) * rs4];
      dst[i] = v;
    }
  };
  const int nseg = (p.L + kAngSeg - 1) / kAngSeg;
  load_seg(0, cur);
  for (int seg = 0; seg < nseg; ++seg) {
    if (seg + 1 < nseg) load_seg(seg + 1, nxt);
    // scan the thread's 8 rows
#pragma unroll
    for (int i = 1; i < kAngRowsPer; ++i) cur[i] += cur[i - 1];
    // exclusive scan of row-group totals within the wave (lanes 8 apart share a quad)
    f32x4 tot = cur[kAngRowsPer - 1];
    f32x4 inc = tot;
#pragma unroll
    for (int d = kAngQuads; d < 64; d <<= 1) {
      f32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = __shfl_up(inc[c], d, 64);
      if (lane >= d) inc += o;
    }
    if (lane >= 64 - kAngQuads) sTot[wave][quad] = inc;  // wave total per quad
    __syncthreads();
    f32x4 off = carry + (inc - tot);
    f32x4 segTot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 wt = sTot[w][quad];
      if (w < wave) off += wt;
      segTot += wt;
    }
#pragma unroll
    for (int i = 0; i < kAngRowsPer; ++i) {
      const int t = seg * kAngSeg + rg * kAngRowsPer + i;
      if (colOk && t < p.L) ph[static_cast<size_t>(t) * rs4] = cur[i] + off;
    }
    carry += segTot;
    __syncthreads();
    if (seg + 1 < nseg) {
#pragma unroll
      for (int i = 0; i < kAngRowsPer; ++i) cur[i] = nxt[i];
    }
  }
}

hipError_t launch_angles(const AnglesParams& p, hipStream_t s) {
  const int HJ4 = p.H * p.J / 4;
  const int tilesPerB = (HJ4 + kAngQuads - 1) / kAngQuads;
  hipLaunchKernelGGL(angles_cumsum_kernel, dim3(p.Bt * tilesPerB), dim3(kAngThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace m3
