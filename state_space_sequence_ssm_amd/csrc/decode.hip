// Single-token MIMO decode step of the Mamba-3 SSM core (gfx950).
//
// Operation ("Znakomstvo s Mamba-3" (chernovdev.ru), sec. 1 displayed
// recurrence, sec. 2 cumulative RoPE on B and C, sec. 3 MIMO; "La dualita:
// Mamba-2 e Mamba-3" (book.paithon.it), sec. "Mamba-3": MIMO adds work per
// byte on an unchanged state):
//   Phi <- Phi + theta_t;  Btil_t = R(Phi)^T B_t;  Ctil_t = R(Phi)^T C_t
//   h   <- alpha h + beta sum_r Btil_prev[r] xprev[r]^T + gamma sum_r Btil_t[r] x_t[r]^T
//   y_t[r] = h^T Ctil_t[r];   carry <- (Btil_t, x_t, Phi)
//
// The step is HBM-bound: the fp32 N x P state is read once and written once
// per token (2.7 flop/byte at N = P = 64, R = 4), so it runs on the vector
// ALUs; one 256-thread workgroup owns one (batch, head) and streams its state
// with 16-byte coalesced accesses.  Small per-token vectors are staged in LDS.
#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {

constexpr int kDecThreads = 256;

// RMAX bounds the rank held in registers (R <= RMAX); two variants keep the
// common small-rank case at low register pressure.
template <typename T, int N, int P, int RMAX>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(DecodeParams p) {
  constexpr int kDecMaxR = RMAX;
  constexpr int QP = P / 4;                  // float4 quads per state row
  constexpr int NQUAD = N * P / 4;           // quads in the state
  static_assert(kDecThreads % QP == 0, "quad column must be fixed per thread");
  // LDS carve-up (sizes depend on the runtime rank R)
  extern __shared__ float smem[];
  const int R = p.R;
  float* sBc = smem;                 // gamma * Btil_t        [R][N]
  float* sBp = sBc + R * N;          // beta  * Btil_prev     [R][N]
  float* sC = sBp + R * N;           // Ctil_t                [R][N]
  float* sX = sC + R * N;            // x_t                   [R][P]
  float* sXp = sX + R * P;           // x_prev                [R][P]
  float* sRed = sXp + R * P;         // per-wave y partials   [4][R][P]
  float* sCS = sRed + 4 * R * P;     // cos/sin of new angle  [N]
  float* sPhi = sCS + N;             // new angle (wrapped)   [N/2]
  float* sBr = sPhi + N / 2;         // raw B_t               [R][N]
  float* sCr = sBr + R * N;          // raw C_t               [R][N]

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int hh = bh % p.H;
  const size_t vecN = static_cast<size_t>(bh) * R * N;
  const size_t vecP = static_cast<size_t>(bh) * R * P;
  const T* x = static_cast<const T*>(p.x) + vecP;
  const T* Bin = static_cast<const T*>(p.B) + vecN;
  const T* Cin = static_cast<const T*>(p.C) + vecN;
  T* xprev = static_cast<T*>(p.xprev) + vecP;
  float* Bprev = p.Bprev_rot + vecN;
  float* h = p.h + static_cast<size_t>(bh) * N * P;

  // issue the state loads first so their latency overlaps the staging below
  constexpr int kIters = (NQUAD + kDecThreads - 1) / kDecThreads;
  f32x4 hv[kIters];
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int q = tid + k * kDecThreads;
    if (q < NQUAD) hv[k] = *reinterpret_cast<const f32x4*>(h + 4 * q);
  }

  const float dt = p.dt[bh];
  const float lm = p.lam[bh];
  const float alpha = __expf(dt * p.A[hh]);
  const float beta = (1.f - lm) * dt * alpha;
  const float gamma = lm * dt;

  // ---- angles: Phi <- wrap(Phi + theta); table of cos/sin per pair
  if (p.theta != nullptr) {
    for (int j = tid; j < N / 2; j += kDecThreads) {
      float* phi = p.phi + static_cast<size_t>(bh) * (N / 2);
      float a = wrap_angle(phi[j] + p.theta[static_cast<size_t>(bh) * (N / 2) + j]);
      sPhi[j] = a;
      float s, c;
      sincosf(a, &s, &c);
      sCS[2 * j] = c;
      sCS[2 * j + 1] = s;
    }
  }
  // ---- small vectors into LDS (read everything before any carry is overwritten)
  for (int e = tid; e < R * P; e += kDecThreads) {
    sX[e] = load_scalar(x + e);
    sXp[e] = load_scalar(xprev + e);
  }
  for (int e = tid; e < R * N; e += kDecThreads) {
    sBp[e] = beta * Bprev[e];
    sBr[e] = load_scalar(Bin + e);
    sCr[e] = load_scalar(Cin + e);
  }
  __syncthreads();
  // rotate B_t, C_t pairwise; write carry-out Btil_t, x_t, Phi
  for (int e = tid; e < R * (N / 2); e += kDecThreads) {
    const int r = e / (N / 2);
    const int j = e % (N / 2);
    float b0 = sBr[r * N + 2 * j], b1 = sBr[r * N + 2 * j + 1];
    float c0 = sCr[r * N + 2 * j], c1 = sCr[r * N + 2 * j + 1];
    if (p.theta != nullptr) {
      const float c = sCS[2 * j], s = sCS[2 * j + 1];
      const float rb0 = c * b0 + s * b1, rb1 = -s * b0 + c * b1;
      const float rc0 = c * c0 + s * c1, rc1 = -s * c0 + c * c1;
      b0 = rb0; b1 = rb1; c0 = rc0; c1 = rc1;
    }
    Bprev[r * N + 2 * j] = b0;
    Bprev[r * N + 2 * j + 1] = b1;
    sBc[r * N + 2 * j] = gamma * b0;
    sBc[r * N + 2 * j + 1] = gamma * b1;
    sC[r * N + 2 * j] = c0;
    sC[r * N + 2 * j + 1] = c1;
  }
  for (int e = tid; e < R * P; e += kDecThreads) store_scalar(xprev + e, sX[e]);
  if (p.theta != nullptr) {
    for (int j = tid; j < N / 2; j += kDecThreads) {
      p.phi[static_cast<size_t>(bh) * (N / 2) + j] = sPhi[j];
    }
  }
  __syncthreads();

  // ---- state update, 16-byte coalesced: thread owns quad column c4, rows n
  const int c4 = tid % QP;
  float yacc[kDecMaxR][4];
#pragma unroll
  for (int r = 0; r < kDecMaxR; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) yacc[r][i] = 0.f;

#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int q = tid + k * kDecThreads;
    if (q < NQUAD) {
      const int n = q / QP;
      f32x4 v = hv[k] * alpha;
      for (int r = 0; r < R; ++r) {
        const float bp = sBp[r * N + n], bc = sBc[r * N + n];
        const f32x4 xp4 = *reinterpret_cast<const f32x4*>(&sXp[r * P + 4 * c4]);
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sX[r * P + 4 * c4]);
        v += bp * xp4 + bc * x4;
      }
      *reinterpret_cast<f32x4*>(h + 4 * q) = v;
#pragma unroll
      for (int r = 0; r < kDecMaxR; ++r) {
        if (r < R) {
          const float c = sC[r * N + n];
#pragma unroll
          for (int i = 0; i < 4; ++i) yacc[r][i] += c * v[i];
        }
      }
    }
  }
  // ---- y = h^T Ctil: reduce over the rows held by lanes sharing column c4
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int r = 0; r < kDecMaxR; ++r) {
    if (r < R) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = yacc[r][i];
        for (int off = QP; off < 64; off <<= 1) v += __shfl_xor(v, off);
        if (lane < QP) sRed[(wave * R + r) * P + 4 * lane + i] = v;
      }
    }
  }
  __syncthreads();
  T* y = static_cast<T*>(p.y) + vecP;
  for (int e = tid; e < R * P; e += kDecThreads) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) s += sRed[w * R * P + e];
    store_scalar(y + e, s);
  }
}

template <typename T, int N, int P>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  const size_t lds = sizeof(float) * (5 * p.R * N + 6 * p.R * P + N + N / 2);
  if (p.R <= 4)
    hipLaunchKernelGGL((decode_step_kernel<T, N, P, 4>), dim3(p.Bt * p.H), dim3(kDecThreads), lds, s, p);
  else
    hipLaunchKernelGGL((decode_step_kernel<T, N, P, 16>), dim3(p.Bt * p.H), dim3(kDecThreads), lds, s, p);
  return hipGetLastError();
}

template <typename T, int N>
static hipError_t launch_decode_n(const DecodeParams& p, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_decode_t<T, N, 16>(p, s);
    case 32: return launch_decode_t<T, N, 32>(p, s);
    case 64: return launch_decode_t<T, N, 64>(p, s);
    case 128: return launch_decode_t<T, N, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeParams& p, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_decode_n<T, 16>(p, s);
    case 32: return launch_decode_n<T, 32>(p, s);
    case 64: return launch_decode_n<T, 64>(p, s);
    case 128: return launch_decode_n<T, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  return p.bf16 ? launch_decode_dt<bf16_t>(p, s) : launch_decode_dt<float>(p, s);
}

}  // namespace m3
