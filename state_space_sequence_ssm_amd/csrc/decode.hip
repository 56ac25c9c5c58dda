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
// per token.  bf16 steps at N in {32, 64, 128}, P in {64, 128} run on the
// matrix cores (decode_mma.hip), whose rate holds up at rank 16; this kernel,
// on the vector ALUs, takes fp32 inputs and the other shapes.  One 256-thread
// workgroup owns one (batch, head) and streams its state with 16-byte
// coalesced accesses.  Small per-token vectors are staged in LDS.
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
  float* sScale = sCr + R * N;       // 1 / RMS of the B, C rows (prologue)  [2][R]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c4 = tid % QP;
  const bool rope = p.theta != nullptr || p.omega != nullptr;
  constexpr int KX = (RMAX * P + kDecThreads - 1) / kDecThreads;  // x elements per thread
  constexpr int KB = (RMAX * N + kDecThreads - 1) / kDecThreads;  // B, C elements per thread
  constexpr int kIters = (NQUAD + kDecThreads - 1) / kDecThreads;  // state quads per thread

  // Everything one unit (batch, head) reads, held in registers from issue to use.
  struct Unit {
    float rx[KX], rxp[KX], rb[KB], rc[KB], rbp[KB], rth, rph;
    f32x4 hv[kIters];
  };
  // The state and this token's inputs are touched once per step: they are
  // loaded (and the state stored) with the nontemporal hint, which keeps them
  // from displacing the carries in the caches (measured ~15% faster with
  // fresh per-step inputs).
  // Loads in the order they are consumed: the small per-token vectors first,
  // then the state.  Wait counters retire loads in issue order, so staging the
  // small vectors (and its barriers) overlaps the state fetch, and a later
  // unit's loads never hold up an earlier one.  Indices are clamped rather
  // than branched so the wait counts stay static.
  auto fetch = [&](int bh, Unit& U) __attribute__((always_inline)) {
    const size_t vecN = static_cast<size_t>(bh) * R * N;
    const size_t vecP = static_cast<size_t>(bh) * R * P;
#pragma unroll
    for (int i = 0; i < KX; ++i) {
      const int e = tid + i * kDecThreads;
      const int ec = e < R * P ? e : 0;
      U.rx[i] = load_scalar_nt(static_cast<const T*>(p.x) + vecP + ec);
      U.rxp[i] = load_scalar(static_cast<const T*>(p.xprev) + vecP + ec);
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int e = tid + i * kDecThreads;
      const int ec = e < R * N ? e : 0;
      U.rb[i] = load_scalar_nt(static_cast<const T*>(p.B) + vecN + ec);
      U.rc[i] = load_scalar_nt(static_cast<const T*>(p.C) + vecN + ec);
      U.rbp[i] = p.Bprev_rot[vecN + ec];
    }
    U.rth = 0.f;
    U.rph = 0.f;
    if (rope) {
      const int j = tid < N / 2 ? tid : 0;
      const float* src = p.omega != nullptr ? p.omega + static_cast<size_t>(bh / p.H) * (N / 2)
                                            : p.theta + static_cast<size_t>(bh) * (N / 2);
      U.rth = __builtin_nontemporal_load(src + j);
      U.rph = p.phi[static_cast<size_t>(bh) * (N / 2) + j];
    }
    const float* h = p.h + static_cast<size_t>(bh) * N * P;
#pragma unroll
    for (int k = 0; k < kIters; ++k) {
      const int q = tid + k * kDecThreads;
      U.hv[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(h + 4 * (q < NQUAD ? q : 0)));
    }
  };

  auto process = [&](int bh, Unit& U) __attribute__((always_inline)) {
    const int hh = bh % p.H;
    const size_t vecN = static_cast<size_t>(bh) * R * N;
    const size_t vecP = static_cast<size_t>(bh) * R * P;
    T* xprev = static_cast<T*>(p.xprev) + vecP;
    float* Bprev = p.Bprev_rot + vecN;
    float* h = p.h + static_cast<size_t>(bh) * N * P;
    // Delta: softplus of the raw value plus the head's bias with the prologue
    const bool proDt = p.pro.dt_softplus != 0;
    const float dt = delta_of(p.dt[bh], proDt, proDt && p.pro.dt_bias != nullptr ? p.pro.dt_bias[hh] : 0.f, true);
    const float lm = p.lam[bh];
    const bool proNorm = p.pro.bc_norm != 0;
    const bool proBC = proNorm || p.pro.B_bias != nullptr || p.pro.C_bias != nullptr;
    const float alpha = __expf(dt * (p.A_tok != nullptr ? p.A_tok[bh] : p.A[hh]));
    const float beta = (1.f - lm) * dt * alpha;
    const float gamma = lm * dt;

    // ---- angles: Phi <- wrap(Phi + theta); table of cos/sin per pair
    if (rope && tid < N / 2) {
      const float a = wrap_angle(U.rph + (p.omega != nullptr ? dt * U.rth : U.rth));
      sPhi[tid] = a;
      float sn, cs;
      sincosf(a, &sn, &cs);
      sCS[2 * tid] = cs;
      sCS[2 * tid + 1] = sn;
    }
    // ---- small vectors into LDS (everything is read before any carry is overwritten)
#pragma unroll
    for (int i = 0; i < KX; ++i) {
      const int e = tid + i * kDecThreads;
      if (e < R * P) {
        sX[e] = U.rx[i];
        sXp[e] = U.rxp[i];
      }
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int e = tid + i * kDecThreads;
      if (e < R * N) {
        sBp[e] = beta * U.rbp[i];
        sBr[e] = U.rb[i];
        sCr[e] = U.rc[i];
      }
    }
    __syncthreads();
    // prologue: 1 / RMS of each rank's row of B (i < R) and C (i >= R), one
    // row per wave at a time, lanes striding over N (a row of zeros stays zero)
    if (proNorm) {
      for (int i = wave; i < 2 * R; i += kDecThreads / 64) {
        const float* row = (i < R ? sBr : sCr) + (i % R) * N;
        float ss = 0.f;
        for (int n = lane; n < N; n += 64) ss += row[n] * row[n];
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
        if (lane == 0) sScale[i] = ss > 0.f ? rsqrtf(ss * (1.f / N) + p.pro.eps) : 0.f;
      }
      __syncthreads();
    }
    // rotate B_t, C_t pairwise; write carry-out Btil_t, x_t, Phi
    for (int e = tid; e < R * (N / 2); e += kDecThreads) {
      const int r = e / (N / 2);
      const int j = e % (N / 2);
      float b0 = sBr[r * N + 2 * j], b1 = sBr[r * N + 2 * j + 1];
      float c0 = sCr[r * N + 2 * j], c1 = sCr[r * N + 2 * j + 1];
      if (proBC) {  // normalised (gain, 1 / RMS) and biased as in the prefill
        const size_t ob = (static_cast<size_t>(hh) * R + r) * N + 2 * j;
        if (proNorm) {
          const float sb = sScale[r], scl = sScale[R + r];
          b0 *= sb * (p.pro.B_w != nullptr ? p.pro.B_w[2 * j] : 1.f);
          b1 *= sb * (p.pro.B_w != nullptr ? p.pro.B_w[2 * j + 1] : 1.f);
          c0 *= scl * (p.pro.C_w != nullptr ? p.pro.C_w[2 * j] : 1.f);
          c1 *= scl * (p.pro.C_w != nullptr ? p.pro.C_w[2 * j + 1] : 1.f);
        }
        if (p.pro.B_bias != nullptr) {
          b0 += p.pro.B_bias[ob];
          b1 += p.pro.B_bias[ob + 1];
        }
        if (p.pro.C_bias != nullptr) {
          c0 += p.pro.C_bias[ob];
          c1 += p.pro.C_bias[ob + 1];
        }
      }
      if (rope) {
        const float c = sCS[2 * j], sn = sCS[2 * j + 1];
        const float rb0 = c * b0 + sn * b1, rb1 = -sn * b0 + c * b1;
        const float rc0 = c * c0 + sn * c1, rc1 = -sn * c0 + c * c1;
        b0 = rb0; b1 = rb1; c0 = rc0; c1 = rc1;
      }
      Bprev[r * N + 2 * j] = b0;
      Bprev[r * N + 2 * j + 1] = b1;
      sBc[r * N + 2 * j] = gamma * b0;
      sBc[r * N + 2 * j + 1] = gamma * b1;
      sC[r * N + 2 * j] = c0;
      sC[r * N + 2 * j + 1] = c1;
    }
#pragma unroll
    for (int i = 0; i < KX; ++i) {
      const int e = tid + i * kDecThreads;
      if (e < R * P) store_scalar(xprev + e, U.rx[i]);
    }
    if (rope && tid < N / 2) p.phi[static_cast<size_t>(bh) * (N / 2) + tid] = sPhi[tid];
    __syncthreads();

    // ---- state update, 16-byte coalesced: thread owns quad column c4, rows n
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
        f32x4 v = U.hv[k] * alpha;
        for (int r = 0; r < R; ++r) {
          const float bp = sBp[r * N + n], bc = sBc[r * N + n];
          const f32x4 xp4 = *reinterpret_cast<const f32x4*>(&sXp[r * P + 4 * c4]);
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sX[r * P + 4 * c4]);
          v += bp * xp4 + bc * x4;
        }
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(h + 4 * q));
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
    // the next process() writes sRed only after two barriers, and the staged
    // vectors read above before this barrier
  };

  Unit U;
  fetch(blockIdx.x, U);
  process(blockIdx.x, U);
}

template <typename T, int N, int P>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  const size_t lds = sizeof(float) * (5 * p.R * N + 6 * p.R * P + N + N / 2 + 2 * p.R);
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

// bf16 steps of the supported shapes run on the matrix cores at every rank
// (measured at N = P = 64: R = 4 50.2 vs 51.1 us, R = 16 70.7 vs 180 us per
// step at B = 256, H = 32).
hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (decode_mma_supported(p)) return launch_decode_mma(p, s);
  return p.bf16 ? launch_decode_dt<bf16_t>(p, s) : launch_decode_dt<float>(p, s);
}

}  // namespace m3
