// Fused chunked prefill of the Mamba-3 SSM core on gfx950 (CDNA4), fp32
// inputs (x, B, C and y in float32; the bf16 path is prefill_pc_impl.hpp).
//
// Operation: the exponential-trapezoidal recurrence ("Znakomstvo s Mamba-3"
// (chernovdev.ru), sec. 1, displayed recurrence) with cumulative RoPE on B
// and C (same page, sec. 2) and rank-R MIMO (same page, sec. 3; "La dualita:
// Mamba-2 e Mamba-3" (book.paithon.it), sec. "Mamba-3"), evaluated chunk by
// chunk as the four pieces of the chunked scan ("La dualita", sec. "Perche
// conviene: i tensor core"): intra-chunk masked product, chunk state,
// inter-chunk recurrence, readout of the previous state.
//
// Chunk algebra used here (derived by unrolling the recurrence).  A chunk holds
// Q tokens s..e; Lam_t = sum_{k=s..t} Delta_k A (chunk-local), gamma_t =
// lambda_t Delta_t, delta_t = gamma_t + (1 - lambda_{t+1}) Delta_{t+1}
// (Delta_{L} := 0 at the sequence end).  With the shifted state
// H' = h_e + (1 - lambda_{e+1}) Delta_{e+1} u_e (u_t = sum_r Btil x^T):
//   y_t     = sum_{j<=t} M_tj <Ctil_t, Btil_j> x_j + exp(Lam_t) Ctil_t^T H'_{prev}
//   M_tj    = exp(Lam_t - Lam_j) delta_j (j < t),  M_tt = gamma_t
//   H'_new  = exp(Lam_e) H'_{prev} + sum_j exp(Lam_e - Lam_j) delta_j Btil_j x_j^T
//   H'_{-1} = h0 + (1 - lambda_0) Delta_0 Btil_{-1} x_{-1}^T;  h_final = H' at the end.
//
// MI355X design: one 512-thread workgroup (8 wave64) owns one (batch, head)
// and walks its chunks in order with the N x P state resident in MFMA
// accumulators (fp32); nothing per chunk is written to HBM except y.  A chunk
// tile holds 64 (token, rank) rows; a chunk is Q = 64 / R tokens, or fewer
// when the caller asks (a power of two): the tile's rows past Q R are then
// empty (zero operands, zero weights, never stored).  Per chunk:
//   * the next chunk's x, B, C, theta, Delta, lambda are loaded into registers
//     while the current chunk computes (software prefetch);
//   * the Delta/lambda scan is one wave64 inclusive scan; the angle scan is a
//     segmented wave scan per rotation pair with a carry across chunks;
//   * B and C are rotated in registers and staged in fp32 LDS tiles: C and B
//     row-major, (w_j B_j)^T and X^T transposed, padded rows;
//   * G^T = B C^T on the 16x16x4 fp32 MFMA, masked in registers, each of its
//     four rows fed back as a k step of Y^T += X^T S^T (no LDS trip);
//     Y^T += diag(exp Lam) H'^T C^T; H' = exp(Lam_e) H' + (wB)^T X.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {

constexpr int kRows = 64;         // (token, rank) rows per chunk tile
constexpr int kThreads = 512;     // 8 waves
constexpr int kWaves = kThreads / 64;

// 16x16x4 fp32 MFMA: operand k index 4 kb + g of row `row`.
struct MmaF32 {
  using E = float;
  using Frag = float;
  static constexpr int K = 4;
  __device__ static __forceinline__ Frag ld(const E* row, int kb, int g) { return row[kb * 4 + g]; }
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Write 4 fp32 values as one 16-byte LDS store.
__device__ __forceinline__ void lds_put4(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T, int N, int P>
struct Layout {
  static_assert(std::is_same<T, float>::value, "fp32 inputs only");
  using E = MmaF32::E;
  static constexpr int EB = sizeof(E);
  static constexpr int VE = 16 / sizeof(T);   // input elements per 16-byte load
  static constexpr int NK = N < MmaF32::K ? MmaF32::K : N;  // contraction length over n (zero padded)
  static constexpr int PN = NK + 16 / EB;     // pitch of rows of length N (padded to NK)
  static constexpr int PR = kRows + 16 / EB;  // pitch of rows of length kRows
  static constexpr int NPT = P / 16;          // p tiles
  static constexpr int NNT = N / 16;          // n tiles
  static constexpr int NHT = NNT * NPT;       // state tiles
  static constexpr int HT = (NHT + kWaves - 1) / kWaves;  // state tiles per wave
  static constexpr int YT = (NPT + 1) / 2;    // y p-tiles per wave
  // staging jobs: 4 rows x VE elements of B, C or X
  static constexpr int JB = (kRows / 4) * (N / VE);
  static constexpr int JX = (kRows / 4) * (P / VE);
  static constexpr int JOBS = 2 * JB + JX;
  static constexpr int JS = (JOBS + kThreads - 1) / kThreads;
  // theta staging: 64 tokens x N/2 angles as float4
  static constexpr int TJ = kRows * (N / 2) / 4;
  static constexpr int TS = (TJ + kThreads - 1) / kThreads;
  // LDS byte offsets
  static constexpr size_t oC = 0;
  static constexpr size_t oB = oC + size_t(kRows) * PN * EB;
  static constexpr size_t oBwT = oB + size_t(kRows) * PN * EB;
  static constexpr size_t oXT = oBwT + size_t(N) * PR * EB;
  static constexpr size_t oHT = oXT + size_t(P) * PR * EB;
  static constexpr size_t oScal = oHT + size_t(P) * PN * EB;
  static constexpr int kScal = 6 * kRows + 4;  // Lam, gamma, delta, w, dec, Delta; chunk decay
  static constexpr size_t oPhiC = oScal + sizeof(float) * kScal;
  static constexpr size_t oTheta = oPhiC + sizeof(float) * (N / 2);
  static constexpr size_t oCS = oTheta + sizeof(float) * kRows * (N / 2);
  static constexpr size_t kBytesReal = oPhiC + sizeof(float) * (N / 2);
  static constexpr size_t kBytesRope = oCS + sizeof(float) * 2 * kRows * (N / 2);
};

template <typename T, int N, int P>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  using Lt = Layout<T, N, P>;
  using M = MmaF32;
  using E = typename Lt::E;
  constexpr int VE = Lt::VE, PN = Lt::PN, PR = Lt::PR, NPT = Lt::NPT, NK = Lt::NK;
  constexpr int K = M::K;

  extern __shared__ __align__(16) unsigned char smem[];
  E* sC = reinterpret_cast<E*>(smem + Lt::oC);
  E* sB = reinterpret_cast<E*>(smem + Lt::oB);
  E* sBwT = reinterpret_cast<E*>(smem + Lt::oBwT);
  E* sXT = reinterpret_cast<E*>(smem + Lt::oXT);
  E* sHT = reinterpret_cast<E*>(smem + Lt::oHT);
  float* sLam = reinterpret_cast<float*>(smem + Lt::oScal);
  float* sGam = sLam + kRows;
  float* sDel = sGam + kRows;
  float* sW = sDel + kRows;
  float* sDec = sW + kRows;
  float* sDt = sDec + kRows;  // Delta, for angles given as rates
  float* sChunkDec = sDt + kRows;
  float* sPhiC = reinterpret_cast<float*>(smem + Lt::oPhiC);
  float* sTheta = reinterpret_cast<float*>(smem + Lt::oTheta);
  float* sCS = reinterpret_cast<float*>(smem + Lt::oCS);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int hh = bh % p.H;
  const int L = p.L, H = p.H, R = p.R, lgR = p.log2R;
  const int Q = p.chunk > 0 ? p.chunk : (kRows >> lgR);  // tokens per chunk (Q R <= 64)
  const bool om = p.omega != nullptr;  // angles as rates: theta = Delta * omega
  const bool rope = p.theta != nullptr || om;
  const float Ah = p.A_tok != nullptr ? 0.f : p.A[hh];
  const int nch = (L + Q - 1) / Q;
  // steps fused in front of the core (normalisation and biases of B and C
  // while staging, Delta = softplus(raw + bias) in the decay scan)
  const bool proNorm = p.pro.bc_norm != 0;
  const bool proBC = proNorm || p.pro.B_bias != nullptr || p.pro.C_bias != nullptr;
  const bool proDt = p.pro.dt_softplus != 0;
  const float dtBias = proDt && p.pro.dt_bias != nullptr ? p.pro.dt_bias[hh] : 0.f;

  const T* xg = static_cast<const T*>(p.x);
  const T* Bg = static_cast<const T*>(p.B);
  const T* Cg = static_cast<const T*>(p.C);
  // element offset of (b, t, h, rank 0) rows: token-major [Bt, L, H, R, .]
  // or head-major [Bt, H, L, R, .]
  const bool hm = p.headMajor != 0;
  auto rowbase = [&](int t) -> size_t {
    const size_t row = hm ? (static_cast<size_t>(b) * H + hh) * L + t : (static_cast<size_t>(b) * L + t) * H + hh;
    return row * static_cast<size_t>(R);
  };

  // ------------------------------------------------------------ prefetch state
  u32x4 raw[Lt::JS][4];
  f32x4 rawTh[Lt::TS];
  float rdt = 0.f, rlam = 0.f, rdtn = 0.f, rlamn = 0.f, rA = 0.f;
  bool vdt = false, vdtn = false;  // the token (and the next one) exist

  auto issue_loads = [&](int c) {
    const int s0 = c * Q;
#pragma unroll
    for (int s = 0; s < Lt::JS; ++s) {
      const int j = tid + s * kThreads;
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[s][k] = u32x4{0u, 0u, 0u, 0u};
      if (j < Lt::JOBS) {
        const T* base;
        int D, idx;
        if (j < Lt::JB) { base = Bg; D = N; idx = j; }
        else if (j < 2 * Lt::JB) { base = Cg; D = N; idx = j - Lt::JB; }
        else { base = xg; D = P; idx = j - 2 * Lt::JB; }
        const int cpr = D / VE;
        const int rb = idx / cpr, cb = idx % cpr;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = 4 * rb + k;
          const int t = s0 + (i >> lgR);
          u32x4 v = {0u, 0u, 0u, 0u};
          if ((i >> lgR) < Q && t < L) {
            const T* src = base + (rowbase(t) + (i & (R - 1))) * D + cb * VE;
            v = *reinterpret_cast<const u32x4*>(src);
          }
          raw[s][k] = v;
        }
      }
    }
    if (rope) {
#pragma unroll
      for (int s = 0; s < Lt::TS; ++s) {
        const int j = tid + s * kThreads;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (j < Lt::TJ) {
          const int tl = j / (N / 8), q4 = j % (N / 8);
          const int t = s0 + tl;
          if (tl < Q && t < L)
            v = om ? *reinterpret_cast<const f32x4*>(p.omega + (static_cast<size_t>(b) * L + t) * (N / 2) + 4 * q4)
                   : *reinterpret_cast<const f32x4*>(p.theta + (static_cast<size_t>(b) * L + t) * H * (N / 2) +
                                                     static_cast<size_t>(hh) * (N / 2) + 4 * q4);
        }
        rawTh[s] = v;
      }
    }
    if (wave == 0) {
      const int t = s0 + lane;
      rdt = rlam = rdtn = rlamn = 0.f;
      rA = Ah;
      vdt = lane < Q && t < L;
      vdtn = lane < Q && t + 1 < L;
      if (lane < Q && t < L) {
        const size_t o = (static_cast<size_t>(b) * L + t) * H + hh;
        rdt = p.dt[o];
        rlam = p.lam[o];
        if (p.A_tok != nullptr) rA = p.A_tok[o];
        if (t + 1 < L) {
          rdtn = p.dt[o + H];
          rlamn = p.lam[o + H];
        }
      }
    }
  };

  // stage A: per-token scalars (wave 0) and raw angles into LDS
  auto stage_scalars = [&]() {
    if (wave == 0) {
      const float d = delta_of(rdt, proDt, dtBias, vdt), dn = delta_of(rdtn, proDt, dtBias, vdtn);
      const float v = d * rA;
      const float lamc = wave_inclusive_scan(v, 64);
      const float lamEnd = __shfl(lamc, Q - 1, 64);
      const float gam = rlam * d;
      const float del = gam + (1.f - rlamn) * dn;
      // every lane: past the chunk's Q tokens Delta is 0, so the weights are 0
      // and the decays finite (read for the tile's empty rows)
      sLam[lane] = lamc;
      sGam[lane] = gam;
      sDel[lane] = del;
      sW[lane] = __expf(lamEnd - lamc) * del;
      sDec[lane] = __expf(lamc);
      sDt[lane] = d;
      if (lane == 0) sChunkDec[0] = __expf(lamEnd);
    }
    if (rope) {
#pragma unroll
      for (int s = 0; s < Lt::TS; ++s) {
        const int j = tid + s * kThreads;
        if (j < Lt::TJ) {
          const int tl = j / (N / 8), q4 = j % (N / 8);
          *reinterpret_cast<f32x4*>(sTheta + tl * (N / 2) + 4 * q4) = rawTh[s];
        }
      }
    }
  };

  // cumulative angles of the chunk + cos/sin table; carry Phi across chunks
  auto stage_angles = [&]() {
    const int total = Q * (N / 2);
    for (int e = tid; e < total; e += kThreads) {
      const int jp = e / Q, tl = e % Q;
      float v = wave_inclusive_scan(sTheta[tl * (N / 2) + jp] * (om ? sDt[tl] : 1.f), Q);
      v += sPhiC[jp];
      float sn, cs;
      sincosf(v, &sn, &cs);
      sCS[2 * (tl * (N / 2) + jp)] = cs;
      sCS[2 * (tl * (N / 2) + jp) + 1] = sn;
      if (tl == Q - 1) sPhiC[jp] = wrap_angle(v);
    }
  };

  // stage B: rotate / scale / transpose the raw tiles into LDS operands
  auto stage_tiles = [&](int c) {
    const int s0 = c * Q;
#pragma unroll
    for (int s = 0; s < Lt::JS; ++s) {
      const int j = tid + s * kThreads;
      const int kind = j < Lt::JB ? 0 : (j < 2 * Lt::JB ? 1 : 2);
      const int idx = kind == 0 ? j : (kind == 1 ? j - Lt::JB : j - 2 * Lt::JB);
      const int D = kind == 2 ? P : N;
      const int cpr = D / VE;
      const int rb = idx / cpr, cb = idx % cpr;
      const int c0 = cb * VE;
      float v[4][VE];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[k][q] = __uint_as_float(raw[s][k][q]);
      // prologue: a row of B or C is N / VE consecutive lanes (aligned: B and C
      // jobs start at multiples of 64), reduced with shuffles on every lane
      float scl[4] = {1.f, 1.f, 1.f, 1.f};
      if (proNorm) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float ss = 0.f;
#pragma unroll
          for (int q = 0; q < VE; ++q) ss += v[k][q] * v[k][q];
#pragma unroll
          for (int off = 1; off < N / VE; off <<= 1) ss += __shfl_xor(ss, off);
          scl[k] = ss > 0.f ? rsqrtf(ss * (1.f / N) + p.pro.eps) : 0.f;
        }
      }
      if (j < Lt::JOBS) {
        if (proBC && kind < 2) {
          const float* w = kind == 0 ? p.pro.B_w : p.pro.C_w;
          const float* bias = kind == 0 ? p.pro.B_bias : p.pro.C_bias;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const size_t ob = (static_cast<size_t>(hh) * R + ((4 * rb + k) & (R - 1))) * N + c0;
#pragma unroll
            for (int q = 0; q < VE; ++q) {
              if (proNorm) v[k][q] *= scl[k] * (w != nullptr ? w[c0 + q] : 1.f);
              if (bias != nullptr) v[k][q] += bias[ob + q];
            }
          }
        }
        if (kind < 2 && rope) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int tl = (4 * rb + k) >> lgR;
            if (tl >= Q) continue;  // an empty row: no angle table entry
#pragma unroll
            for (int q = 0; q < VE / 2; ++q) {
              const float2 csn = *reinterpret_cast<const float2*>(sCS + 2 * (tl * (N / 2) + c0 / 2 + q));
              const float a0 = v[k][2 * q], a1 = v[k][2 * q + 1];
              v[k][2 * q] = csn.x * a0 + csn.y * a1;
              v[k][2 * q + 1] = -csn.y * a0 + csn.x * a1;
            }
          }
        }
        if (kind < 2) {
          E* dst = kind == 0 ? sB : sC;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            E* rowp = dst + (4 * rb + k) * PN + c0;
#pragma unroll
            for (int q = 0; q < VE; q += 4) lds_put4(rowp + q, v[k][q], v[k][q + 1], v[k][q + 2], v[k][q + 3]);
          }
        }
        if (kind == 0) {
          float w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = sW[(4 * rb + k) >> lgR];
#pragma unroll
          for (int e = 0; e < VE; ++e)
            lds_put4(sBwT + (c0 + e) * PR + 4 * rb, w[0] * v[0][e], w[1] * v[1][e], w[2] * v[2][e], w[3] * v[3][e]);
        } else if (kind == 2) {
#pragma unroll
          for (int e = 0; e < VE; ++e)
            lds_put4(sXT + (c0 + e) * PR + 4 * rb, v[0][e], v[1][e], v[2][e], v[3][e]);
        }
        // carry-out of the last token: rotated B (fp32) and x (storage type)
        if (kind != 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i = 4 * rb + k;
            if ((i >> lgR) < Q && s0 + (i >> lgR) == L - 1) {
              const size_t o = (static_cast<size_t>(bh) * R + (i & (R - 1))) * D + c0;
              if (kind == 0 && p.Bprev_rot_out != nullptr) {
#pragma unroll
                for (int q = 0; q < VE; q += 4)
                  store4<float>(p.Bprev_rot_out + o + q, v[k][q], v[k][q + 1], v[k][q + 2], v[k][q + 3]);
              } else if (kind == 2 && p.xprev_out != nullptr) {
                *reinterpret_cast<u32x4*>(static_cast<T*>(p.xprev_out) + o) = raw[s][k];
              }
            }
          }
        }
      }
    }
  };

  // H' accumulators (fp32 state, MFMA C/D layout: row n = 16nt+4g+jj, col p = 16pt+l16)
  f32x4 acc_h[Lt::HT];
  auto write_HT = [&]() {
#pragma unroll
    for (int k = 0; k < Lt::HT; ++k) {
      const int idx = wave + k * kWaves;
      if (idx < Lt::NHT) {
        const int nt = idx / NPT, pt = idx % NPT;
        lds_put4(sHT + (16 * pt + l16) * PN + 16 * nt + 4 * g, acc_h[k][0], acc_h[k][1], acc_h[k][2], acc_h[k][3]);
      }
    }
  };

  // ------------------------------------------------------------ prologue
  if constexpr (NK > N) {
    // contraction padding n in [N, NK) of C, B and H'^T stays zero for the whole walk
    for (int e = tid; e < kRows * (NK - N); e += kThreads) {
      const int r = e / (NK - N), cc = N + e % (NK - N);
      sC[r * PN + cc] = E(0);
      sB[r * PN + cc] = E(0);
    }
    for (int e = tid; e < P * (NK - N); e += kThreads) sHT[(e / (NK - N)) * PN + N + e % (NK - N)] = E(0);
  }
  if (rope) {
    for (int j = tid; j < N / 2; j += kThreads)
      sPhiC[j] = p.phi0 != nullptr ? p.phi0[static_cast<size_t>(bh) * (N / 2) + j] : 0.f;
  }
  issue_loads(0);
  stage_scalars();
  __syncthreads();
  if (rope) {
    stage_angles();
    __syncthreads();
  }
  stage_tiles(0);
  {
    // H'_{-1} = h0 + (1 - lambda_0) Delta_0 sum_r Bprev_rot[r] xprev[r]^T
    const size_t o0 = static_cast<size_t>(b) * L * H + hh;
    const float coef = (1.f - p.lam[o0]) * delta_of(p.dt[o0], proDt, dtBias, true);
    const bool hasCarry = p.Bprev_rot != nullptr && p.xprev != nullptr;
#pragma unroll
    for (int k = 0; k < Lt::HT; ++k) {
      const int idx = wave + k * kWaves;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      if (idx < Lt::NHT) {
        const int nt = idx / NPT, pt = idx % NPT;
        const int pc = 16 * pt + l16;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int n = 16 * nt + 4 * g + jj;
          float v = p.h0 != nullptr ? p.h0[static_cast<size_t>(bh) * N * P + static_cast<size_t>(n) * P + pc] : 0.f;
          if (hasCarry) {
            float u = 0.f;
            for (int r = 0; r < R; ++r)
              u += p.Bprev_rot[(static_cast<size_t>(bh) * R + r) * N + n] *
                   load_scalar(static_cast<const T*>(p.xprev) + (static_cast<size_t>(bh) * R + r) * P + pc);
            v += coef * u;
          }
          a[jj] = v;
        }
      }
      acc_h[k] = a;
    }
  }
  write_HT();
  __syncthreads();

  // ------------------------------------------------------------ chunk walk
  const int it = wave & 3;   // i tile (16 rows of the chunk) for the y product
  const int ph = wave >> 2;  // p half
  const int iRow = 16 * it + l16;
  T* yg = static_cast<T*>(p.y);

  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) issue_loads(c + 1);

    // ---- y for rows iRow: intra-chunk masked product + readout of H'_{prev}
    typename M::Frag cfr[NK / K];
#pragma unroll
    for (int kb = 0; kb < NK / K; ++kb) cfr[kb] = M::ld(sC + iRow * PN, kb, g);
    f32x4 yacc[Lt::YT];
#pragma unroll
    for (int k = 0; k < Lt::YT; ++k) yacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ti = iRow >> lgR;
    const float lamI = sLam[ti];
    const float gamI = sGam[ti];
    auto gram_masked = [&](int jt) -> f32x4 {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NK / K; ++kb) acc = M::mma(M::ld(sB + (16 * jt + l16) * PN, kb, g), cfr[kb], acc);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int tj = (16 * jt + 4 * g + jj) >> lgR;
        float m;
        if (tj < ti) m = __expf(lamI - sLam[tj]) * sDel[tj];
        else if (tj == ti) m = gamI;
        else m = 0.f;
        acc[jj] *= m;
      }
      return acc;
    };

#pragma unroll
    for (int jt = 0; jt < kRows / 16; ++jt) {
      if (jt <= it) {
        const f32x4 sm = gram_masked(jt);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
          for (int k = 0; k < Lt::YT; ++k) {
            const int pt = ph + 2 * k;
            if (pt < NPT) {
              const float a = sXT[(16 * pt + l16) * PR + 16 * jt + 4 * g + jj];
              yacc[k] = M::mma(a, sm[jj], yacc[k]);
            }
          }
        }
      }
    }
    // readout of the carried state: Y^T += diag(exp Lam_i) H'^T Ctil^T
    const float decI = sDec[ti];
#pragma unroll
    for (int k = 0; k < Lt::YT; ++k) {
      const int pt = ph + 2 * k;
      if (pt < NPT) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NK / K; ++kb) z = M::mma(M::ld(sHT + (16 * pt + l16) * PN, kb, g), cfr[kb], z);
        yacc[k] += decI * z;
      }
    }
    // ---- state update: H' = exp(Lam_e) H' + (w B)^T X
    const float cdec = sChunkDec[0];
#pragma unroll
    for (int k = 0; k < Lt::HT; ++k) {
      const int idx = wave + k * kWaves;
      if (idx < Lt::NHT) {
        const int nt = idx / NPT, pt = idx % NPT;
        f32x4 a = acc_h[k] * cdec;
#pragma unroll
        for (int kb = 0; kb < kRows / K; ++kb)
          a = M::mma(M::ld(sBwT + (16 * nt + l16) * PR, kb, g), M::ld(sXT + (16 * pt + l16) * PR, kb, g), a);
        acc_h[k] = a;
      }
    }
    // ---- store y rows of this chunk
    {
      const int t = c * Q + ti;
      if (ti < Q && t < L) {
        T* yrow = yg + (rowbase(t) + (iRow & (R - 1))) * P;
#pragma unroll
        for (int k = 0; k < Lt::YT; ++k) {
          const int pt = ph + 2 * k;
          if (pt < NPT) store4<T>(yrow + 16 * pt + 4 * g, yacc[k][0], yacc[k][1], yacc[k][2], yacc[k][3]);
        }
      }
    }
    __syncthreads();
    write_HT();
    if (c + 1 < nch) {
      stage_scalars();
      __syncthreads();
      if (rope) {
        stage_angles();
        __syncthreads();
      }
      stage_tiles(c + 1);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  if (p.h_final != nullptr) {
#pragma unroll
    for (int k = 0; k < Lt::HT; ++k) {
      const int idx = wave + k * kWaves;
      if (idx < Lt::NHT) {
        const int nt = idx / NPT, pt = idx % NPT;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          p.h_final[static_cast<size_t>(bh) * N * P + static_cast<size_t>(16 * nt + 4 * g + jj) * P + 16 * pt + l16] =
              acc_h[k][jj];
      }
    }
  }
  if (rope && p.phi_out != nullptr) {
    for (int j = tid; j < N / 2; j += kThreads) p.phi_out[static_cast<size_t>(bh) * (N / 2) + j] = sPhiC[j];
  }
}

template <typename T, int N, int P>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  using Lt = Layout<T, N, P>;
  const bool rope = p.theta != nullptr || p.omega != nullptr;
  const size_t lds = rope ? Lt::kBytesRope : Lt::kBytesReal;
  // cleared once per device for the larger of the two layouts that fit a CU
  constexpr size_t kMax = 160 * 1024;
  constexpr size_t kAllow = Lt::kBytesRope <= kMax && Lt::kBytesRope > Lt::kBytesReal ? Lt::kBytesRope
                                                                                      : Lt::kBytesReal;
  static std::atomic<uint64_t> cleared{0};
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&prefill_kernel<T, N, P>), kAllow, cleared);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<T, N, P>), dim3(p.Bt * p.H), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

template <typename T, int N>
static hipError_t prefill_n(const PrefillParams& p, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_prefill_t<T, N, 16>(p, s);
    case 32: return launch_prefill_t<T, N, 32>(p, s);
    case 64: return launch_prefill_t<T, N, 64>(p, s);
    case 128: return launch_prefill_t<T, N, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t prefill_dt(const PrefillParams& p, hipStream_t s) {
  switch (p.N) {
    case 16: return prefill_n<T, 16>(p, s);
    case 32: return prefill_n<T, 32>(p, s);
    case 64: return prefill_n<T, 64>(p, s);
    case 128: return prefill_n<T, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int N>
static size_t lds_p(int P, bool rope) {
  switch (P) {
    case 16: return rope ? Layout<T, N, 16>::kBytesRope : Layout<T, N, 16>::kBytesReal;
    case 32: return rope ? Layout<T, N, 32>::kBytesRope : Layout<T, N, 32>::kBytesReal;
    case 64: return rope ? Layout<T, N, 64>::kBytesRope : Layout<T, N, 64>::kBytesReal;
    case 128: return rope ? Layout<T, N, 128>::kBytesRope : Layout<T, N, 128>::kBytesReal;
  }
  return 0;
}
template <typename T>
static size_t lds_n(int N, int P, bool rope) {
  switch (N) {
    case 16: return lds_p<T, 16>(P, rope);
    case 32: return lds_p<T, 32>(P, rope);
    case 64: return lds_p<T, 64>(P, rope);
    case 128: return lds_p<T, 128>(P, rope);
  }
  return 0;
}
}  // namespace m3
