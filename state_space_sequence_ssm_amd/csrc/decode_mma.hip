// Single-token MIMO decode step on the matrix cores (gfx950), bf16 inputs.
//
// Same operation as the vector-ALU step ("Znakomstvo s Mamba-3"
// (chernovdev.ru), sec. 1 displayed recurrence, sec. 2 cumulative RoPE, sec. 3
// MIMO: with R ranks the state update becomes a matrix product):
//   h <- alpha h + [beta Btil_prev ; gamma Btil_t]^T [xprev ; x_t]   (rank 2R)
//   y_t = Ctil_t h
// At rank R the step does about 6 R N P flops on the same 2 N P * 4 bytes of
// state traffic; on the vector ALUs (with the operands from LDS) that ran at
// ~18 TFLOP/s and fell to 31% of HBM at R = 16, so both products run on
// v_mfma_f32_16x16x32_bf16 with the 2R ranks as the k dimension (padded to 32).
//
// MI355X design.  One workgroup per (batch, head), W waves of 64 (W = 1 for
// N = P = 64); each wave keeps 16 state tiles of 16 x 16 in MFMA accumulators
// for the whole step.  Tile (nt, pt), lane (g, l16) holds
// h[16 nt + 4 g + jj][PT l16 + pt], jj = 0..3: the P columns are interleaved
// over the PT tiles so that a lane's PT values of a row are contiguous, and the
// state streams with 16-byte loads and stores of whole rows.  The same layout
// is the B operand of the readout (k = n), so y = Ctil h takes the state
// straight from the accumulators.  Operands are split into a bf16 high part
// and a bf16 remainder (gamma Btil, beta Btil_prev, Ctil and the state in the
// readout), which keeps the products at about fp32 accuracy: the state never
// passes through a single bf16 rounding.
#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {
namespace dmma {

constexpr int kMaxR = 16;  // 2R ranks fill one k block of 32

template <int N, int P>
struct Cfg {
  static constexpr int NT = N / 16, PT = P / 16, J = N / 2;
  static constexpr int W = NT * PT > 16 ? NT * PT / 16 : 1;  // waves per unit
  static constexpr int NTW = NT / W;                         // n tiles per wave (even)
  static constexpr int T = 64 * W;
  static constexpr int PN = N + 4, PX = P + 4;               // bf16 row pitches
  static constexpr size_t oBwH = 0;                          // [32][PN] gamma Btil ; beta Btil_prev (high)
  static constexpr size_t oBwL = oBwH + 32 * PN * 2;         // remainder
  static constexpr size_t oX = oBwL + 32 * PN * 2;           // [32][PX] x ; xprev, columns interleaved
  static constexpr size_t oCH = oX + 32 * PX * 2;            // [16][PN] Ctil (high)
  static constexpr size_t oCL = oCH + 16 * PN * 2;           // remainder
  static constexpr size_t oCS = oCL + 16 * PN * 2;           // float [N]: cos, sin per pair
  static constexpr size_t oY = oCS + N * 4;                  // float [W][16][P]: y parts (W > 1)
  static constexpr size_t kBytes = oY + (W > 1 ? size_t(W) * 16 * P * 4 : 0);
  static_assert(NTW % 2 == 0 && PT % 4 == 0, "shape outside the matrix-core decode");
};

__device__ __forceinline__ float hi_of(uint32_t h, int k) {
  return __uint_as_float(k == 0 ? h << 16 : h & 0xffff0000u);
}
// a pair as bf16 high parts and bf16 remainders
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - hi_of(hi, 0), b - hi_of(hi, 1));
}

template <int N, int P, int RMAX>
__global__ __launch_bounds__((Cfg<N, P>::T)) void decode_mma_kernel(DecodeParams p) {
  using Cf = Cfg<N, P>;
  constexpr int PT = Cf::PT, J = Cf::J, W = Cf::W, NTW = Cf::NTW, T = Cf::T, PN = Cf::PN, PX = Cf::PX;
  constexpr int KB = (RMAX * J + T - 1) / T;        // (rank, pair) items of B and C per thread
  constexpr int KX = (RMAX * P / 2 + T - 1) / T;    // (rank, column pair) items of x per thread
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* const sBwH = reinterpret_cast<uint16_t*>(smem + Cf::oBwH);
  uint16_t* const sBwL = reinterpret_cast<uint16_t*>(smem + Cf::oBwL);
  uint16_t* const sX = reinterpret_cast<uint16_t*>(smem + Cf::oX);
  uint16_t* const sCH = reinterpret_cast<uint16_t*>(smem + Cf::oCH);
  uint16_t* const sCL = reinterpret_cast<uint16_t*>(smem + Cf::oCL);
  float* const sCS = reinterpret_cast<float*>(smem + Cf::oCS);
  float* const sY = reinterpret_cast<float*>(smem + Cf::oY);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x, hh = bh % p.H, R = p.R;
  const bool rope = p.theta != nullptr || p.omega != nullptr;
  const size_t vecN = static_cast<size_t>(bh) * R * N;
  const size_t vecP = static_cast<size_t>(bh) * R * P;

  // ---- every load of the step, in the order of use: the token's small
  // vectors, then the state.  Wait counters retire loads in issue order, so
  // the small vectors are staged while the state is still in flight.
  // Indices are clamped, not branched, so the wait counts stay static.
  float phiOld = 0.f, thRaw = 0.f;
  if (rope) {
    const int j = tid < J ? tid : 0;
    phiOld = p.phi[static_cast<size_t>(bh) * J + j];
    thRaw = p.omega != nullptr ? p.omega[static_cast<size_t>(bh / p.H) * J + j] : p.theta[static_cast<size_t>(bh) * J + j];
  }
  uint32_t bu[KB], cu[KB];
  float2 bp[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const int e = tid + T * i, ec = e < R * J ? e : 0;
    bu[i] = *reinterpret_cast<const uint32_t*>(static_cast<const bf16_t*>(p.B) + vecN + 2 * ec);
    cu[i] = *reinterpret_cast<const uint32_t*>(static_cast<const bf16_t*>(p.C) + vecN + 2 * ec);
    bp[i] = *reinterpret_cast<const float2*>(p.Bprev_rot + vecN + 2 * ec);
  }
  uint32_t xNew[KX], xo[KX];
#pragma unroll
  for (int i = 0; i < KX; ++i) {
    const int e = tid + T * i, ec = e < R * (P / 2) ? e : 0;
    xNew[i] = *reinterpret_cast<const uint32_t*>(static_cast<const bf16_t*>(p.x) + vecP + 2 * ec);
    xo[i] = *reinterpret_cast<const uint32_t*>(static_cast<const bf16_t*>(p.xprev) + vecP + 2 * ec);
  }
  // the state: this wave's rows n = 16 (wave NTW + nt) + 4 g + jj, columns PT l16 .. PT l16 + PT - 1
  const float* hsrc = p.h + static_cast<size_t>(bh) * N * P;
  f32x4 raw[NTW][4][PT / 4];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int qd = 0; qd < PT / 4; ++qd)
        raw[nt][jj][qd] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
            hsrc + static_cast<size_t>(16 * (wave * NTW + nt) + 4 * g + jj) * P + PT * l16 + 4 * qd));

  // ---- scalars of the token (as in the vector-ALU step)
  const bool proDt = p.pro.dt_softplus != 0;
  const float dt = delta_of(p.dt[bh], proDt, proDt && p.pro.dt_bias != nullptr ? p.pro.dt_bias[hh] : 0.f, true);
  const float lm = p.lam[bh];
  const bool proNorm = p.pro.bc_norm != 0;
  const float alpha = __expf(dt * (p.A_tok != nullptr ? p.A_tok[bh] : p.A[hh]));
  const float beta = (1.f - lm) * dt * alpha;
  const float gamma = lm * dt;

  // ---- angles: Phi <- wrap(Phi + theta), cos / sin per pair
  float phiNew = 0.f;
  if (rope && tid < J) {
    phiNew = wrap_angle(phiOld + (p.omega != nullptr ? dt * thRaw : thRaw));
    float sn, cs;
    sincosf(phiNew, &sn, &cs);
    sCS[2 * tid] = cs;
    sCS[2 * tid + 1] = sn;
  }
  // k rows 2R..31 of the update operands are zero
  for (int e = tid; e < (32 - 2 * R) * (PN / 2); e += T) {
    const int r = 2 * R + e / (PN / 2), c = e % (PN / 2);
    reinterpret_cast<uint32_t*>(sBwH + r * PN)[c] = 0u;
    reinterpret_cast<uint32_t*>(sBwL + r * PN)[c] = 0u;
  }
  for (int e = tid; e < (32 - 2 * R) * (PX / 2); e += T) {
    const int r = 2 * R + e / (PX / 2), c = e % (PX / 2);
    reinterpret_cast<uint32_t*>(sX + r * PX)[c] = 0u;
  }
  // ---- x, xprev (rank r, columns 2c, 2c + 1) into the interleaved column order
#pragma unroll
  for (int i = 0; i < KX; ++i) {
    const int e = tid + T * i;
    if (e < R * (P / 2)) {
      const int r = (2 * e) / P, c = (2 * e) % P;
      const int s0 = (c % PT) * 16 + c / PT, s1 = ((c + 1) % PT) * 16 + (c + 1) / PT;
      sX[r * PX + s0] = static_cast<uint16_t>(xNew[i] & 0xffffu);
      sX[r * PX + s1] = static_cast<uint16_t>(xNew[i] >> 16);
      sX[(R + r) * PX + s0] = static_cast<uint16_t>(xo[i] & 0xffffu);
      sX[(R + r) * PX + s1] = static_cast<uint16_t>(xo[i] >> 16);
    }
  }
  __syncthreads();

  // ---- B, C (rank r, pair j): prologue, rotation, operands; the carry keeps Btil in fp32
  float2 bNew[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const int e = tid + T * i;
    const bool v = e < R * J;
    const int ec = v ? e : 0;
    const int r = ec / J, j = ec % J;
    float b0 = hi_of(bu[i], 0), b1 = hi_of(bu[i], 1), c0 = hi_of(cu[i], 0), c1 = hi_of(cu[i], 1);
    if (proNorm) {
      // 1 / RMS of the row: its J pairs sit on J aligned lanes of one wave (a zero row stays zero)
      float sb = v ? b0 * b0 + b1 * b1 : 0.f, sc = v ? c0 * c0 + c1 * c1 : 0.f;
#pragma unroll
      for (int off = 1; off < J; off <<= 1) {
        sb += __shfl_xor(sb, off);
        sc += __shfl_xor(sc, off);
      }
      const float kb = sb > 0.f ? rsqrtf(sb * (1.f / N) + p.pro.eps) : 0.f;
      const float kc = sc > 0.f ? rsqrtf(sc * (1.f / N) + p.pro.eps) : 0.f;
      b0 *= kb * (p.pro.B_w != nullptr ? p.pro.B_w[2 * j] : 1.f);
      b1 *= kb * (p.pro.B_w != nullptr ? p.pro.B_w[2 * j + 1] : 1.f);
      c0 *= kc * (p.pro.C_w != nullptr ? p.pro.C_w[2 * j] : 1.f);
      c1 *= kc * (p.pro.C_w != nullptr ? p.pro.C_w[2 * j + 1] : 1.f);
    }
    const size_t ob = (static_cast<size_t>(hh) * R + r) * N + 2 * j;
    if (p.pro.B_bias != nullptr) {
      b0 += p.pro.B_bias[ob];
      b1 += p.pro.B_bias[ob + 1];
    }
    if (p.pro.C_bias != nullptr) {
      c0 += p.pro.C_bias[ob];
      c1 += p.pro.C_bias[ob + 1];
    }
    if (rope) {
      const float cs = sCS[2 * j], sn = sCS[2 * j + 1];
      const float rb0 = cs * b0 + sn * b1, rb1 = cs * b1 - sn * b0;
      const float rc0 = cs * c0 + sn * c1, rc1 = cs * c1 - sn * c0;
      b0 = rb0; b1 = rb1; c0 = rc0; c1 = rc1;
    }
    bNew[i] = make_float2(b0, b1);
    if (v) {
      uint32_t hi, lo;
      split2(gamma * b0, gamma * b1, hi, lo);
      reinterpret_cast<uint32_t*>(sBwH + r * PN)[j] = hi;
      reinterpret_cast<uint32_t*>(sBwL + r * PN)[j] = lo;
      split2(beta * bp[i].x, beta * bp[i].y, hi, lo);
      reinterpret_cast<uint32_t*>(sBwH + (R + r) * PN)[j] = hi;
      reinterpret_cast<uint32_t*>(sBwL + (R + r) * PN)[j] = lo;
      split2(c0, c1, hi, lo);
      reinterpret_cast<uint32_t*>(sCH + r * PN)[j] = hi;
      reinterpret_cast<uint32_t*>(sCL + r * PN)[j] = lo;
    }
  }
  __syncthreads();  // every old carry value has been read (and staged) before the new one is written

  // ---- carry-out: Btil_t, x_t, Phi
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    const int e = tid + T * i;
    if (e < R * J) *reinterpret_cast<float2*>(p.Bprev_rot + vecN + 2 * e) = bNew[i];
  }
#pragma unroll
  for (int i = 0; i < KX; ++i) {
    const int e = tid + T * i;
    if (e < R * (P / 2)) *reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(p.xprev) + vecP + 2 * e) = xNew[i];
  }
  if (rope && tid < J) p.phi[static_cast<size_t>(bh) * J + tid] = phiNew;

  // ---- operand fragments (k = 32 rows of a row-major LDS tile, or its rows as M)
  auto frag_col = [&](const uint16_t* base, int pitch, int c0) __attribute__((always_inline)) {
    const int rT = 4 * g + (l16 >> 2), c4 = 4 * (l16 & 3);
    return cat8(lds_read_tr(base + rT * pitch + c0 + c4), lds_read_tr(base + (16 + rT) * pitch + c0 + c4));
  };
  auto frag_row = [&](const uint16_t* base, int pitch, int kb) __attribute__((always_inline)) {
    const uint16_t* q = base + l16 * pitch + 32 * kb + 4 * g;
    return cat8(*reinterpret_cast<const u32x2*>(q), *reinterpret_cast<const u32x2*>(q + 16));
  };

  // ---- h <- alpha h + Bw^T X on the matrix cores
  f32x4 acc[NTW][PT];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const bf16x8 bx = frag_col(sX, PX, 16 * pt);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      f32x4 a;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) a[jj] = alpha * raw[nt][jj][pt / 4][pt % 4];
      const int n0 = 16 * (wave * NTW + nt);
      a = mma(frag_col(sBwH, PN, n0), bx, a);
      a = mma(frag_col(sBwL, PN, n0), bx, a);
      acc[nt][pt] = a;
    }
  }
  float* hdst = p.h + static_cast<size_t>(bh) * N * P;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int qd = 0; qd < PT / 4; ++qd) {
        const f32x4 v = {acc[nt][4 * qd][jj], acc[nt][4 * qd + 1][jj], acc[nt][4 * qd + 2][jj], acc[nt][4 * qd + 3][jj]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(
            hdst + static_cast<size_t>(16 * (wave * NTW + nt) + 4 * g + jj) * P + PT * l16 + 4 * qd));
      }

  // ---- y = Ctil h: rows r (M, padded to 16), k = this wave's n, columns of tile pt
  f32x4 yv[PT];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NTW / 2; ++k) {
      const int kb = wave * (NTW / 2) + k;
      const f32x4 h0 = acc[2 * k][pt], h1 = acc[2 * k + 1][pt];
      const u32x2 a0 = pack4(h0), a1 = pack4(h1);
      const f32x4 r0 = {h0[0] - hi_of(a0[0], 0), h0[1] - hi_of(a0[0], 1), h0[2] - hi_of(a0[1], 0),
                        h0[3] - hi_of(a0[1], 1)};
      const f32x4 r1 = {h1[0] - hi_of(a1[0], 0), h1[1] - hi_of(a1[0], 1), h1[2] - hi_of(a1[1], 0),
                        h1[3] - hi_of(a1[1], 1)};
      const bf16x8 bh8 = cat8(a0, a1), bl8 = cat8(pack4(r0), pack4(r1));
      const bf16x8 ch = frag_row(sCH, PN, kb), cl = frag_row(sCL, PN, kb);
      y = mma(ch, bh8, y);
      y = mma(ch, bl8, y);
      y = mma(cl, bh8, y);
    }
    yv[pt] = y;
  }
  bf16_t* yg = static_cast<bf16_t*>(p.y) + vecP;
  if constexpr (W == 1) {
    // lane holds y[4 g + jj][PT l16 + pt]: PT consecutive columns of a row
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 4 * g + jj;
      if (r < R) {
#pragma unroll
        for (int qd = 0; qd < PT / 4; ++qd)
          *reinterpret_cast<u32x2*>(yg + r * P + PT * l16 + 4 * qd) =
              u32x2{pack_bf16x2(yv[4 * qd][jj], yv[4 * qd + 1][jj]), pack_bf16x2(yv[4 * qd + 2][jj], yv[4 * qd + 3][jj])};
      }
    }
  } else {
    // the waves' parts over their n rows, summed in wave order
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 4 * g + jj;
      if (r < R)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) sY[(wave * 16 + r) * P + PT * l16 + pt] = yv[pt][jj];
    }
    __syncthreads();
    for (int e = tid; e < R * P; e += T) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) s += sY[w * 16 * P + e];
      yg[e].bits = f32_to_bf16(s);
    }
  }
}

template <int N, int P, int RMAX>
hipError_t launch_npr(const DecodeParams& p, hipStream_t s) {
  using Cf = Cfg<N, P>;
  static std::atomic<uint64_t> cleared{0};
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&decode_mma_kernel<N, P, RMAX>), Cf::kBytes, cleared);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_mma_kernel<N, P, RMAX>), dim3(p.Bt * p.H), dim3(Cf::T), Cf::kBytes, s, p);
  return hipGetLastError();
}
// RMAX bounds the rank held in registers; the small-rank variant keeps fewer
template <int N, int P>
hipError_t launch_np(const DecodeParams& p, hipStream_t s) {
  return p.R <= 4 ? launch_npr<N, P, 4>(p, s) : launch_npr<N, P, kMaxR>(p, s);
}

template <int N>
hipError_t launch_n(const DecodeParams& p, hipStream_t s) {
  switch (p.P) {
    case 64: return launch_np<N, 64>(p, s);
    case 128: return launch_np<N, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dmma

bool decode_mma_supported(const DecodeParams& p) {
  return p.bf16 && p.R >= 1 && p.R <= dmma::kMaxR && (p.N == 32 || p.N == 64 || p.N == 128) &&
         (p.P == 64 || p.P == 128);
}

hipError_t launch_decode_mma(const DecodeParams& p, hipStream_t s) {
  switch (p.N) {
    case 32: return dmma::launch_n<32>(p, s);
    case 64: return dmma::launch_n<64>(p, s);
    case 128: return dmma::launch_n<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace m3
