// Backward pass of the chunked prefill of the Mamba-3 SSM core: gradients of
// x, B, C, Delta, lambda, A, theta and the carry-in, bf16 inputs (gfx950).
//
// The pages print no backward pass.  This is the adjoint of the chunked
// evaluation ("La dualita: Mamba-2 e Mamba-3" (book.paithon.it), sec. "Perche
// conviene: i tensor core") of the recurrence ("Znakomstvo s Mamba-3"
// (chernovdev.ru), sec. 1-3), obtained by differentiating the chunk equations.
// Forward, per chunk of tokens s..e with H the shifted state entering it
// (Lam_t = sum_{k=s..t} Delta_k A_k, E_t = exp(Lam_t), D = exp(Lam_e),
// w_j = exp(Lam_e - Lam_j) delta_j, M_ij = exp(Lam_i - Lam_j) delta_j for j < i,
// M_ii = gamma_i):
//   y_i    = sum_{j<=i} M_ij <Ctil_i, Btil_j> x_j + E_i Ctil_i^T H
//   H_next = D H + sum_j w_j Btil_j x_j^T
// Backward, with G the gradient of H_next and dY that of y:
//   S1 = M o (C B^T),  S2 = M o (dY X^T)
//   dX = S1^T dY + w (B G),  dBtil = S2^T C + w (X G^T),  dCtil = S2 B + E (dY H^T)
//   G <- D G + C^T E dY                          (the gradient of H)
//   dM = (C B^T) o (dY X^T), dE_i = <dY_i H^T, Ctil_i>, dw_j = <(B G)_j, x_j>,
//   dD = <G, H>  -> Lam, delta, gamma -> Delta, lambda, A
// and through the rotation dB = R(Phi) dBtil, dPhi = dBtil_0 Btil_1 -
// dBtil_1 Btil_0 per pair (likewise for C); dtheta_t, the sum of dPhi over
// tokens >= t, is <dh_final, J h_final> - <G, J H> at each chunk start (the
// state carried across it) plus this chunk's dPhi after t.
//
// MI355X design.  One 512-thread workgroup (8 wave64) per (batch, head).  It
// first walks the chunks forward for the state only (B and X staged in LDS,
// H <- D H + Btil^T (w X) on MFMA) and writes the shifted state entering each
// chunk, and the angle entering it, to the workspace; then it walks the chunks
// backward with G in MFMA accumulators.  All products are bf16 MFMA 16x16x32
// with fp32 accumulation on bf16 LDS tiles; operands needed along the token
// axis come straight from the row-major tiles through the transposing LDS
// read.  dX, dB and dC are formed as transposed tiles, so a lane holds four
// consecutive columns of one row: 8-byte stores, and whole rotation pairs in
// registers.  Reductions run in a fixed order (no atomics): results are
// bit-reproducible.
//
// Sequence split.  With too few (batch, head) units to fill the chip, the
// chunks are cut at chunk cm into an earlier segment 0 and a later segment 1,
// two workgroups per unit, in two launches:
//   pre:  segment 0 walks its chunks forward for the states (as above) and
//         writes the shifted state and the angle entering chunk cm; segment 1
//         sums, forward in time from a zero start and with angles counted
//         from its first token, its chunks' part of the gradient entering
//         chunk cm: G_rel = sum_c Dcum_c Ctil_rel^T (E dY) with Dcum_c the
//         decay from chunk cm to chunk c, and the decay Dcum over the segment.
//   main: segment 1 walks forward from that state, then backward from
//         dh_final; segment 0 walks backward only, from the gradient entering
//         chunk cm, Rot(Phi) G_rel + Dcum dh_final (Phi the angle entering
//         chunk cm: rotations compose), with <G, J H> at chunk cm as its
//         dtheta anchor.
// Segment 0's last delta term reaches token cm Q (the beta term of the
// recurrence), so that token's Delta and lambda gradients, and every dtheta
// of segment 0 (which lacks segment 1's sum of dPhi), are completed by a small
// joining kernel afterwards.
#pragma once
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {
namespace bw {

constexpr int kRows = 64;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int N, int P, bool ROPE>
struct Lay {
  static constexpr int NK = N < 32 ? 32 : N;  // contractions over n padded to k blocks of 32
  static constexpr int PK = P < 32 ? 32 : P;
  static constexpr int PN = NK + 4;  // bf16 row pitches (rows stay 8-byte aligned)
  static constexpr int PP = PK + 4;
  static constexpr int PR = kRows + 4;
  static constexpr int NT = N / 16, PT = P / 16;
  static constexpr int NST = NT * PT;                      // 16 x 16 state tiles
  static constexpr int STW = (NST + kWaves - 1) / kWaves;  // state tiles per wave
  static constexpr int J = N / 2;
  static constexpr int JP = J + 1;  // angle-table row pitch (odd: a column spreads over the banks)
  // bf16 tiles (element offsets)
  static constexpr size_t oCr = 0;                           // [64][PN] rotated C
  static constexpr size_t oBr = oCr + size_t(kRows) * PN;    // [64][PN] rotated B
  static constexpr size_t oX = oBr + size_t(kRows) * PN;     // [64][PP] x
  static constexpr size_t oDY = oX + size_t(kRows) * PP;     // [64][PP] dy
  static constexpr size_t oHT = oDY + size_t(kRows) * PP;    // [PK][PN] H^T (row p)
  static constexpr size_t oGT = oHT + size_t(PK) * PN;       // [PK][PN] G^T
  static constexpr size_t oS1 = oGT + size_t(PK) * PN;       // [64][PR] S1^T
  static constexpr size_t oS2 = oS1 + size_t(kRows) * PR;    // [64][PR] S2^T
  static constexpr size_t kBf = oS2 + size_t(kRows) * PR;
  static constexpr size_t fBase = (kBf * 2 + 15) / 16 * 16;  // bytes: fp32 region
  // fp32 region (float offsets)
  static constexpr int kSc = 80;
  static constexpr size_t fSc = 0;                      // [10][kSc] per-token scalars
  static constexpr size_t fRow = fSc + 10 * kSc;        // [4][64][2] row sums of the Gram tiles
  static constexpr size_t fCol = fRow + 4 * 64 * 2;     // [4][64][2] column sums
  static constexpr size_t fE = fCol + 4 * 64 * 2;       // [NT][64] readout-decay gradient parts
  static constexpr size_t fW = fE + NT * 64;            // [PT][64] column-weight gradient parts
  static constexpr size_t fD = fW + PT * 64;            // [16] per-wave parts
  static constexpr size_t fPhiC = fD + 16;              // [J] angle carry (forward walk)
  static constexpr size_t fPhi = fPhiC + J;             // [64][JP] angles of the chunk's tokens
  static constexpr size_t fDPhi = fPhi + (ROPE ? 64 * JP : 0);  // [64 rows][JP] angle gradients
  static constexpr size_t fThC = fDPhi + (ROPE ? 64 * JP : 0);   // [J] dtheta at the next chunk start
  // second buffers of the per-chunk scalars, Gram row / column sums and
  // per-wave parts: a chunk's scalar gradients are formed during the next
  // chunk's Gram phase, while that chunk fills the other buffer
  static constexpr size_t fSc2 = fThC + (ROPE ? J : 0);
  static constexpr size_t fRow2 = fSc2 + 10 * kSc;
  static constexpr size_t fCol2 = fRow2 + 4 * 64 * 2;
  static constexpr size_t fD2 = fCol2 + 4 * 64 * 2;
  static constexpr size_t fEnd = fD2 + 16;
  static constexpr size_t kBytes = fBase + fEnd * 4;
};
// scalar rows of fSc
enum { kLam2 = 0, kGam, kDel, kE, kW, kDt, kLamb, kA, kMisc };

// w-scaled MFMA operand: slots 0-3 by w0, slots 4-7 by w1 (one bf16 rounding)
__device__ __forceinline__ bf16x8 scale8(bf16x8 x, f32x4 w0, f32x4 w1) {
  const u32x4 v = __builtin_bit_cast(u32x4, x);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float wa = q < 2 ? w0[2 * q] : w1[2 * q - 4], wb = q < 2 ? w0[2 * q + 1] : w1[2 * q - 3];
    o[q] = pack_bf16x2(wa * __uint_as_float(v[q] << 16), wb * __uint_as_float(v[q] & 0xffff0000u));
  }
  return as_bf16x8(o);
}

// MODE 0: the whole sequence per workgroup; 1: the split's pre launch; 2: its
// main launch (blockIdx.y = segment)
template <int N, int P, bool ROPE, int MODE>
__global__ __launch_bounds__(kThreads) void backward_kernel(BackwardParams p) {
  using Lt = Lay<N, P, ROPE>;
  constexpr int PN = Lt::PN, PP = Lt::PP, PR = Lt::PR, NT = Lt::NT, PT = Lt::PT, NST = Lt::NST;
  constexpr int STW = Lt::STW, J = Lt::J, JP = Lt::JP, NKB = Lt::NK / 32, PKB = Lt::PK / 32;
  constexpr int kSc = Lt::kSc;
  // Register budget of the reverse walk: below the largest tiles with RoPE or
  // P = 128 the operand fragments of a wave's fixed tiles are held across a
  // chunk's products (at those tiles the extra live registers would spill).
  constexpr bool kHoist = !(ROPE && (N >= 128 || P >= 128)) && !(P >= 128 && N >= 64);
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* const sm16 = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const sCr = sm16 + Lt::oCr;
  uint16_t* const sBr = sm16 + Lt::oBr;
  uint16_t* const sX = sm16 + Lt::oX;
  uint16_t* const sDY = sm16 + Lt::oDY;
  uint16_t* const sHT = sm16 + Lt::oHT;
  uint16_t* const sGT = sm16 + Lt::oGT;
  uint16_t* const sS1 = sm16 + Lt::oS1;
  uint16_t* const sS2 = sm16 + Lt::oS2;
  float* const f32 = reinterpret_cast<float*>(smem + Lt::fBase);
  // per-chunk tables, one of two buffers by the chunk's parity
  auto scb = [&](int c) { return f32 + ((c & 1) ? Lt::fSc2 : Lt::fSc); };
  auto rowb = [&](int c) { return f32 + ((c & 1) ? Lt::fRow2 : Lt::fRow); };
  auto colb = [&](int c) { return f32 + ((c & 1) ? Lt::fCol2 : Lt::fCol); };
  auto dpb = [&](int c) { return f32 + ((c & 1) ? Lt::fD2 : Lt::fD); };
  float* const sEp = f32 + Lt::fE;
  float* const sWp = f32 + Lt::fW;
  float* const phiC = f32 + Lt::fPhiC;
  float* const sPhi = f32 + Lt::fPhi;
  float* const sDPhi = f32 + Lt::fDPhi;
  float* const sThC = f32 + Lt::fThC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x, b = bh / p.H, hh = bh % p.H;
  const int L = p.L, H = p.H, R = p.R, lgR = p.log2R;
  const int Q = kRows >> lgR;
  const int nch = (L + Q - 1) / Q;
  const int seg = MODE == 0 ? 0 : static_cast<int>(blockIdx.y);
  const int cA = seg == 1 ? p.cm : 0;                     // this workgroup's chunks [cA, cB)
  const int cB = (MODE != 0 && seg == 0) ? p.cm : nch;
  const size_t units = static_cast<size_t>(p.Bt) * H;
  const bf16_t* xg = static_cast<const bf16_t*>(p.x);
  const bf16_t* Bg = static_cast<const bf16_t*>(p.B);
  const bf16_t* Cg = static_cast<const bf16_t*>(p.C);
  const bf16_t* dYg = static_cast<const bf16_t*>(p.dy);
  const float Ah = p.A_tok != nullptr ? 0.f : p.A[hh];
  // chunk-entry states, bf16 in the accumulator tile order (one 8-byte unit per lane per tile)
  uint16_t* const stBase = static_cast<uint16_t*>(p.states) + static_cast<size_t>(bh) * nch * NST * 256;
  float* const phBase = ROPE ? p.phis + static_cast<size_t>(bh) * nch * J : nullptr;
  const rsrc_t rPh = make_rsrc(ROPE ? static_cast<const void*>(phBase) : static_cast<const void*>(p.dt),
                               ROPE ? static_cast<uint32_t>(nch * J * 4) : 0u);

  auto valid = [&](int c, int r) { return c * Q + (r >> lgR) < L; };
  // Output resources spanning this unit's rows (tokens): an out-of-range
  // offset (kBad) drops a store, so every wave issues the same number of
  // stores every chunk and the wait for a chunk's early loads is not held up
  // by the previous chunk's stores.
  const size_t row0 = (static_cast<size_t>(b) * L * H + hh) * R;  // token 0, rank 0 of this unit
  const uint32_t rowsU = static_cast<uint32_t>((static_cast<size_t>(L - 1) * H + 1) * R);
  const size_t tok0 = static_cast<size_t>(b) * L * H + hh;
  const uint32_t toksU = static_cast<uint32_t>(static_cast<size_t>(L - 1) * H + 1);
  const rsrc_t rdX = make_rsrc(static_cast<bf16_t*>(p.dx) + row0 * P, rowsU * P * 2u);
  const rsrc_t rdB = make_rsrc(static_cast<bf16_t*>(p.dB) + row0 * N, rowsU * N * 2u);
  const rsrc_t rdC = make_rsrc(static_cast<bf16_t*>(p.dC) + row0 * N, rowsU * N * 2u);
  const rsrc_t rDdt = make_rsrc(p.ddt + tok0, toksU * 4u);
  const rsrc_t rDlam = make_rsrc(p.dlam + tok0, toksU * 4u);
  const rsrc_t rDAt = make_rsrc(p.dA_tok != nullptr ? p.dA_tok + tok0 : p.ddt, p.dA_tok != nullptr ? toksU * 4u : 0u);
  const rsrc_t rDth = make_rsrc(ROPE ? p.dtheta + tok0 * J : p.ddt, ROPE ? toksU * J * 4u : 0u);
  // Input resources over the same rows: a row past the end reads zeros, so a
  // load needs no branch and its offset is a short 32-bit sum.
  const rsrc_t rXi = make_rsrc(xg + row0 * P, rowsU * P * 2u);
  const rsrc_t rBi = make_rsrc(Bg + row0 * N, rowsU * N * 2u);
  const rsrc_t rCi = make_rsrc(Cg + row0 * N, rowsU * N * 2u);
  const rsrc_t rDYi = make_rsrc(dYg + row0 * P, rowsU * P * 2u);
  const rsrc_t rDti = make_rsrc(p.dt + tok0, toksU * 4u);
  const rsrc_t rLmi = make_rsrc(p.lam + tok0, toksU * 4u);
  const rsrc_t rAti = make_rsrc(p.A_tok != nullptr ? p.A_tok + tok0 : p.dt, p.A_tok != nullptr ? toksU * 4u : 0u);
  const rsrc_t rThi = make_rsrc(ROPE ? p.theta + tok0 * J : p.dt, ROPE ? toksU * J * 4u : 0u);
  // row of (chunk c, tile row r) relative to row0, and its token's offset in a [Bt, L, H] tensor
  auto rrow = [&](int c, int r) -> uint32_t {
    return static_cast<uint32_t>((c * Q + (r >> lgR)) * H * R + (r & (R - 1)));
  };
  auto toff = [&](int t) -> uint32_t { return static_cast<uint32_t>(t) * static_cast<uint32_t>(H) * 4u; };
  // MFMA operand fragments: rows r0 + l16 of a row-major tile (k along the
  // row), or columns c0 + l16 of a tile whose rows are k (transposing read);
  // both take k = 32 kb + {4g..4g+3, 16+4g..16+4g+3}
  auto frag_row = [&](const uint16_t* base, int pitch, int r0, int kb) __attribute__((always_inline)) {
    const uint16_t* q = base + (r0 + l16) * pitch + 32 * kb + 4 * g;
    return cat8(*reinterpret_cast<const u32x2*>(q), *reinterpret_cast<const u32x2*>(q + 16));
  };
  auto frag_col = [&](const uint16_t* base, int pitch, int c0, int kb) __attribute__((always_inline)) {
    const int rT = 4 * g + (l16 >> 2), c4 = 4 * (l16 & 3);
    return cat8(lds_read_tr(base + (32 * kb + rT) * pitch + c0 + c4),
                lds_read_tr(base + (32 * kb + 16 + rT) * pitch + c0 + c4));
  };
  // per-row scalar of the k rows of a transposing fragment (rows 32kb + 4g..,
  // 32kb + 16 + 4g..), token-indexed table v
  auto krow4 = [&](const float* v, int kb, int half) __attribute__((always_inline)) {
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[(32 * kb + 16 * half + 4 * g + e) >> lgR];
    return o;
  };

  // ---------------------------------------------------------------- set-up
  // zero every tile and partial-sum area: padding rows / columns and the
  // never-written (acausal) tile positions stay zero for the whole kernel
  for (int e = tid; e < static_cast<int>(Lt::kBytes / 4); e += kThreads) reinterpret_cast<float*>(smem)[e] = 0.f;
  __syncthreads();

  // (Tile loads, the state dump and its reread, and the dtheta rows move
  // whole lines once: non-temporal cache policy.)
  // ---- staging of a chunk, split into its global loads (into registers,
  // issued a chunk ahead so that they overlap the previous chunk's products)
  // and the LDS stores that consume them.  Every load is unconditional: an
  // index past the end reads this tensor's first element instead, and the
  // value is zeroed when it is stored, so no wait sits where a load is issued.
  constexpr int UB = (kRows * (N / 8) + kThreads - 1) / kThreads;  // 16-byte units of a B or C tile per thread
  constexpr int UX = (kRows * (P / 8) + kThreads - 1) / kThreads;  // of an x or dy tile
  constexpr int UT = ROPE ? (kRows * J + kThreads - 1) / kThreads : 1;  // theta values (Q J <= 64 J)
  struct Stage {
    u32x4 b[UB], c[UB], x[UX], dy[UX];
    float th[UT];
    float dt, lam, At, dn, ln;  // wave 0, lane = token of the chunk (and the next token)
  };
  auto load_tile = [&](int c, rsrc_t src, auto DD, u32x4* dst) __attribute__((always_inline)) {
    constexpr int D = decltype(DD)::value;
    constexpr int U = (kRows * (D / 8) + kThreads - 1) / kThreads;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int e = tid + i * kThreads;
      const int r = e / (D / 8), k8 = e % (D / 8);
      dst[i] = bload16_nt(src, e < kRows * (D / 8) ? rrow(c, r) * (D * 2u) + 16u * k8 : kBad);
    }
  };
  // per-token scalars of chunk c (wave 0, lane = token): the raw Delta, lambda,
  // A of the chunk's tokens and of the next token (index Q)
  auto load_scalars = [&](int c, Stage& S) __attribute__((always_inline)) {
    // Without the split every wave issues these loads (out-of-range offsets
    // outside wave 0: no request), so that the wait counts are the same in
    // every wave; in the split's launches wave 0 alone issues them (each form
    // measured 2-3% faster where it is used).
    if (MODE != 0 && wave != 0) return;
    const int t = lane;
    const bool mine = wave == 0 && t < Q;
    const uint32_t o0 = mine ? toff(c * Q + t) : kBad, o1 = mine ? toff(c * Q + t + 1) : kBad;
    S.dt = bloadf(rDti, o0);
    S.lam = bloadf(rLmi, o0);
    const float at = bloadf(rAti, o0);
    S.At = p.A_tok != nullptr ? at : Ah;
    S.dn = bloadf(rDti, o1);
    S.ln = bloadf(rLmi, o1);
  };
  auto load_theta = [&](int c, Stage& S) __attribute__((always_inline)) {
    if constexpr (ROPE) {
#pragma unroll
      for (int i = 0; i < UT; ++i) {
        const int e = tid + i * kThreads;
        const int tl = e / J, q = e % J;
        S.th[i] = bloadf(rThi, e < Q * J ? (static_cast<uint32_t>(c * Q + tl) * H * J + q) * 4u : kBad);
      }
    }
  };
  // Lam (log2 units), gamma, delta, E, w and the raw values into the scalar table
  auto store_scalars = [&](int c, const Stage& S) __attribute__((always_inline)) {
    if (wave != 0) return;
    float* const sc = scb(c);
    const int t = lane;
    const bool v0 = t < Q && c * Q + t < L;
    const bool v1 = t < Q && c * Q + t + 1 < L;
    const float dt = v0 ? S.dt : 0.f, lm = v0 ? S.lam : 0.f;
    const float At = v0 ? S.At : 0.f;
    const float dn = v1 ? S.dn : 0.f, ln = v1 ? S.ln : 0.f;
    const float lam2 = seg_scan<64>(dt * At * kLog2e);
    const float lamE = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lam2), Q - 1));
    const float gam = lm * dt;
    const float del = gam + (1.f - ln) * dn;
    sc[kLam2 * kSc + t] = lam2;
    sc[kGam * kSc + t] = gam;
    sc[kDel * kSc + t] = del;
    sc[kE * kSc + t] = __builtin_amdgcn_exp2f(lam2);
    sc[kW * kSc + t] = __builtin_amdgcn_exp2f(lamE - lam2) * del;
    sc[kDt * kSc + t] = dt;
    sc[kLamb * kSc + t] = lm;
    sc[kA * kSc + t] = At;
    if (t == Q - 1) {
      sc[kDt * kSc + Q] = dn;  // the token after the chunk
      sc[kLamb * kSc + Q] = ln;
      sc[kMisc * kSc + 0] = __builtin_amdgcn_exp2f(lamE);  // D
      sc[kMisc * kSc + 1] = lamE;
    }
  };
  // raw theta of chunk c into the angle table (threads q < J then add them up
  // from the carry, reduced modulo 2 pi)
  auto store_theta = [&](int c, const Stage& S) __attribute__((always_inline)) {
    if constexpr (ROPE) {
#pragma unroll
      for (int i = 0; i < UT; ++i) {
        const int e = tid + i * kThreads;
        const int tl = e / J, q = e % J;
        if (e < Q * J) sPhi[tl * JP + q] = c * Q + tl < L ? S.th[i] : 0.f;
      }
    }
  };
  // inclusive scan over aligned segments of Q lanes (Q = 64 / R, 8..64, a
  // runtime power of two): row_shr 1/2/4/8 within rows of 16, then
  // row_bcast 15 / 31 across rows, each step masked to the segment
  auto seg_scan_q = [&](float v) __attribute__((always_inline)) {
    const int sl = lane & (Q - 1);
    float t = dpp<0x111, 0xF, true>(v);
    v += sl >= 1 ? t : 0.f;
    t = dpp<0x112, 0xF, true>(v);
    v += sl >= 2 ? t : 0.f;
    t = dpp<0x114, 0xF, true>(v);
    v += sl >= 4 ? t : 0.f;
    t = dpp<0x118, 0xF, true>(v);
    v += sl >= 8 ? t : 0.f;
    t = dpp<0x142, 0xA, false>(v);
    v += Q >= 32 ? t : 0.f;
    t = dpp<0x143, 0xC, false>(v);
    v += Q >= 64 ? t : 0.f;
    return v;
  };
  // cumulative angles of chunk c in place in the table (after a barrier since
  // its raw theta was stored): lane = token, one segment of Q lanes per pair,
  // the pair's carry in phiC, replaced by the chunk's last angle; every angle
  // reduced modulo 2 pi.  With `dump`, the angle entering the chunk is
  // written to the workspace for the reverse walk.
  auto scan_angles = [&](int c, bool dump) __attribute__((always_inline)) {
    if constexpr (ROPE) {
      const int tl = lane & (Q - 1);
      for (int q0 = wave * R; q0 < J; q0 += kWaves * R) {  // R pairs per wave pass
        const int q = q0 + (lane >> (6 - lgR));
        const bool ok = q < J;
        const float v = seg_scan_q(ok ? sPhi[tl * JP + q] : 0.f);
        const float cin = ok ? phiC[q] : 0.f;
        if (ok) {
          sPhi[tl * JP + q] = wrap_angle(cin + v);
          if (tl == Q - 1) phiC[q] = wrap_angle(cin + v);
        }
        bstoref(rPh, (dump && ok && tl == 0) ? static_cast<uint32_t>(c * J + q) * 4u : kBad, cin);
      }
    }
  };
  // rows of a B / C tile (rotated) or x / dy tile of chunk c into LDS (bf16)
  auto store_bc = [&](int c, const u32x4* src, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int e = tid + i * kThreads;
      if (e >= kRows * (N / 8)) break;
      const int r = e / (N / 8), k8 = e % (N / 8);
      u32x4 v = src[i];  // zeros past the end
      if constexpr (ROPE) {
        const float* ang = sPhi + (r >> lgR) * JP + 4 * k8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a0 = __uint_as_float(v[q] << 16), a1 = __uint_as_float(v[q] & 0xffff0000u);
          const float cs = __cosf(ang[q]), sn = __sinf(ang[q]);
          v[q] = pack_bf16x2(cs * a0 + sn * a1, cs * a1 - sn * a0);
        }
      }
      uint16_t* d = dst + r * PN + 8 * k8;
      *reinterpret_cast<u32x2*>(d) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(d + 4) = u32x2{v[2], v[3]};
    }
  };
  auto store_xp = [&](int c, const u32x4* src, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int e = tid + i * kThreads;
      if (e >= kRows * (P / 8)) break;
      const int r = e / (P / 8), k8 = e % (P / 8);
      const u32x4 v = src[i];  // zeros past the end
      uint16_t* d = dst + r * PP + 8 * k8;
      *reinterpret_cast<u32x2*>(d) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(d + 4) = u32x2{v[2], v[3]};
    }
  };

  // state tiles of this wave: k = wave + 8 m -> (nt, pt); accumulator lane
  // layout [n = 16 nt + 4 g + jj][p = 16 pt + l16]
  f32x4 acc[STW];
  auto tile_ok = [&](int m) { return wave + kWaves * m < NST; };
  auto tile_nt = [&](int m) { return (wave + kWaves * m) / PT; };
  auto tile_pt = [&](int m) { return (wave + kWaves * m) % PT; };
  // this unit's chunk-entry states (bf16, 512 bytes per tile); an absent tile
  // of the last round is a dropped access
  const rsrc_t rSt = make_rsrc(stBase, static_cast<uint32_t>(nch) * NST * 512u);
  auto st_off = [&](int c, int m) -> uint32_t {
    return (NST % kWaves == 0 || tile_ok(m)) ? (static_cast<uint32_t>(c) * NST + wave + kWaves * m) * 512u + lane * 8u
                                              : kBad;
  };
  // carried term u_{-1}[n][p] = sum_r Bprev_rot[r][n] xprev[r][p]
  const bool carry = p.Bprev_rot != nullptr && p.xprev != nullptr;
  auto u_prev = [&](int n, int pc) {
    float u = 0.f;
    if (carry)
      for (int rr = 0; rr < R; ++rr)
        u += p.Bprev_rot[(static_cast<size_t>(bh) * R + rr) * N + n] *
             bf16_to_f32(static_cast<const bf16_t*>(p.xprev)[(static_cast<size_t>(bh) * R + rr) * P + pc].bits);
    return u;
  };
  const size_t o0 = static_cast<size_t>(b) * L * H + hh;  // token 0 of this (batch, head)
  const float kappa = (1.f - p.lam[o0]) * p.dt[o0];       // weight of the carried term

  // this unit's [N][P] slot of a split's fp32 workspace, at the lane's (n, p)
  auto ws_at = [&](const float* base, int m, int jj) {
    return base[static_cast<size_t>(bh) * N * P + static_cast<size_t>(16 * tile_nt(m) + 4 * g + jj) * P +
                16 * tile_pt(m) + l16];
  };
  // which walks this workgroup takes
  const bool doFwd = MODE == 0 || (MODE == 1 && seg == 0) || (MODE == 2 && seg == 1);
  const bool doGsum = MODE == 1 && seg == 1;

  // ================================================================ forward walk (state only)
  // H entering chunk cA: H_{-1} = h0 + kappa u_{-1}, or the state the pre
  // launch left at chunk cm; the pre launch's G sum starts from zero
#pragma unroll
  for (int m = 0; m < STW; ++m) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (tile_ok(m) && doFwd) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = 16 * tile_nt(m) + 4 * g + jj, pc = 16 * tile_pt(m) + l16;
        if (MODE == 2)
          a[jj] = ws_at(p.sH, m, jj);
        else
          a[jj] = (p.h0 != nullptr ? p.h0[static_cast<size_t>(bh) * N * P + static_cast<size_t>(n) * P + pc] : 0.f) +
                  kappa * u_prev(n, pc);
      }
    }
    acc[m] = a;
  }
  if constexpr (ROPE)
    for (int q = tid; q < J; q += kThreads)
      phiC[q] = (MODE == 2 && seg == 1) ? p.sPhiM[static_cast<size_t>(bh) * J + q]
                : (doGsum || p.phi0 == nullptr) ? 0.f
                                                : p.phi0[static_cast<size_t>(bh) * J + q];
  __syncthreads();
  using NC = std::integral_constant<int, N>;
  using PC = std::integral_constant<int, P>;
  // Forward walk: little work per chunk, so two chunks of loads are in
  // flight (register sets S0 and S1 in turn, the loop unrolled by two so that
  // they are indexed statically).
  Stage S0, S1;
  auto load_fwd = [&](int c, Stage& S) __attribute__((always_inline)) {
    load_scalars(c, S);
    load_theta(c, S);
    load_tile(c, rBi, NC{}, S.b);
    load_tile(c, rXi, PC{}, S.x);
  };
  auto fwd_chunk = [&](int c, Stage& S) __attribute__((always_inline)) {
    store_scalars(c, S);
    store_theta(c, S);
    __syncthreads();
    if constexpr (ROPE) {
      scan_angles(c, true);
      __syncthreads();
    }
    store_bc(c, S.b, sBr);
    store_xp(c, S.x, sX);
    // in flight during the next two chunks; issued past the last chunk too
    // (rows past the end read zeros), so that no branch makes the wait counts
    // of the loop conservative
    load_fwd(c + 2, S);
    // the shifted state entering chunk c, in the accumulator layout
#pragma unroll
    for (int m = 0; m < STW; ++m) bstore8_nt(rSt, st_off(c, m), pack4(acc[m]));
    __syncthreads();
    // H <- D H + Btil^T (w X): k = the chunk's 64 rows
    const float* const sc = scb(c);
    const float D = sc[kMisc * kSc];
    const float* w = sc + kW * kSc;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      if (!tile_ok(m)) continue;
      f32x4 a = acc[m] * D;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        a = mma(frag_col(sBr, PN, 16 * tile_nt(m), kb),
                scale8(frag_col(sX, PP, 16 * tile_pt(m), kb), krow4(w, kb, 0), krow4(w, kb, 1)), a);
      acc[m] = a;
    }
    __syncthreads();
  };
  if (doFwd) {
    load_fwd(cA, S0);
    if (cA + 1 < cB) load_fwd(cA + 1, S1);
    for (int c = cA; c < cB; c += 2) {
      fwd_chunk(c, S0);
      if (c + 1 < cB) fwd_chunk(c + 1, S1);
    }
  }

  if constexpr (MODE == 1) {
    if (seg == 0) {
      // the shifted state and the angle entering chunk cm
#pragma unroll
      for (int m = 0; m < STW; ++m)
        if (tile_ok(m))
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            p.sH[static_cast<size_t>(bh) * N * P + static_cast<size_t>(16 * tile_nt(m) + 4 * g + jj) * P +
                 16 * tile_pt(m) + l16] = acc[m][jj];
      if constexpr (ROPE)
        for (int q = tid; q < J; q += kThreads) p.sPhiM[static_cast<size_t>(bh) * J + q] = phiC[q];
      return;
    }
    // ---- segment 1's part of the gradient entering chunk cm, forward in
    // time: G_rel += Dcum Ctil^T (E dY) with the angles counted from chunk
    // cm, Dcum = exp(Lam summed over the earlier chunks of the segment)
    float lsum = 0.f;  // log2 of Dcum
    auto load_gs = [&](int c, Stage& S) __attribute__((always_inline)) {
      load_scalars(c, S);
      load_theta(c, S);
      load_tile(c, rCi, NC{}, S.c);
      load_tile(c, rDYi, PC{}, S.dy);
    };
    auto gs_chunk = [&](int c, Stage& S) __attribute__((always_inline)) {
      store_scalars(c, S);
      store_theta(c, S);
      __syncthreads();
      if constexpr (ROPE) {
        scan_angles(c, false);
        __syncthreads();
      }
      store_bc(c, S.c, sCr);
      store_xp(c, S.dy, sDY);
      if (c + 2 < cB) load_gs(c + 2, S);
      __syncthreads();
      const float dc = __builtin_amdgcn_exp2f(lsum);
      const float* const sc = scb(c);
      const float* E = sc + kE * kSc;
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        if (!tile_ok(m)) continue;
        f32x4 a = acc[m];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          a = mma(frag_col(sCr, PN, 16 * tile_nt(m), kb),
                  scale8(frag_col(sDY, PP, 16 * tile_pt(m), kb), dc * krow4(E, kb, 0), dc * krow4(E, kb, 1)), a);
        acc[m] = a;
      }
      lsum += sc[kMisc * kSc + 1];
      __syncthreads();
    };
    load_gs(cA, S0);
    if (cA + 1 < cB) load_gs(cA + 1, S1);
    for (int c = cA; c < cB; c += 2) {
      gs_chunk(c, S0);
      if (c + 1 < cB) gs_chunk(c + 1, S1);
    }
#pragma unroll
    for (int m = 0; m < STW; ++m)
      if (tile_ok(m))
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          p.sG[static_cast<size_t>(bh) * N * P + static_cast<size_t>(16 * tile_nt(m) + 4 * g + jj) * P +
               16 * tile_pt(m) + l16] = acc[m][jj];
    if (tid == 0) p.sDc[bh] = __builtin_amdgcn_exp2f(lsum);
    return;
  }

  // ================================================================ backward walk
  // dtheta at a chunk start s has a closed form: a common extra rotation of
  // every token from s on changes only the state carried across s, so
  // dtheta_s = <dh_final, J h_final> - <G, J H> per pair, H the shifted state
  // entering the chunk, G its gradient, J the derivative of the pair rotation
  // (J (v0, v1) = (v1, -v0)).  Inside a chunk dtheta is that value at the next
  // chunk start plus a running sum of at most Q tokens' dPhi: no sum over the
  // whole sequence, whose terms would mostly cancel.  Per-pair partial sums of
  // <., J .> (row p reduced over the 16 lanes of a tile) go to sAnc [PT][J].
  float* const sAnc = reinterpret_cast<float*>(sS1);  // free from the G update to the next Gram phase
  auto turn_parts = [&](int m, f32x4 gv, f32x4 hv) __attribute__((always_inline)) {
    const float v0 = seg_scan<16>(gv[0] * hv[1] - gv[1] * hv[0]);
    const float v1 = seg_scan<16>(gv[2] * hv[3] - gv[3] * hv[2]);
    if (l16 == 15) {
      const int q = 8 * tile_nt(m) + 2 * g;
      sAnc[tile_pt(m) * J + q] = v0;
      sAnc[tile_pt(m) * J + q + 1] = v1;
    }
  };
  auto turn_sum = [&](int q) {
    float s = 0.f;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) s += sAnc[pt * J + q];
    return s;
  };
  // G (gradient of the shifted state) starts from dh_final; in the main
  // launch's segment 0, from the gradient entering chunk cm,
  // Rot(Phi) G_rel + Dcum dh_final, with the anchor <G, J H> at chunk cm
#pragma unroll
  for (int m = 0; m < STW; ++m) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    f32x4 hv = acc[m];  // the final state (or the state entering chunk cm)
    if (tile_ok(m)) {
      if (MODE == 2 && seg == 0) {
        const float dcum = p.sDc[bh];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float cs = 1.f, sn = 0.f;
          if constexpr (ROPE) sincosf(p.sPhiM[static_cast<size_t>(bh) * J + 8 * tile_nt(m) + 2 * g + h2], &sn, &cs);
          const float g0 = ws_at(p.sG, m, 2 * h2), g1 = ws_at(p.sG, m, 2 * h2 + 1);
          const float d0 = p.dh_final != nullptr ? ws_at(p.dh_final, m, 2 * h2) : 0.f;
          const float d1 = p.dh_final != nullptr ? ws_at(p.dh_final, m, 2 * h2 + 1) : 0.f;
          a[2 * h2] = cs * g0 + sn * g1 + dcum * d0;
          a[2 * h2 + 1] = cs * g1 - sn * g0 + dcum * d1;
          hv[2 * h2] = ws_at(p.sH, m, 2 * h2);
          hv[2 * h2 + 1] = ws_at(p.sH, m, 2 * h2 + 1);
        }
      } else if (p.dh_final != nullptr) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) a[jj] = ws_at(p.dh_final, m, jj);
      }
    }
    if constexpr (ROPE)
      if (tile_ok(m)) turn_parts(m, a, hv);
    acc[m] = a;
  }
  float Tq = 0.f;                               // <dh_final, J h_final> of pair q (thread 64 + q)
  if constexpr (ROPE) {
    __syncthreads();
    const int q = tid - 64;
    if (q >= 0 && q < J) Tq = turn_sum(q);
  }
  constexpr int kSW = 2;                        // the wave that forms the scalar gradients
  float pendDt = 0.f, pendLam = 0.f;            // first token of the later chunk (wave kSW, lane 0)
  int pendTok = (MODE == 2 && seg == 0) ? cB * Q : -1;  // segment 0: token cm Q's part (to the workspace)
  float dAsum = 0.f;                            // sum of dA over tokens (wave kSW, lane 0)
  // Per-token scalar gradients of chunk c (wave kSW, lane = token), formed
  // during the Gram phase of the chunk before it in the walk (waves 0 and 1
  // compute two Gram tiles there, kSW one), from the chunk's buffers of the
  // scalars, the Gram row / column sums and the per-wave parts; every wave
  // issues the stores, with dropped offsets outside wave kSW.  The pending
  // Delta / lambda term of the later chunk's first token is carried in wave
  // kSW's registers from one call to the next (chunks in reverse order).
  auto scalar_grads = [&](int c) __attribute__((always_inline)) {
    float stDt = 0.f, stLam = 0.f, stA = 0.f, stPdt = 0.f, stPlam = 0.f;
    uint32_t offT = kBad, offA = kBad, offP = kBad;
    if (wave == kSW) {
      const int t = lane;
      const float* const sc = scb(c);
      const float* const sRow = rowb(c);
      const float* const sCol = colb(c);
      const float* const sDp = dpb(c);
      float rlo = 0.f, rdg = 0.f, clo = 0.f, cdd = 0.f, dE = 0.f, dw = 0.f;
      if (t < Q) {
        for (int rr = 0; rr < R; ++rr) {
          const int r = t * R + rr;
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            rlo += sRow[(k4 * 64 + r) * 2 + 0];
            rdg += sRow[(k4 * 64 + r) * 2 + 1];
            clo += sCol[(k4 * 64 + r) * 2 + 0];
            cdd += sCol[(k4 * 64 + r) * 2 + 1];
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) dE += sEp[nt * 64 + r];
#pragma unroll
          for (int pt = 0; pt < PT; ++pt) dw += sWp[pt * 64 + r];
        }
      }
      float dD = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < kWaves; ++w8) dD += sDp[w8];
      const float lam2 = t < Q ? sc[kLam2 * kSc + t] : 0.f;
      const float lamE = sc[kMisc * kSc + 1];
      const float D = sc[kMisc * kSc];
      const float Et = t < Q ? sc[kE * kSc + t] : 0.f, wt = t < Q ? sc[kW * kSc + t] : 0.f;
      const float sdw = wave_sum(dw * wt);
      float dLam = t < Q ? rlo - clo + dE * Et - dw * wt : 0.f;
      if (t == Q - 1) dLam += sdw + dD * D;
      const float ddl = t < Q ? cdd + dw * __builtin_amdgcn_exp2f(lamE - lam2) : 0.f;
      const float dgam = t < Q ? rdg + ddl : 0.f;
      // da_t = sum_{k >= t} dLam_k
      const float incl = seg_scan<64>(dLam);
      const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
      const float da = tot - incl + dLam;
      const float dtv = t < Q ? sc[kDt * kSc + t] : 0.f, lmv = t < Q ? sc[kLamb * kSc + t] : 0.f;
      const float At = t < Q ? sc[kA * kSc + t] : 0.f;
      const float ddlPrev = dpp<0x138, 0xF, true>(ddl);  // lane t - 1 (wave_shr 1)
      float gdt = da * At + dgam * lmv;
      float glam = dgam * dtv;
      if (t >= 1) {  // delta_{t-1} = gamma_{t-1} + (1 - lambda_t) Delta_t
        gdt += ddlPrev * (1.f - lmv);
        glam -= ddlPrev * dtv;
      }
      const float dA = da * dtv;
      const bool v = t < Q && c * Q + t < L;
      stDt = gdt;
      stLam = glam;
      stA = dA;
      if (v && t >= 1) offT = toff(c * Q + t);
      if (v) offA = toff(c * Q + t);
      const float sA = wave_sum(v ? dA : 0.f);
      // the later chunk's first token takes this chunk's last delta term
      const float ddlLast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ddl), Q - 1));
      if (t == 0) {
        if (pendTok >= 0) {
          const float dn = sc[kDt * kSc + Q], ln = sc[kLamb * kSc + Q];
          stPdt = pendDt + ddlLast * (1.f - ln);
          stPlam = pendLam - ddlLast * dn;
          if (MODE == 2 && seg == 0 && c == cB - 1) {
            p.sTok[bh * 2] = stPdt;  // token cm Q: joined with segment 1's part afterwards
            p.sTok[bh * 2 + 1] = stPlam;
          } else {
            offP = toff(pendTok);
          }
        }
        pendDt = gdt;
        pendLam = glam;
        pendTok = c * Q;
        dAsum += sA;
      }
    }
    bstoref(rDdt, offT, stDt);
    bstoref(rDlam, offT, stLam);
    bstoref(rDAt, offA, stA);
    bstoref(rDdt, offP, stPdt);
    bstoref(rDlam, offP, stPlam);
  };
  Stage& S = S0;                                // the reverse walk's loads, one chunk ahead
  u32x2 hsave[STW];                             // the shifted state entering the chunk (bf16)
  u32x2 hpre[STW];                              // the same (bf16), loaded a chunk ahead
  float phPre = 0.f;                            // the angle entering the chunk (tid < J), loaded a chunk ahead
  // The reverse walk's loads of chunk c, issued during chunk c + 1 in four
  // parts spread over its phases (the scalars, angles and state at the Gram
  // phase, C after it, B between the dX and dB / dC products, x and dy after
  // the products): all at one point, every workgroup's requests arrive at once
  // and the issuing waves stall on them.
  auto load_rev_s = [&](int c) __attribute__((always_inline)) {
    load_scalars(c, S);
    load_theta(c, S);
    if constexpr (ROPE) phPre = bloadf(rPh, tid < J ? static_cast<uint32_t>(c * J + tid) * 4u : kBad);
#pragma unroll
    for (int m = 0; m < STW; ++m) hpre[m] = bload8_nt(rSt, st_off(c, m));
  };
  auto load_rev_c = [&](int c) __attribute__((always_inline)) { load_tile(c, rCi, NC{}, S.c); };
  auto load_rev_b = [&](int c) __attribute__((always_inline)) { load_tile(c, rBi, NC{}, S.b); };
  auto load_rev_x = [&](int c) __attribute__((always_inline)) {
    load_tile(c, rXi, PC{}, S.x);
    load_tile(c, rDYi, PC{}, S.dy);
  };
  load_rev_s(cB - 1);
  load_rev_c(cB - 1);
  load_rev_b(cB - 1);
  load_rev_x(cB - 1);
  for (int c = cB - 1; c >= cA; --c) {
    float* const sRow = rowb(c);
    float* const sCol = colb(c);
    float* const sDp = dpb(c);
    const float* const sc = scb(c);
    if constexpr (ROPE) {
      // dtheta at the start of chunk c + 1, from the parts its pass left in sAnc
      const int q = tid - 64;
      if (q >= 0 && q < J) sThC[q] = c < cB - 1 ? Tq - turn_sum(q) : 0.f;
    }
    store_scalars(c, S);
    store_theta(c, S);
    if (ROPE && tid < J) phiC[tid] = phPre;  // the angle entering the chunk (forward walk's dump)
    __syncthreads();
    if constexpr (ROPE) {
      scan_angles(c, false);
      __syncthreads();
    }
    store_bc(c, S.c, sCr);
    store_bc(c, S.b, sBr);
    store_xp(c, S.x, sX);
    store_xp(c, S.dy, sDY);
    {
      // H^T from the forward walk's (bf16) dump and G^T from the accumulators
      // (own tiles); dD = <G, H> from G in fp32 and the bf16 state
      float dd = 0.f;
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        if (!tile_ok(m)) continue;
        const f32x4 hv = unpack4(hpre[m]);
        hsave[m] = hpre[m];
        const int at = (16 * tile_pt(m) + l16) * PN + 16 * tile_nt(m) + 4 * g;
        *reinterpret_cast<u32x2*>(sHT + at) = hpre[m];
        *reinterpret_cast<u32x2*>(sGT + at) = pack4(acc[m]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dd += acc[m][jj] * hv[jj];
      }
      dd = wave_sum(dd);
      if (lane == 0) sDp[wave] = dd;
    }
    __syncthreads();
    // the next chunk's loads are issued in every chunk, the last one too (its
    // chunk c - 1 lies before the walk: the rows read zeros or are unused), so
    // that no branch around them makes the loop's wait counts conservative
    load_rev_s(c - 1);

    // ---- Gram tiles (i tile it >= j tile jt): G1 = C B^T, G2 = dY X^T, masks
    {
      const float* lam2 = sc + kLam2 * kSc;
      const float* del = sc + kDel * kSc;
      const float* gam = sc + kGam * kSc;
      // Tiles 0..7 on waves 0..7, tile 8 on wave 3 and tile 9 on wave 1.  Waves
      // w and w + 4 share a SIMD; with tile 8 on wave 0 the first SIMD ended
      // this phase last (the third SIMD carries the scalar gradients).
      for (int s = 0; s < 2; ++s) {
        const int k = s == 0 ? wave : (wave == 3 ? 8 : (wave == 1 ? 9 : -1));
        if (k < 0) break;
        // causal tiles numbered (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
        const int it = k < 1 ? 0 : (k < 3 ? 1 : (k < 6 ? 2 : 3));
        const int jt = k - it * (it + 1) / 2;
        const int j = 16 * jt + l16, tj = j >> lgR;
        // the mask's per-token scalars, read (unconditionally) before the
        // products so that their latency overlaps them
        const float lamJ = lam2[tj], delJ = del[tj];
        float lamI[4], gamI[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int ti = (16 * it + 4 * g + jj) >> lgR;
          lamI[jj] = lam2[ti];
          gamI[jj] = gam[ti];
        }
        f32x4 g1 = {0.f, 0.f, 0.f, 0.f}, g2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) g1 = mma(frag_row(sCr, PN, 16 * it, kb), frag_row(sBr, PN, 16 * jt, kb), g1);
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) g2 = mma(frag_row(sDY, PP, 16 * it, kb), frag_row(sX, PP, 16 * jt, kb), g2);
        f32x4 s1, s2;
        float colLo = 0.f, colDd = 0.f;
        float rowLo[4], rowDg[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 16 * it + 4 * g + jj, ti = i >> lgR;
          const bool lower = tj < ti, diag = tj == ti;
          const float ex = __builtin_amdgcn_exp2f(lamI[jj] - lamJ);  // selected away above the diagonal
          const float mlo = lower ? ex * delJ : 0.f;
          const float mv = lower ? mlo : (diag ? gamI[jj] : 0.f);
          s1[jj] = mv * g1[jj];
          s2[jj] = mv * g2[jj];
          const float dm = g1[jj] * g2[jj];
          rowLo[jj] = lower ? dm * mlo : 0.f;
          rowDg[jj] = diag ? dm : 0.f;
          colLo += rowLo[jj];
          colDd += lower ? dm * ex : 0.f;
        }
        // S^T rows j, four consecutive i
        *reinterpret_cast<u32x2*>(sS1 + j * PR + 16 * it + 4 * g) = pack4(s1);
        *reinterpret_cast<u32x2*>(sS2 + j * PR + 16 * it + 4 * g) = pack4(s2);
        // row sums over the 16 lanes of a row (j), column sums over the 4 lane groups
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float a = seg_scan<16>(rowLo[jj]), d = seg_scan<16>(rowDg[jj]);
          if (l16 == 15) {
            sRow[(jt * 64 + 16 * it + 4 * g + jj) * 2 + 0] = a;
            sRow[(jt * 64 + 16 * it + 4 * g + jj) * 2 + 1] = d;
          }
        }
        colLo = add_x32(add_x16(colLo));
        colDd = add_x32(add_x16(colDd));
        if (g == 0) {
          sCol[(it * 64 + j) * 2 + 0] = colLo;
          sCol[(it * 64 + j) * 2 + 1] = colDd;
        }
      }
    }
    if (c + 1 < cB) scalar_grads(c + 1);  // the later chunk's, from its buffers
    __syncthreads();
    load_rev_c(c - 1);

    {
      const float* w = sc + kW * kSc;
      const float* E = sc + kE * kSc;
      // The p tile of every dX pass and the n tile of every dB / dC pass of a
      // wave are fixed (PT and NT divide the wave count): their operand
      // fragments are read from LDS once per chunk, not once per pass.
      // (kHoist)
      static_assert(kWaves % PT == 0 && kWaves % NT == 0, "fixed tile per wave");
      const int ptw = wave % PT, ntw = wave % NT;
      bf16x8 fDYp[2], fGTp[NKB], fGn[PKB], fHn[PKB];
      if constexpr (kHoist) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) fDYp[kb] = frag_col(sDY, PP, 16 * ptw, kb);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) fGTp[kb] = frag_row(sGT, PN, 16 * ptw, kb);
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) {
          fGn[kb] = frag_col(sGT, PN, 16 * ntw, kb);
          fHn[kb] = frag_col(sHT, PN, 16 * ntw, kb);
        }
      }
      // (without kHoist: read in each pass, for that pass's tile pt / nt)
      auto fDY = [&](int kb, int pt) __attribute__((always_inline)) {
        if constexpr (kHoist) return fDYp[kb]; else return frag_col(sDY, PP, 16 * pt, kb);
      };
      auto fGTrow = [&](int kb, int pt) __attribute__((always_inline)) {
        if constexpr (kHoist) return fGTp[kb]; else return frag_row(sGT, PN, 16 * pt, kb);
      };
      auto fGTcol = [&](int kb, int nt) __attribute__((always_inline)) {
        if constexpr (kHoist) return fGn[kb]; else return frag_col(sGT, PN, 16 * nt, kb);
      };
      auto fHTcol = [&](int kb, int nt) __attribute__((always_inline)) {
        if constexpr (kHoist) return fHn[kb]; else return frag_col(sHT, PN, 16 * nt, kb);
      };
      // ---- dX^T tiles: [p][j] = (S1^T dY)^T + w_j (B G)^T
      // (compile-time trip counts, fully unrolled: the same stores in every wave)
#pragma unroll
      for (int it = 0; it < (4 * PT + kWaves - 1) / kWaves; ++it) {
        const int k = wave + kWaves * it;
        if ((4 * PT) % kWaves != 0 && k >= 4 * PT) break;
        const int jt = k / PT, pt = k % PT;  // = ptw
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (32 * kb + 31 >= 16 * jt) a1 = mma(fDY(kb, pt), frag_row(sS1, PR, 16 * jt, kb), a1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) a2 = mma(fGTrow(kb, pt), frag_row(sBr, PN, 16 * jt, kb), a2);
        const int j = 16 * jt + l16;
        const float wj = w[j >> lgR];
        const f32x4 dx = a1 + wj * a2;
        bstore8(rdX, valid(c, j) ? (rrow(c, j) * P + 16 * pt + 4 * g) * 2u : kBad, pack4(dx));
        // dw_j part: <(B G)_j, x_j> over this tile's four columns
        const u32x2 xv = *reinterpret_cast<const u32x2*>(sX + j * PP + 16 * pt + 4 * g);
        float s = a2[0] * __uint_as_float(xv[0] << 16) + a2[1] * __uint_as_float(xv[0] & 0xffff0000u) +
                  a2[2] * __uint_as_float(xv[1] << 16) + a2[3] * __uint_as_float(xv[1] & 0xffff0000u);
        s = add_x32(add_x16(s));
        if (g == 0) sWp[pt * 64 + j] = s;
      }
      load_rev_b(c - 1);
      // ---- dB^T and dC^T tiles of the same rows (row tile t, n tile nt)
      // (rolled at N = 128, where unrolling spills)
      constexpr int kUnrollBC = NT >= 8 ? 1 : 4;
#pragma unroll kUnrollBC
      for (int it = 0; it < (4 * NT + kWaves - 1) / kWaves; ++it) {
        const int k = wave + kWaves * it;
        if ((4 * NT) % kWaves != 0 && k >= 4 * NT) break;
        const int t = k / NT, nt = k % NT;  // = ntw
        f32x4 b1 = {0.f, 0.f, 0.f, 0.f}, b2 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f},
              c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (32 * kb + 31 >= 16 * t) b1 = mma(frag_col(sCr, PN, 16 * nt, kb), frag_row(sS2, PR, 16 * t, kb), b1);
          if (32 * kb <= 16 * t + 15) c1 = mma(frag_col(sBr, PN, 16 * nt, kb), frag_col(sS2, PR, 16 * t, kb), c1);
        }
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) {
          b2 = mma(fGTcol(kb, nt), frag_row(sX, PP, 16 * t, kb), b2);
          c2 = mma(fHTcol(kb, nt), frag_row(sDY, PP, 16 * t, kb), c2);
        }
        const int r = 16 * t + l16, tl = r >> lgR;
        f32x4 db = b1 + w[tl] * b2;
        f32x4 dc = c1 + E[tl] * c2;
        // dE_i part: <(dY H^T)_i, Ctil_i> over the four columns
        const u32x2 cv = *reinterpret_cast<const u32x2*>(sCr + r * PN + 16 * nt + 4 * g);
        const float cr[4] = {__uint_as_float(cv[0] << 16), __uint_as_float(cv[0] & 0xffff0000u),
                             __uint_as_float(cv[1] << 16), __uint_as_float(cv[1] & 0xffff0000u)};
        float s = c2[0] * cr[0] + c2[1] * cr[1] + c2[2] * cr[2] + c2[3] * cr[3];
        s = add_x32(add_x16(s));
        if (g == 0) sEp[nt * 64 + r] = s;
        if constexpr (ROPE) {
          // the pair's angle gradient from the rotated tiles (dtheta adds at
          // most a chunk of these to the chunk-start value, so their bf16
          // rounding does not accumulate), then back through the rotation
          const u32x2 bv = *reinterpret_cast<const u32x2*>(sBr + r * PN + 16 * nt + 4 * g);
          const float br[4] = {__uint_as_float(bv[0] << 16), __uint_as_float(bv[0] & 0xffff0000u),
                               __uint_as_float(bv[1] << 16), __uint_as_float(bv[1] & 0xffff0000u)};
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int q = 8 * nt + 2 * g + h2;
            const float ang = sPhi[tl * JP + q];
            const float cs = __cosf(ang), sn = __sinf(ang);
            const float d0 = db[2 * h2], d1 = db[2 * h2 + 1], e0 = dc[2 * h2], e1 = dc[2 * h2 + 1];
            sDPhi[r * JP + q] = d0 * br[2 * h2 + 1] - d1 * br[2 * h2] + e0 * cr[2 * h2 + 1] - e1 * cr[2 * h2];
            db[2 * h2] = cs * d0 - sn * d1;
            db[2 * h2 + 1] = sn * d0 + cs * d1;
            dc[2 * h2] = cs * e0 - sn * e1;
            dc[2 * h2 + 1] = sn * e0 + cs * e1;
          }
        }
        const uint32_t ob = valid(c, r) ? (rrow(c, r) * N + 16 * nt + 4 * g) * 2u : kBad;
        bstore8(rdB, ob, pack4(db));
        bstore8(rdC, ob, pack4(dc));
      }
      // ---- G <- D G + Ctil^T (E dY) on the own tiles (G^T in LDS keeps the old G)
      const float D = sc[kMisc * kSc];
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        if (!tile_ok(m)) continue;
        f32x4 a = acc[m] * D;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)  // tile_pt(m) = ptw
          a = mma(frag_col(sCr, PN, 16 * tile_nt(m), kb), scale8(fDY(kb, tile_pt(m)), krow4(E, kb, 0), krow4(E, kb, 1)), a);
        acc[m] = a;
      }
    }
    __syncthreads();
    if constexpr (ROPE) {
      // parts of <G, J H> for the start of this chunk (read at the next chunk's pass)
#pragma unroll
      for (int m = 0; m < STW; ++m)
        if (tile_ok(m)) turn_parts(m, acc[m], unpack4(hsave[m]));
    }

    load_rev_x(c - 1);

    if constexpr (ROPE) {
      // dtheta_t = dtheta at the next chunk start + dPhi of this chunk's tokens
      // >= t: a segmented scan over the tokens in reverse order (lane tl holds
      // token Q - 1 - tl), one segment of Q lanes per pair, R pairs per wave
      // pass.  The result goes back into the table, in the token's rank-0 row
      // (read above by this lane alone), and leaves as whole rows below.
      const int tl = lane & (Q - 1), tok = Q - 1 - tl;
#pragma unroll
      for (int it = 0; it < (J + kWaves - 1) / kWaves; ++it) {
        const int q = (wave + kWaves * it) * R + (lane >> (6 - lgR));
        if (q < J) {  // the same in every lane of the wave (R divides J)
          float v = 0.f;
          for (int rr = 0; rr < R; ++rr) v += sDPhi[(tok * R + rr) * JP + q];
          v = seg_scan_q(v);
          const float d = sThC[q] + v;
          sDPhi[tok * R * JP + q] = d;
          if (c * Q + tok == cA * Q) sThC[q] = d;  // dtheta of the first token (dphi0), written after the walk
        }
      }
    }
    if constexpr (ROPE) {
      __syncthreads();
      // the chunk's dtheta rows, 16 bytes (four pairs of one token) per lane
      // and a compile-time number of stores per thread; the table is next
      // rewritten in the next chunk's products
      constexpr int kDU = (kRows * (J / 4) + kThreads - 1) / kThreads;
#pragma unroll
      for (int i = 0; i < kDU; ++i) {
        const int u = tid + i * kThreads;
        const bool ok = u < Q * (J / 4);
        const int tok = ok ? u / (J / 4) : 0, q4 = u % (J / 4);
        const float* src = sDPhi + tok * R * JP + 4 * q4;
        const f32x4 v = {src[0], src[1], src[2], src[3]};
        const int t = c * Q + tok;
        bstore16_nt(rDth, (ok && t < L) ? (static_cast<uint32_t>(t) * H * J + 4 * q4) * 4u : kBad,
                 __builtin_bit_cast(u32x4, v));
      }
    }
  }
  scalar_grads(cA);  // every table of chunk cA is complete since the walk's last barrier

  if (MODE == 2 && seg == 1) {
    // segment 1's part of token cm Q's Delta and lambda gradients, its dtheta
    // (the sum of dPhi over the segment) and its sum of dA
    if (tid == kSW * 64) {
      p.sTok[(units + bh) * 2] = pendDt;
      p.sTok[(units + bh) * 2 + 1] = pendLam;
      if (p.dA_part != nullptr) p.dA_part[units + bh] = dAsum;
    }
    if constexpr (ROPE)
      for (int q = tid; q < J; q += kThreads) p.sDth[static_cast<size_t>(bh) * J + q] = sThC[q];
    return;
  }

  // ================================================================ carry-in
  // G is now the gradient of H_{-1} = h0 + kappa u_{-1}
  {
    if constexpr (ROPE)
      if (p.dphi0 != nullptr)
        for (int q = tid; q < J; q += kThreads) p.dphi0[static_cast<size_t>(bh) * J + q] = sThC[q];
    float dk = 0.f;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      if (!tile_ok(m)) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = 16 * tile_nt(m) + 4 * g + jj, pc = 16 * tile_pt(m) + l16;
        if (carry) dk += acc[m][jj] * u_prev(n, pc);
        if (p.dh0 != nullptr) p.dh0[static_cast<size_t>(bh) * N * P + static_cast<size_t>(n) * P + pc] = acc[m][jj];
      }
    }
    dk = wave_sum(dk);
    float* const sDk = dpb(cA + 1);  // not the buffer the last scalar gradients read
    if (lane == 0) sDk[wave] = dk;
    // G in fp32 [N][P] over the (now free) bf16 tile area
    float* sG = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int m = 0; m < STW; ++m)
      if (tile_ok(m))
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sG[(16 * tile_nt(m) + 4 * g + jj) * P + 16 * tile_pt(m) + l16] = acc[m][jj];
    __syncthreads();
    if (tid == kSW * 64) {  // the lane that holds the pending terms and the sum of dA
      float dkap = 0.f;
      for (int w8 = 0; w8 < kWaves; ++w8) dkap += sDk[w8];
      const float dn = p.dt[o0], ln = p.lam[o0];
      if (pendTok == 0) {
        p.ddt[o0] = pendDt + dkap * (1.f - ln);
        p.dlam[o0] = pendLam - dkap * dn;
      }
      if (p.dA_part != nullptr) p.dA_part[bh] = dAsum;
    }
    if (carry) {
      if (p.dBprev_rot != nullptr)
        for (int e = tid; e < R * N; e += kThreads) {
          const int rr = e / N, n = e % N;
          float s = 0.f;
          for (int pc = 0; pc < P; ++pc)
            s += sG[n * P + pc] *
                 bf16_to_f32(static_cast<const bf16_t*>(p.xprev)[(static_cast<size_t>(bh) * R + rr) * P + pc].bits);
          p.dBprev_rot[(static_cast<size_t>(bh) * R + rr) * N + n] = kappa * s;
        }
      if (p.dxprev != nullptr)
        for (int e = tid; e < R * P; e += kThreads) {
          const int rr = e / P, pc = e % P;
          float s = 0.f;
          for (int n = 0; n < N; ++n) s += sG[n * P + pc] * p.Bprev_rot[(static_cast<size_t>(bh) * R + rr) * N + n];
          static_cast<bf16_t*>(p.dxprev)[(static_cast<size_t>(bh) * R + rr) * P + pc].bits = f32_to_bf16(kappa * s);
        }
    }
  }
}

template <int N, int P, bool ROPE, int MODE>
hipError_t launch_t(const BackwardParams& p, hipStream_t s) {
  constexpr size_t lds = Lay<N, P, ROPE>::kBytes;
  if constexpr (lds > 160 * 1024) {
    return hipErrorInvalidValue;
  } else {
    static std::atomic<uint64_t> cleared{0};
    hipError_t e = allow_lds(reinterpret_cast<const void*>(&backward_kernel<N, P, ROPE, MODE>), lds, cleared);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((backward_kernel<N, P, ROPE, MODE>), dim3(p.Bt * p.H, MODE == 0 ? 1 : 2), dim3(kThreads), lds,
                       s, p);
    return hipGetLastError();
  }
}
template <int N, bool ROPE, int MODE>
hipError_t launch_p(const BackwardParams& p, hipStream_t s) {
  switch (p.P) {
    case 16: return launch_t<N, 16, ROPE, MODE>(p, s);
    case 32: return launch_t<N, 32, ROPE, MODE>(p, s);
    case 64: return launch_t<N, 64, ROPE, MODE>(p, s);
    case 128: return launch_t<N, 128, ROPE, MODE>(p, s);
  }
  return hipErrorInvalidValue;
}
template <bool ROPE, int MODE>
hipError_t launch_n(const BackwardParams& p, hipStream_t s) {
  switch (p.N) {
    case 16: return launch_p<16, ROPE, MODE>(p, s);
    case 32: return launch_p<32, ROPE, MODE>(p, s);
    case 64: return launch_p<64, ROPE, MODE>(p, s);
    case 128: return launch_p<128, ROPE, MODE>(p, s);
  }
  return hipErrorInvalidValue;
}
template <int MODE>
hipError_t launch_mode(const BackwardParams& p, hipStream_t s) {
  return p.theta != nullptr ? launch_n<true, MODE>(p, s) : launch_n<false, MODE>(p, s);
}
template <int N>
size_t lds_p(int P, bool rope) {
  switch (P) {
    case 16: return rope ? Lay<N, 16, true>::kBytes : Lay<N, 16, false>::kBytes;
    case 32: return rope ? Lay<N, 32, true>::kBytes : Lay<N, 32, false>::kBytes;
    case 64: return rope ? Lay<N, 64, true>::kBytes : Lay<N, 64, false>::kBytes;
    case 128: return rope ? Lay<N, 128, true>::kBytes : Lay<N, 128, false>::kBytes;
  }
  return 0;
}

}  // namespace bw
}  // namespace m3
