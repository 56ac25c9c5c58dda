// Producer/consumer fused chunked prefill of the Mamba-3 SSM core, bf16 inputs
// (gfx950, CDNA4).
//
// Operation: the exponential-trapezoidal recurrence ("Znakomstvo s Mamba-3"
// (chernovdev.ru), sec. 1, displayed recurrence) with cumulative RoPE on B and
// C (same page, sec. 2) and rank-R MIMO (same page, sec. 3; "La dualita:
// Mamba-2 e Mamba-3" (book.paithon.it), sec. "Mamba-3"), evaluated as the four
// pieces of the chunked scan ("La dualita", sec. "Perche conviene: i tensor
// core").  Chunk algebra (derived by unrolling the recurrence): with chunk-local
// Lam_t = sum_{k=s..t} Delta_k A, gamma_t = lambda_t Delta_t and
// delta_t = gamma_t + (1 - lambda_{t+1}) Delta_{t+1} (Delta_L := 0), and the
// shifted state H' = h_e + (1 - lambda_{e+1}) Delta_{e+1} Btil_e x_e^T:
//   y_t    = sum_{j<=t} M_tj <Ctil_t, Btil_j> x_j + exp(Lam_t) Ctil_t^T H'_prev,
//   M_tj   = exp(Lam_t - Lam_j) delta_j (j < t),  M_tt = gamma_t,
//   H'_new = exp(Lam_e) H'_prev + sum_j exp(Lam_e - Lam_j) delta_j Btil_j x_j^T,
//   H'_{-1} = h0 + (1 - lambda_0) Delta_0 Btil_{-1} x_{-1}^T, h_final = H' at the end.
//
// MI355X design.  Written naively the kernel is issue-bound on the vector ALU
// long before HBM (a wave64 VALU op occupies a SIMD16 for four cycles), so the
// per-chunk VALU work is kept to a few hundred instructions per SIMD:
//   * rank R (hence chunk length Q = 64/R) is a template parameter: token
//     indices are shifts by constants and scans are DPP row operations;
//   * loads and stores use buffer resources spanning one batch item, so the
//     ragged tail and padded columns read as zero and stores past the end are
//     dropped by the hardware range check (no per-element branches);
//   * decays are exp2 of log2-scaled cumulative sums (one v_exp per element);
//     rotations use the hardware sin/cos on angles kept within [-pi, pi] plus
//     one chunk of growth;
//   * off-diagonal mask tiles need no token comparisons.
// One 512-thread workgroup owns one (batch, head).  Waves 0-3 are consumers,
// waves 4-7 producers; one workgroup barrier per chunk hands a double-buffered
// LDS operand slot from producers to consumers:
//   iteration k: consumers compute chunk k from slot k%2; producers build slot
//   (k+1)%2 from registers holding chunk k+1, issue the loads of chunk k+3 (two
//   register sets in flight; one set, i.e. chunk k+2, at N = 128), and scan the
//   decay scalars and angles of chunk k+2.
// Producer wave w owns rows 16w..16w+15 of every chunk.  It loads them as
// 16-byte pieces in the bf16 MFMA A-operand layout, rotates B and C pairwise in
// fp32, stores them row-major for the consumers, and transposes B (scaled by
// w_j = exp(Lam_e - Lam_j) delta_j) and X with MFMA products against an identity
// operand: the 16x16 fp32 result of A x I holds per lane four consecutive rows
// of one column, the k-contiguous operand the token contractions need.  These
// pieces go to LDS in lane-linear order (no bank-conflicted transposes).
// Consumer wave c owns p tiles c, c+4, ...: H' (N x 16 per p tile) lives in its
// MFMA accumulators; it computes G^T = B C^T on its causal tiles, masks it in
// registers and feeds it straight into Y^T += X^T S^T, reads the previous state
// out of its own accumulators (Y^T += diag(exp Lam) H'^T C^T), stores y and
// updates H'.  MFMA k index: a k-block of 32 holds, for lane group g, indices
// {4g..4g+3} and {16+4g..16+4g+3}, matching the accumulator rows of two
// adjacent 16-row tiles, so accumulators feed the next product unchanged.
#pragma once
#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {
namespace pc {

constexpr int kRows = 64;
constexpr int kThreads = 512;
constexpr int kConsumers = 4;
constexpr int kProducers = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kBad = 0x7FFFFFF0u;  // buffer offset past any valid range -> reads 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 cat8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(v);
}
__device__ __forceinline__ u32x2 pack4(f32x4 v) { return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}; }
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float bloadf(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 bloadf4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
template <int CTRL, int ROWMASK, bool BOUND>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xF, BOUND));
}
// Inclusive scan over aligned segments of W lanes (W a power of two, 8..64):
// row_shr 1/2/4/8 within rows of 16, then row_bcast 15 / 31 across rows.
template <int W>
__device__ __forceinline__ float seg_scan(float v) {
  const int sl = threadIdx.x & (W - 1);
  float t;
  t = dpp<0x111, 0xF, true>(v);
  v += (W >= 16 || sl >= 1) ? t : 0.f;
  t = dpp<0x112, 0xF, true>(v);
  v += (W >= 16 || sl >= 2) ? t : 0.f;
  t = dpp<0x114, 0xF, true>(v);
  v += (W >= 16 || sl >= 4) ? t : 0.f;
  if constexpr (W >= 16) v += dpp<0x118, 0xF, true>(v);
  if constexpr (W >= 32) v += dpp<0x142, 0xA, false>(v);
  if constexpr (W >= 64) v += dpp<0x143, 0xC, false>(v);
  return v;
}

template <int N, int P>
struct PcLayout {
  static constexpr int NK = N < 32 ? 32 : N;  // n contraction length (zero padded)
  static constexpr int NKB = NK / 32;         // k blocks over n
  static constexpr int NTH = N / 16;          // state n tiles
  static constexpr int NPT = P / 16;          // p tiles
  static constexpr int PKB = (P + 31) / 32;   // k blocks over p (X pieces)
  static constexpr int UPT = (NPT + kConsumers - 1) / kConsumers;  // p tiles per consumer
  static constexpr int UPW = 2 * NKB + PKB;   // producer pieces per chunk and wave
  static constexpr int PN = NK + 8;           // bf16 pitch of B/C rows (16-byte pad)
  static constexpr int NG = N / 8;            // float4 groups of angles per token
  static constexpr int TSL = (NG + 3) / 4;    // angle groups per producer lane (at Q = 64)
  // LDS (bytes)
  static constexpr size_t kSlotC = size_t(kRows) * PN * 2;
  static constexpr size_t kSlotBwT = size_t(NTH) * 4 * 64 * 8;  // [nt][m][half][lane] x 8 B
  static constexpr size_t kSlotXT = size_t(NPT) * 4 * 64 * 8;   // [pt][m][half][lane] x 8 B
  static constexpr size_t oC = 0;
  static constexpr size_t oB = oC + kSlotC;
  static constexpr size_t oBwT = oB + kSlotC;
  static constexpr size_t oXT = oBwT + kSlotBwT;
  static constexpr size_t kSlot = oXT + kSlotXT;
  static constexpr size_t oSC = 2 * kSlot;                // [3][6][64] fp32 scalars
  static constexpr size_t kSC = 6 * 64 * 4;
  static constexpr size_t oPhiC = oSC + 3 * kSC;          // [N/2] fp32 angle carry
  static constexpr size_t oPhi = oPhiC + (N / 2) * 4;     // [2][64][N/2] fp32 angles
  static constexpr size_t kBytesReal = oPhi;
  static constexpr size_t kBytesRope = oPhi + 2 * size_t(kRows) * (N / 2) * 4;
};

template <int N, int P, int LGR, bool ROPE>
__global__ __launch_bounds__(kThreads) void prefill_pc_kernel(PrefillParams p) {
  using Lt = PcLayout<N, P>;
  constexpr int R = 1 << LGR;
  constexpr int Q = kRows >> LGR;  // tokens per chunk
  constexpr int NKB = Lt::NKB, NTH = Lt::NTH, NPT = Lt::NPT, PKB = Lt::PKB, UPT = Lt::UPT;
  constexpr int UPW = Lt::UPW, PN = Lt::PN, NG = Lt::NG, TSL = Lt::TSL;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int hh = bh % p.H;
  const int L = p.L, H = p.H;
  constexpr bool rope = ROPE;  // theta != nullptr
  const float A2 = p.A[hh] * kLog2e;  // decays in log2 units
  const int nch = (L + Q - 1) / Q;
  const bool consumer = wave < kConsumers;
  const int pw = wave - kConsumers;

  // per-batch-item buffer resources (the range check zero-fills t >= L)
  const size_t tokB = static_cast<size_t>(L) * H;  // (t, h) pairs per batch item
  const rsrc_t rX = make_rsrc(static_cast<const bf16_t*>(p.x) + b * tokB * R * P, uint32_t(tokB * R * P * 2));
  const rsrc_t rB = make_rsrc(static_cast<const bf16_t*>(p.B) + b * tokB * R * N, uint32_t(tokB * R * N * 2));
  const rsrc_t rC = make_rsrc(static_cast<const bf16_t*>(p.C) + b * tokB * R * N, uint32_t(tokB * R * N * 2));
  const rsrc_t rY = make_rsrc(static_cast<bf16_t*>(p.y) + b * tokB * R * P, uint32_t(tokB * R * P * 2));
  const rsrc_t rDt = make_rsrc(p.dt + b * tokB, uint32_t(tokB * 4));
  const rsrc_t rLam = make_rsrc(p.lam + b * tokB, uint32_t(tokB * 4));
  const rsrc_t rTh = make_rsrc(rope ? p.theta + b * tokB * (N / 2) : p.dt, uint32_t(rope ? tokB * (N / 2) * 4 : 0));

  auto slotC = [&](int s) { return reinterpret_cast<uint16_t*>(smem + s * Lt::kSlot + Lt::oC); };
  auto slotB = [&](int s) { return reinterpret_cast<uint16_t*>(smem + s * Lt::kSlot + Lt::oB); };
  auto slotBwT = [&](int s) { return reinterpret_cast<u32x2*>(smem + s * Lt::kSlot + Lt::oBwT); };
  auto slotXT = [&](int s) { return reinterpret_cast<u32x2*>(smem + s * Lt::kSlot + Lt::oXT); };
  auto sc = [&](int s) { return reinterpret_cast<float*>(smem + Lt::oSC + s * Lt::kSC); };
  float* phiC = reinterpret_cast<float*>(smem + Lt::oPhiC);
  auto phiTab = [&](int s) { return reinterpret_cast<float*>(smem + Lt::oPhi) + s * kRows * (N / 2); };

  // ================================================================ producer
  // Register sets of in-flight B/C/X loads (chunk c lives in set c % NSET): two
  // when they fit next to the consumer's state, else one.
  constexpr int NSET = UPW <= 6 ? 2 : 1;
  u32x4 raw[NSET][UPW];
  f32x4 rawTh[2][ROPE ? TSL : 1];
  float rdt[2], rlam[2], rdtn[2], rlamn[2];
  bf16x8 Ilo, Ihi;  // identity selectors: column c <- k slot (g, e) with 8g + e == c (+16)
  {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t one = 0x3F80u << (16 * (e & 1));
      if (8 * g + e == l16) lo[e >> 1] |= one;
      if (8 * g + e == 16 + l16) hi[e >> 1] |= one;
    }
    Ilo = as_bf16x8(lo);
    Ihi = as_bf16x8(hi);
  }
  // producer row of the chunk and its (token offset, rank)
  const int prow = 16 * pw + l16;
  const int ptok = prow >> LGR;
  const int prank = prow & (R - 1);

  // pieces: u < NKB -> B k-block u, u < 2 NKB -> C k-block u - NKB, else X k-block
  auto issue_bcx = [&](int c, u32x4 (&dst)[UPW]) {
    const uint32_t row = static_cast<uint32_t>(((c * Q + ptok) * H + hh) * R + prank);
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const bool isX = u >= 2 * NKB;
      const int kb = isX ? u - 2 * NKB : (u % NKB);
      const int D = isX ? P : N;
      const int col = 32 * kb + 8 * g;
      const uint32_t off = col < D ? (row * D + col) * 2u : kBad;
      dst[u] = bload16(isX ? rX : (u < NKB ? rB : rC), off);
    }
  };
  auto issue_small = [&](int c, int set) {
    if (pw == 0) {
      const uint32_t off = lane < Q ? static_cast<uint32_t>((c * Q + lane) * H + hh) * 4u : kBad;
      rdt[set] = bloadf(rDt, off);
      rlam[set] = bloadf(rLam, off);
      const uint32_t offn = lane < Q ? off + H * 4u : kBad;
      rdtn[set] = bloadf(rDt, offn);
      rlamn[set] = bloadf(rLam, offn);
    }
    if constexpr (ROPE) {
      const int tl = lane % Q, pg = lane / Q;
#pragma unroll
      for (int s = 0; s < TSL; ++s) {
        const int q4 = (s * kProducers + pw) * R + pg;
        const uint32_t off = q4 < NG ? (static_cast<uint32_t>((c * Q + tl) * H + hh) * (N / 2) + 4 * q4) * 4u : kBad;
        rawTh[set][s] = bloadf4(rTh, off);
      }
    }
  };
  // decay scalars (log2 units) and cumulative angles of chunk c -> SC[c%3], Phi[c%2]
  auto stage_small = [&](int c, int set) {
    if (pw == 0) {
      float* S = sc(c % 3);
      const float lamc = seg_scan<64>(rdt[set] * A2);
      const float lamEnd = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lamc), Q - 1));
      const float gam = rlam[set] * rdt[set];
      const float del = gam + (1.f - rlamn[set]) * rdtn[set];
      S[0 * 64 + lane] = lamc;
      S[1 * 64 + lane] = gam;
      S[2 * 64 + lane] = del;
      S[3 * 64 + lane] = __builtin_amdgcn_exp2f(lamEnd - lamc) * del;
      S[4 * 64 + lane] = __builtin_amdgcn_exp2f(lamc);
      if (lane == 0) S[5 * 64] = __builtin_amdgcn_exp2f(lamEnd);
    }
    if constexpr (ROPE) {
      const int tl = lane % Q, pg = lane / Q;
      float* tab = phiTab(c & 1);
#pragma unroll
      for (int s = 0; s < TSL; ++s) {
        const int q4 = (s * kProducers + pw) * R + pg;  // uniform within a Q-lane segment
        if ((s * kProducers + pw) * R < NG) {
          f32x4 v = rawTh[set][s];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = seg_scan<Q>(v[e]);
          if (q4 < NG) {
            const f32x4 cin = *reinterpret_cast<const f32x4*>(phiC + 4 * q4);
            const f32x4 a = v + cin;
            *reinterpret_cast<f32x4*>(tab + tl * (N / 2) + 4 * q4) = a;
            if (tl == Q - 1) {
              f32x4 w;
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = wrap_angle(a[e]);
              *reinterpret_cast<f32x4*>(phiC + 4 * q4) = w;
            }
          }
        }
      }
    }
  };
  // build operand slot c%2 from one register set
  auto build_slot = [&](int c, const u32x4 (&src)[UPW]) {
    const int s = c & 1;
    const bool lastTok = (c * Q + ptok == L - 1);
    const float* S = sc(c % 3);
    f32x4 wj;  // w of the four rows (16pw + 4g + jj) this lane holds after a transpose
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wj[jj] = S[3 * 64 + ((16 * pw + 4 * g + jj) >> LGR)];
    uint16_t* sB = slotB(s);
    uint16_t* sC = slotC(s);
    u32x2* bwt = slotBwT(s);
    u32x2* xt = slotXT(s);
    const float* tab = phiTab(c & 1);
    const int m = pw >> 1, half = pw & 1;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int col = 32 * kb + 8 * g;
      float cs[4], sn[4];
      if constexpr (ROPE) {
        const int q = (N >= 32 || 16 * kb + 4 * g < N / 2) ? 16 * kb + 4 * g : 0;
        const f32x4 a = *reinterpret_cast<const f32x4*>(tab + ptok * (N / 2) + q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sn[e] = __sinf(a[e]);
          cs[e] = __cosf(a[e]);
        }
      }
#pragma unroll
      for (int which = 0; which < 2; ++which) {  // 0: B, 1: C
        const u32x4 v = src[which * NKB + kb];
        u32x4 o = v;
        float f[8];
        if (ROPE || (which == 0 && lastTok)) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
          }
          if constexpr (ROPE) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float a0 = f[2 * q], a1 = f[2 * q + 1];
              f[2 * q] = cs[q] * a0 + sn[q] * a1;
              f[2 * q + 1] = cs[q] * a1 - sn[q] * a0;
              o[q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
            }
          }
        }
        *reinterpret_cast<u32x4*>((which ? sC : sB) + prow * PN + col) = o;
        if (which == 0) {
          if (lastTok && p.Bprev_rot_out != nullptr && col < N) {
            float* dst = p.Bprev_rot_out + (static_cast<size_t>(bh) * R + prank) * N + col;
            store4<float>(dst, f[0], f[1], f[2], f[3]);
            store4<float>(dst + 4, f[4], f[5], f[6], f[7]);
          }
          const bf16x8 a = as_bf16x8(o);
          if (2 * kb < NTH) bwt[(((2 * kb) * 2 + m) * 2 + half) * 64 + lane] = pack4(mma(a, Ilo, z) * wj);
          if (2 * kb + 1 < NTH) bwt[(((2 * kb + 1) * 2 + m) * 2 + half) * 64 + lane] = pack4(mma(a, Ihi, z) * wj);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < PKB; ++kb) {
      const u32x4 v = src[2 * NKB + kb];
      const bf16x8 a = as_bf16x8(v);
      if (2 * kb < NPT) xt[(((2 * kb) * 2 + m) * 2 + half) * 64 + lane] = pack4(mma(a, Ilo, z));
      if (2 * kb + 1 < NPT) xt[(((2 * kb + 1) * 2 + m) * 2 + half) * 64 + lane] = pack4(mma(a, Ihi, z));
      const int col = 32 * kb + 8 * g;
      if (lastTok && p.xprev_out != nullptr && col < P)
        *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(p.xprev_out) + (static_cast<size_t>(bh) * R + prank) * P + col) = v;
    }
  };
  // one producer iteration; `bcx` holds chunk k+1 on entry and chunk k+1+NSET on exit
  auto producer_iter = [&](int k, u32x4 (&bcx)[UPW], int sset) {
    if (k + 1 < nch) build_slot(k + 1, bcx);
    if (k + 1 + NSET < nch) issue_bcx(k + 1 + NSET, bcx);
    if (k + 2 < nch) stage_small(k + 2, sset);
    if (k + 4 < nch) issue_small(k + 4, sset);
  };

  // ================================================================ consumer
  f32x4 acc[UPT][NTH];
  const int cw = wave;
  auto consumer_iter = [&](int k) {
    const int s = k & 1;
    const float* S = sc(k % 3);
    const uint16_t* sB = slotB(s);
    const uint16_t* sC = slotC(s);
    const u32x2* bwt = slotBwT(s);
    const u32x2* xt = slotXT(s);
    const float cdec = S[5 * 64];
    bf16x8 xfr[UPT][2];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int pt = cw + kConsumers * u;
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (pt < NPT) xfr[u][m] = cat8(xt[((pt * 2 + m) * 2 + 0) * 64 + lane], xt[((pt * 2 + m) * 2 + 1) * 64 + lane]);
    }
    // H'^T operand pieces straight from the accumulators (state before chunk k)
    bf16x8 hfr[UPT][NKB];
#pragma unroll
    for (int u = 0; u < UPT; ++u)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        constexpr u32x2 zero2 = {0u, 0u};
        const u32x2 lo = (2 * kb < NTH) ? pack4(acc[u][2 * kb < NTH ? 2 * kb : 0]) : zero2;
        const u32x2 hi = (2 * kb + 1 < NTH) ? pack4(acc[u][2 * kb + 1 < NTH ? 2 * kb + 1 : 0]) : zero2;
        hfr[u][kb] = cat8(lo, hi);
      }
#pragma unroll 1
    for (int it = 0; it < 4; ++it) {
      const int iRow = 16 * it + l16;
      const int ti = iRow >> LGR;
      const float lamI = S[ti], gamI = S[64 + ti], decI = S[4 * 64 + ti];
      bf16x8 cfr[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint16_t* rp = sC + iRow * PN + 32 * kb + 4 * g;
        cfr[kb] = cat8(*reinterpret_cast<const u32x2*>(rp), *reinterpret_cast<const u32x2*>(rp + 16));
      }
      f32x4 yacc[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) yacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto gram = [&](int jt) -> f32x4 {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const uint16_t* rp = sB + (16 * jt + l16) * PN + 32 * kb + 4 * g;
          a = mma(cat8(*reinterpret_cast<const u32x2*>(rp), *reinterpret_cast<const u32x2*>(rp + 16)), cfr[kb], a);
        }
        if (jt < it) {  // every token of tile jt precedes every token of tile it
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int tj = (16 * jt + 4 * g + jj) >> LGR;
            a[jj] *= __builtin_amdgcn_exp2f(lamI - S[tj]) * S[2 * 64 + tj];
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int tj = (16 * jt + 4 * g + jj) >> LGR;
            const float mk = __builtin_amdgcn_exp2f(lamI - S[tj]) * S[2 * 64 + tj];
            a[jj] *= tj < ti ? mk : (tj == ti ? gamI : 0.f);
          }
        }
        return a;
      };
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (2 * m <= it) {
          const f32x4 g0 = gram(2 * m);
          const f32x4 g1 = (2 * m + 1 <= it) ? gram(2 * m + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
          const bf16x8 sop = cat8(pack4(g0), pack4(g1));
#pragma unroll
          for (int u = 0; u < UPT; ++u)
            if (cw + kConsumers * u < NPT) yacc[u] = mma(xfr[u][m], sop, yacc[u]);
        }
      }
      const uint32_t yrow = static_cast<uint32_t>(((k * Q + ti) * H + hh) * R + (iRow & (R - 1))) * P;
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int pt = cw + kConsumers * u;
        if (pt < NPT) {
          f32x4 zz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) zz = mma(hfr[u][kb], cfr[kb], zz);
          const f32x4 yv = yacc[u] + decI * zz;
          bstore8(rY, (yrow + 16 * pt + 4 * g) * 2u, pack4(yv));  // rows past L are dropped
        }
      }
    }
    // H' = exp(Lam_e) H' + (w B)^T X
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (cw + kConsumers * u < NPT) {
#pragma unroll
        for (int nt = 0; nt < NTH; ++nt) {
          f32x4 a = acc[u][nt] * cdec;
#pragma unroll
          for (int m = 0; m < 2; ++m)
            a = mma(cat8(bwt[((nt * 2 + m) * 2 + 0) * 64 + lane], bwt[((nt * 2 + m) * 2 + 1) * 64 + lane]),
                    xfr[u][m], a);
          acc[u][nt] = a;
        }
      }
    }
  };

  // ================================================================ prologue
  if (!consumer) {
    if constexpr (ROPE)
      for (int q = lane + 64 * pw; q < N / 2; q += 64 * kProducers)
        phiC[q] = p.phi0 != nullptr ? p.phi0[static_cast<size_t>(bh) * (N / 2) + q] : 0.f;
    issue_small(0, 0);
    if (nch > 1) issue_small(1, 1);
    issue_bcx(0, raw[0]);
    if (NSET > 1 && nch > 1) issue_bcx(1, raw[NSET - 1]);
  } else {
    // H'_{-1} = h0 + (1 - lambda_0) Delta_0 sum_r Bprev_rot[r] xprev[r]^T
    const size_t o0 = static_cast<size_t>(b) * L * H + hh;
    const float coef = (1.f - p.lam[o0]) * p.dt[o0];
    const bool hasCarry = p.Bprev_rot != nullptr && p.xprev != nullptr;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int pt = cw + kConsumers * u;
#pragma unroll
      for (int nt = 0; nt < NTH; ++nt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (pt < NPT) {
          const int pc = 16 * pt + l16;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int n = 16 * nt + 4 * g + jj;
            float v = p.h0 != nullptr ? p.h0[static_cast<size_t>(bh) * N * P + static_cast<size_t>(n) * P + pc] : 0.f;
            if (hasCarry) {
              float uu = 0.f;
#pragma unroll
              for (int rr = 0; rr < R; ++rr)
                uu += p.Bprev_rot[(static_cast<size_t>(bh) * R + rr) * N + n] *
                      bf16_to_f32(static_cast<const bf16_t*>(p.xprev)[(static_cast<size_t>(bh) * R + rr) * P + pc].bits);
              v += coef * uu;
            }
            a[jj] = v;
          }
        }
        acc[u][nt] = a;
      }
    }
  }
  __syncthreads();  // angle carry visible
  if (!consumer) {
    stage_small(0, 0);
    if (nch > 2) issue_small(2, 0);
  }
  __syncthreads();  // SC(0), Phi(0) visible
  if (!consumer) {
    build_slot(0, raw[0]);
    if (nch > NSET) issue_bcx(NSET, raw[0]);
    if (nch > 1) stage_small(1, 1);
    if (nch > 3) issue_small(3, 1);
  }
  __syncthreads();  // slot 0, SC(1), Phi(1) visible

  // ================================================================ chunk walk, unrolled by two so the
  // register sets are indexed statically
  for (int k = 0; k < nch; k += 2) {
    if (consumer) consumer_iter(k);
    else producer_iter(k, raw[1 % NSET], 0);
    __syncthreads();
    if (k + 1 < nch) {
      if (consumer) consumer_iter(k + 1);
      else producer_iter(k + 1, raw[0], 1);  // (k + 2) % NSET == 0
      __syncthreads();
    }
  }

  // ================================================================ epilogue
  if (consumer) {
    if (p.h_final != nullptr) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int pt = cw + kConsumers * u;
        if (pt < NPT) {
#pragma unroll
          for (int nt = 0; nt < NTH; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              p.h_final[static_cast<size_t>(bh) * N * P + static_cast<size_t>(16 * nt + 4 * g + jj) * P + 16 * pt + l16] =
                  acc[u][nt][jj];
        }
      }
    }
  } else if (ROPE && p.phi_out != nullptr) {
    for (int q = lane + 64 * pw; q < N / 2; q += 64 * kProducers)
      p.phi_out[static_cast<size_t>(bh) * (N / 2) + q] = phiC[q];
  }
}

}  // namespace pc
}  // namespace m3
