// Fused chunked prefill of the Mamba-3 SSM core, bf16 inputs (gfx950, CDNA4).
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
// MI355X design.  One 512-thread workgroup (8 wave64, two per SIMD) owns one
// (segment, batch, head) and walks its chunks of 64 (token, rank) rows with the
// N x P state in MFMA accumulators.  Wave w has a row tile / p-tile group
// quad = w & 3 and a half upper = w >> 2.  Two workgroup barriers per chunk hand
// a double-buffered LDS operand slot over:
//   * phase A -- staging of chunk k+1 into slot (k+1)%2: the two waves of row
//     tile quad own rows 16 quad..+15 and split their loads (whole 128-byte
//     lines, 8 lanes per row, at R = 1; 16-byte pieces in the MFMA operand
//     layout at R > 1), issued one chunk ahead into registers through buffer
//     resources that span the segment of one batch item (the range check
//     zero-fills the ragged tail, so every wave issues the same loads every
//     chunk and the wait counters stay static).  B and C are rotated pairwise
//     in fp32 (hardware sin/cos of the cumulative angle, reduced modulo 2 pi
//     by the angle scan), rounded to bf16 and
//     stored row-major with X, in tiles whose 8-byte units are XOR-swizzled by
//     row.  Wave 0 scans the decays of chunk k+2 (log2 units, one DPP wave
//     scan; with RoPE at R = 1 wave 3 does so in phase B instead); the raw
//     angles of chunk k+2 go to the angle table.  Every wave
//     then computes the readout partials C^T H'_prev of chunk k from the state
//     it keeps.
//   * phase B -- products of chunk k from slot k%2: the angle scan of chunk k+2
//     (DPP segments of Q lanes, carry across chunks), Y^T += X^T S^T for the
//     wave's p tiles quad + 4u and i tiles {0,3} (lower) or {1,2} (upper) from
//     the masked Gram tiles, the readout (own and partner's partials), the y
//     stores (at R = 1 into an LDS tile that leaves as whole rows during the
//     next chunk) and H' = exp(Lam_e) H' + B^T (w X) on the kept n tiles (the
//     two waves of a p tile split the n tiles when the readout exchange
//     fits); then the 10 causal Gram tiles G^T = B C^T of chunk k+1, masked in
//     registers (one exp2 per element, no comparisons off the diagonal), and
//     the X^T fragments of chunk k+1.
// The token contractions need token-contiguous operands: X^T and B^T come
// straight from the row-major tiles through the gfx950 transposing LDS read,
// and w_j = exp(Lam_e - Lam_j) delta_j is applied to the X^T fragments in
// registers, so no transposed copy is ever stored.
// MFMA k index: a k-block of 32 holds, for lane group g, indices {4g..4g+3} and
// {16+4g..16+4g+3}, matching the accumulator rows of two adjacent 16-row tiles,
// so accumulators feed the next product without a trip through LDS.
// Rank R (chunk length Q = 64/R) and RoPE are template parameters: token
// indices are constant shifts, scans are DPP row operations and every tile is
// straight-line code, which keeps the vector-ALU work per chunk small (a wave64
// VALU op occupies a SIMD16 for four cycles).
#pragma once
#include <type_traits>

#include "common.hpp"
#include "m3ssm_internal.hpp"

namespace m3 {
namespace pc {

constexpr int kRows = 64;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kPGroups = 4;  // p tiles are dealt round-robin over wave & 3
constexpr float kLog2e = 1.4426950408889634f;
// Row-major bf16 tiles of D columns (D = 32, 64 or 128) keep their 8-byte
// units XOR-swizzled by row.  Measured on gfx950: an 8-byte read (plain or
// transposing) is served 32 lanes at a time from 64 four-byte banks, a
// 16-byte store 8 lanes at a time on 32 banks.  With r0..r3 the low row bits,
// the swizzle puts r0 ^ r3 (r1 ^ r3 at D = 32) in unit bit 1 and the next row
// bits above it, so that all four access shapes used here are conflict-free:
// 16 rows x 2 units (MFMA operand fragments), 8 aligned rows x 4 units
// (transposing reads), 8 rows x 1 16-byte unit (stores in the MFMA layout) and
// 8 lanes along one row (stores of whole-line pieces).  Row bits that the row
// length already spreads over the banks are left out.
template <int D>
__device__ __forceinline__ int swz_unit(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  if constexpr (D >= 128)
    return ((r0 ^ r3) << 1) | (r1 << 2) | (r2 << 3) | (r0 << 4);
  else if constexpr (D == 64)
    return ((r0 ^ r3) << 1) | (r1 << 2) | (r2 << 3);
  else
    return ((r1 ^ r3) << 1) | (r2 << 2);
}
// element offset of (r, c); c is a multiple of 4 (8 when 16 bytes are accessed)
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return r * D + ((((c >> 2) ^ swz_unit<D>(r))) << 2);
}
// w-scaled copy of an MFMA operand: slots 0-3 by w0, slots 4-7 by w1 (one
// rounding of the product to bf16)
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
// One staging load instruction: instruction i of the unit (16 rows x column
// block cb of B, C or X: kind 0, 1, 2).  Lanes read whole 128-byte lines, 8
// lanes per row (64-byte rows when the block is narrower), so each load asks
// for full lines; half-line loads kept the vector L1 from accepting addresses
// ~40% of the time.
struct Piece {
  int kind, cb, i;
};
// MFMA-layout staging (used at R > 1): a load is 16 rows x 32 columns (k block
// cb), lane (g, l16) reading row l16, 8 columns at 8 g.

// BAL: the balanced whole-line ownership at N = 64 (kernels with the prologue)
template <int N, int P, bool BAL = false>
struct PcLayout {
  static constexpr int NK = N < 32 ? 32 : N;  // n contraction length (zero padded)
  static constexpr int PK = P < 32 ? 32 : P;  // X row length (columns past P unused)
  static constexpr int NKB = NK / 32;         // k blocks over n
  static constexpr int NTH = N / 16;          // state n tiles
  static constexpr int NPT = P / 16;          // p tiles
  static constexpr int PKB = (P + 31) / 32;   // k blocks over p (X pieces)
  static constexpr int UPT = (NPT + kPGroups - 1) / kPGroups;  // p tiles per wave
  static constexpr int NG = N / 8;            // float4 groups of angles per token
  static constexpr int TSL = (NG + kWaves - 1) / kWaves;  // angle groups per lane (Q = 64)
  static constexpr int PH = N / 2 + 4;        // padded angle-table row (spreads banks)
  // staging units: 16-byte chunks per row per load, loads per unit, blocks
  static constexpr int cpr(int D) { return D >= 64 ? 8 : 4; }
  static constexpr int ipu(int D) { return D >= 64 ? 2 : 1; }
  static constexpr int ncb(int D) { return D >= 64 ? D / 64 : 1; }
  static constexpr int NCBN = ncb(N), NCBP = ncb(P);
  // Unit ownership between the two waves of a row tile (whole lines): B and C
  // column blocks by halves of n; X blocks alternate (all to the upper wave
  // when B and C have a single block, all to the lower one when X has a
  // single block).  With the prologue at N = 64 (one column block of two
  // loads) the two waves instead take one load (8 rows) of B, C and X each,
  // so that both normalise and rotate: with B and C whole on the lower wave
  // the RoPE SISO prefill with the prologue ran 7% longer (the plain one
  // measured within noise either way and keeps whole blocks).  With the
  // prologue at N = 128 the lower wave takes whole rows of B and the upper
  // one whole rows of C (and one load of X each): every row's sum of squares
  // is then in one wave, with no exchange through LDS behind a workgroup
  // barrier (SISO real with the prologue 0.189 -> 0.181 ms).  Without the
  // prologue a single X block stays with the lower waves at N = 128 (split by
  // rows too, the SISO real prefill ran 3% longer).
  static constexpr bool kBcByI = BAL && NCBN == 1 && ipu(N) == 2;
  static constexpr bool kByKind = BAL && NCBN == 2;
  static constexpr bool kXByI = (kBcByI || kByKind) && NCBP == 1 && ipu(P) == 2;
  static constexpr int bc_half(int cb, int i) { return NCBN == 1 ? (kBcByI ? i : 0) : (2 * cb) / NCBN; }
  // half of B (kind 0) or C (kind 1) piece (cb, i)
  static constexpr int bck_half(int kind, int cb, int i) { return kByKind ? kind : bc_half(cb, i); }
  static constexpr int x_half(int cb, int i) {
    return kXByI ? i : (NCBN == 1 ? 1 : (NCBP == 1 ? 0 : (cb & 1)));
  }
  static constexpr int count(int h) {
    int n = 0;
    for (int cb = 0; cb < NCBN; ++cb)
      for (int i = 0; i < ipu(N); ++i) n += (bck_half(0, cb, i) == h) + (bck_half(1, cb, i) == h);
    for (int cb = 0; cb < NCBP; ++cb)
      for (int i = 0; i < ipu(P); ++i) n += x_half(cb, i) == h ? 1 : 0;
    return n;
  }
  static constexpr int UPH_FL = count(0) > count(1) ? count(0) : count(1);  // loads per wave
  // load s of half h; B(cb, i) directly precedes C(cb, i) of the same half,
  // which reuses its sin/cos
  static constexpr Piece piece_fl(int h, int s) {
    int n = 0;
    for (int cb = 0; cb < NCBN; ++cb)
      for (int i = 0; i < ipu(N); ++i)
        for (int kind = 0; kind < 2; ++kind)
          if (bck_half(kind, cb, i) == h) {
            if (n == s) return Piece{kind, cb, i};
            n += 1;
          }
    for (int cb = 0; cb < NCBP; ++cb)
      for (int i = 0; i < ipu(P); ++i)
        if (x_half(cb, i) == h) {
          if (n == s) return Piece{2, cb, i};
          n += 1;
        }
    return Piece{-1, 0, 0};
  }
  // MFMA-layout pieces: B/C k block kb -> half (2 kb / NKB); X k block -> alternate
  static constexpr int mf_bc_half(int kb) { return NKB == 1 ? 0 : (2 * kb) / NKB; }
  // With the prologue (R > 1, rows of two or more k blocks): B whole on the
  // lower wave and C whole on the upper one, so that each row's sum of squares
  // stays in one wave (no exchange through LDS behind a workgroup barrier;
  // MIMO with the prologue 0.774 -> 0.745 ms).
  static constexpr bool kByKindMf = BAL && NKB >= 2;
  static constexpr int mf_bck_half(int kind, int kb) { return kByKindMf ? kind : mf_bc_half(kb); }
  static constexpr int mf_x_half(int kb) { return PKB == 1 ? (NKB == 1 ? 1 : 0) : (kb & 1); }
  static constexpr int mf_count(int h) {
    int n = 0;
    for (int kb = 0; kb < NKB; ++kb) n += (mf_bck_half(0, kb) == h) + (mf_bck_half(1, kb) == h);
    for (int kb = 0; kb < PKB; ++kb) n += mf_x_half(kb) == h ? 1 : 0;
    return n;
  }
  static constexpr int UPH_MF = mf_count(0) > mf_count(1) ? mf_count(0) : mf_count(1);
  static constexpr Piece piece_mf(int h, int s) {
    int n = 0;
    for (int kb = 0; kb < NKB; ++kb)
      for (int kind = 0; kind < 2; ++kind)
        if (mf_bck_half(kind, kb) == h) {
          if (n == s) return Piece{kind, kb, 0};
          n += 1;
        }
    for (int kb = 0; kb < PKB; ++kb)
      if (mf_x_half(kb) == h) {
        if (n == s) return Piece{2, kb, 0};
        n += 1;
      }
    return Piece{-1, 0, 0};
  }
  static constexpr int uph(bool fl) { return fl ? UPH_FL : UPH_MF; }
  static constexpr Piece piece(bool fl, int h, int s) { return fl ? piece_fl(h, s) : piece_mf(h, s); }
  // LDS (bytes)
  // slot: C, B (NK columns) and X (PK columns), row-major and swizzled; B and
  // X are also read transposed, which replaces any transposed copy
  static constexpr size_t kSlotC = size_t(kRows) * NK * 2;
  static constexpr size_t kSlotX = size_t(kRows) * PK * 2;
  static constexpr size_t oC = 0;
  static constexpr size_t oB = oC + kSlotC;
  static constexpr size_t oX = oB + kSlotC;
  static constexpr size_t kSlot = oX + kSlotX;
  static constexpr size_t oSC = 2 * kSlot;                // [3][7][64] fp32 scalars
  static constexpr size_t kSC = 7 * 64 * 4;
  static constexpr size_t kSBytes = 10 * 64 * 8;          // [10][64] x 8 B masked S^T pieces
  static constexpr size_t oS = oSC + 3 * kSC;
  static constexpr size_t oPhiC = oS + kSBytes;           // [N/2] fp32 angle carry
  static constexpr size_t oPhi = oPhiC + (N / 2) * 4;     // [2][64][PH] fp32 angles
  static constexpr size_t kBytesReal0 = oPhi;
  static constexpr size_t kBytesRope0 = oPhi + 2 * size_t(kRows) * PH * 4;
  // The two waves of a p tile split the state's n tiles when the exchange of
  // readout partials fits: [wave][u][2][lane] x f32x4.
  static constexpr size_t kLdsMax = 160 * 1024;
  static constexpr size_t kExBytes = size_t(kWaves) * UPT * 2 * 64 * 16;
  static constexpr size_t base(bool rope) { return rope ? kBytesRope0 : kBytesReal0; }
  static constexpr bool split_n(bool rope) { return NTH >= 2 && base(rope) + kExBytes <= kLdsMax; }
  static constexpr size_t oEx(bool rope) { return base(rope); }
  static constexpr size_t used(bool rope) { return base(rope) + (split_n(rope) ? kExBytes : 0); }
  // The Gram tiles of chunk k+1 are computed while chunk k finishes when a
  // second S buffer fits.
  static constexpr bool early_gram(bool rope) { return used(rope) + kSBytes <= kLdsMax; }
  static constexpr size_t oS2(bool rope) { return used(rope); }
  static constexpr size_t used2(bool rope) { return used(rope) + (early_gram(rope) ? kSBytes : 0); }
  // y of one chunk staged as [64][PY] bf16 so that it leaves in whole rows
  static constexpr int PY = P + 8;
  static constexpr size_t kYBytes = size_t(kRows) * PY * 2;
  static constexpr bool stage_y(bool rope) { return used2(rope) + kYBytes <= kLdsMax; }
  static constexpr size_t oY(bool rope) { return used2(rope); }
  static constexpr size_t kBytesReal = used2(false) + (stage_y(false) ? kYBytes : 0);
  static constexpr size_t kBytesRope = used2(true) + (stage_y(true) ? kYBytes : 0);
  // Prologue: the exchange of row sums of squares between the two waves of a
  // row tile [2 halves][2 (B, C)][64 rows], appended only for calls that
  // normalise B and C (gains and biases live in registers).
  static constexpr size_t kProBytes = 4 * 64 * 4;
  static constexpr size_t bytes(bool rope, bool pro) { return (rope ? kBytesRope : kBytesReal) + (pro ? kProBytes : 0); }
  // B and C columns of one row are staged by both waves of a row tile (whole
  // lines at R = 1: column blocks of 64; MFMA layout at R > 1: k blocks of 32)
  static constexpr bool rows_split(bool fl) { return fl ? NCBN > 1 && !kByKind : NKB > 1 && !kByKindMf; }
  static constexpr bool has_bc(bool fl, int h) {
    for (int s = 0; s < uph(fl); ++s) {
      const Piece pc = piece(fl, h, s);
      if (pc.kind == 0 || pc.kind == 1) return true;
    }
    return false;
  }
  // column blocks of B / C staged by half h: the first one and how many
  static constexpr int bc_first(bool fl, int h) {
    for (int s = 0; s < uph(fl); ++s)
      if (piece(fl, h, s).kind == 0 || piece(fl, h, s).kind == 1) return piece(fl, h, s).cb;
    return 0;
  }
  static constexpr int bc_blocks(bool fl, int h) {
    int n = 0, last = -1;
    for (int s = 0; s < uph(fl); ++s) {
      const Piece pc = piece(fl, h, s);
      if ((pc.kind == 0 || pc.kind == 1) && pc.cb != last) {
        ++n;
        last = pc.cb;
      }
    }
    return n;
  }
  static constexpr int bc_blocks_max(bool fl) {
    return bc_blocks(fl, 0) > bc_blocks(fl, 1) ? (bc_blocks(fl, 0) > 0 ? bc_blocks(fl, 0) : 1)
                                               : (bc_blocks(fl, 1) > 0 ? bc_blocks(fl, 1) : 1);
  }
};

// SO (state only): the walk keeps only what the state needs -- no C, no Gram
// tiles, no readout, no y -- and ends with h_final and the carry-out.  It
// produces the state in the middle of a sequence so that the second half can
// run at the same time as the first.
// PRO: the call uses the prologue (B / C normalisation or biases, softplus of
// the step); without it the kernel compiles to the plain core.
template <int N, int P, int LGR, bool ROPE, bool SO = false, bool PRO = false>
__global__ __launch_bounds__(kThreads) void prefill_pc_kernel(PrefillParams p) {
  using Lt = PcLayout<N, P, PRO && !SO>;  // (the state-only walk stages no C)
  constexpr int R = 1 << LGR;
  constexpr int Q = kRows >> LGR;  // tokens per chunk
  constexpr int NKB = Lt::NKB, NTH = Lt::NTH, NPT = Lt::NPT, UPT = Lt::UPT;
  // whole-line staging at R = 1 (the loads there are address-bound),
  // MFMA-layout staging at R > 1 (measured 5% faster at R = 4)
  constexpr bool kFL = LGR == 0;
  constexpr int UPH = Lt::uph(kFL), NG = Lt::NG, TSL = Lt::TSL, PH = Lt::PH;
  constexpr int NK = Lt::NK, PK = Lt::PK;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int quad = wave & 3;             // row tile (staging) and p-tile group (compute)
  const bool upper = (wave >> 2) & 1;    // piece half (staging) and i-tile pair (compute)
  const int units = p.Bt * p.H;
  // Workgroups are dealt to the 8 XCDs in turn; renumber them so that each XCD
  // walks a contiguous range of (segment, batch, head) units.  The heads of one
  // token are adjacent in memory: Delta and lambda of 32 heads share one cache
  // line, which every XCD holding one of those heads fetched again into its own
  // L2 (HBM reads fell from 1.08x to 1.00x the algorithmic bytes, 1-2% faster).
  // The decode step, whose units are whole state blocks, measured 16% slower
  // this way and keeps the plain order.
  int wg = blockIdx.x;
  if ((gridDim.x & 7) == 0) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
  const int seg = wg / units;
  const int bh = wg % units;
  const int b = bh / p.H;
  const int hh = bh % p.H;
  const int H = p.H;
  const int t0 = seg * p.segLen;                                // first token of the segment
  const int L = seg == p.nseg - 1 ? p.L - t0 : p.segLen;       // tokens of the segment
  const bool lastSeg = seg == p.nseg - 1;
  const int nch = (L + Q - 1) / Q;
  // carry-in of this segment
  const float* cH0 = seg == 0 ? p.h0 : p.h_mid;
  const float* cBprev = seg == 0 ? p.Bprev_rot : p.Bprev_mid;
  const void* cXprev = seg == 0 ? p.xprev : p.xprev_mid;
  const float* cPhi0 = seg == 0 ? p.phi0 : p.phi_mid;

  // buffer resources spanning the segment of one batch item: the range check
  // zero-fills tokens past its end (Delta = 0 there: the segment ends like a
  // sequence, and its successor adds the pending term through its carry-in)
  const size_t tok0 = static_cast<size_t>(b) * p.Lfull + t0;  // first (t, h) row / H
  const size_t tokB = static_cast<size_t>(L) * H;              // (t, h) pairs of the segment
  // x, B, C and y are token-major [Bt, L, H, R, .] (consecutive tokens of a
  // head H * R rows apart) or head-major [Bt, H, L, R, .] (R rows apart); the
  // resources start at this unit's first (token, rank) row and end after its
  // last one, so tokens past the segment read zeros and their stores drop
  const int tsR = p.headMajor ? R : H * R;  // rows between consecutive tokens
  const size_t row0 = p.headMajor ? (static_cast<size_t>(bh) * p.Lfull + t0) * R : (tok0 * H + hh) * R;
  const size_t rowsU = static_cast<size_t>(L - 1) * tsR + R;  // rows the segment spans
  const rsrc_t rX = make_rsrc(static_cast<const bf16_t*>(p.x) + row0 * P, uint32_t(rowsU * P * 2));
  const rsrc_t rB = make_rsrc(static_cast<const bf16_t*>(p.B) + row0 * N, uint32_t(rowsU * N * 2));
  const rsrc_t rC = make_rsrc(static_cast<const bf16_t*>(p.C) + row0 * N, uint32_t(SO ? 0 : rowsU * N * 2));
  const rsrc_t rY = make_rsrc(SO ? p.x : static_cast<bf16_t*>(p.y) + row0 * P, uint32_t(SO ? 0 : rowsU * P * 2));
  const rsrc_t rDt = make_rsrc(p.dt + tok0 * H, uint32_t(tokB * 4));
  const rsrc_t rLam = make_rsrc(p.lam + tok0 * H, uint32_t(tokB * 4));
  // A per token (null: the head's A for every token)
  const bool aTok = p.A_tok != nullptr;
  const rsrc_t rAtok = make_rsrc(aTok ? p.A_tok + tok0 * H : p.dt, uint32_t(aTok ? tokB * 4 : 0));
  const float A2 = aTok ? 0.f : p.A[hh] * kLog2e;  // decays in log2 units
  // steps fused in front of the core: B / C normalisation and head biases
  // (applied while staging), Delta = softplus(raw + bias) (in the decay scan)
  const bool proNorm = PRO && p.pro.bc_norm != 0;
  const bool proBC = PRO && (proNorm || p.pro.B_bias != nullptr || p.pro.C_bias != nullptr);
  const bool proDt = PRO && p.pro.dt_softplus != 0;
  const float dtBias = proDt && p.pro.dt_bias != nullptr ? p.pro.dt_bias[hh] : 0.f;
  const float proEps = p.pro.eps;
  // angles: theta [.., H, N/2] per (token, head), or omega [.., N/2] per token
  // (shared by the heads; scaled by Delta in the angle scan)
  const bool om = ROPE && p.omega != nullptr;
  const int thTok = om ? N / 2 : H * (N / 2);  // floats per token
  const int thHead = om ? 0 : hh * (N / 2);
  const rsrc_t rTh = make_rsrc(!ROPE ? p.dt : (om ? p.omega + (static_cast<size_t>(b) * p.Lfull + t0) * (N / 2)
                                                   : p.theta + tok0 * H * (N / 2)),
                               uint32_t(ROPE ? static_cast<size_t>(L) * thTok * 4 : 0));

  auto slotC = [&](int s) __attribute__((always_inline)) { return reinterpret_cast<uint16_t*>(smem + s * Lt::kSlot + Lt::oC); };
  auto slotB = [&](int s) __attribute__((always_inline)) { return reinterpret_cast<uint16_t*>(smem + s * Lt::kSlot + Lt::oB); };
  auto slotX = [&](int s) __attribute__((always_inline)) { return reinterpret_cast<uint16_t*>(smem + s * Lt::kSlot + Lt::oX); };
  auto sc = [&](int s) __attribute__((always_inline)) { return reinterpret_cast<float*>(smem + Lt::oSC + s * Lt::kSC); };
  float* phiC = reinterpret_cast<float*>(smem + Lt::oPhiC);
  // y leaves through LDS in whole rows at R = 1 (fewer, full-line stores:
  // measured ~2% faster); at R > 1 the direct fragment stores are faster
  constexpr bool kStageY = !SO && LGR == 0 && Lt::stage_y(ROPE);
  u32x2* sY = reinterpret_cast<u32x2*>(smem + Lt::oY(ROPE));  // [64][PY/4] 8-byte units
  auto phiTab = [&](int s) __attribute__((always_inline)) { return reinterpret_cast<float*>(smem + Lt::oPhi) + s * kRows * PH; };
  // row sums of squares exchanged by the two waves of a row tile [2][2][64]
  // (allocated only when the call normalises B and C)
  float* const proEx = reinterpret_cast<float*>(smem + (ROPE ? Lt::kBytesRope : Lt::kBytesReal));

  // ================================================================ staging state
  // chunk c's pieces live in register set c % 2 (two chunks in flight)
  // Piece registers: loads run kSets chunks ahead.  One chunk (~3 us) covers
  // the memory latency; two sets kept ~1300 cache-line requests in flight per
  // CU and stalled the load issue of the later waves (measured 2-5% slower).
  constexpr int kSets = 1;
  // Decay scan placement.  With RoPE at R = 1 it runs in phase B on wave 3,
  // which computes one masked Gram tile there (waves 0 and 1 compute two) and
  // refills nothing; the staging phase, where every wave waits for the
  // slowest, then carries only the raw angles (and Delta, for angles given as
  // rates).  Measured 3-5% faster on the RoPE SISO workloads; on the real and
  // the R > 1 workloads phase B is the longer phase and the scan stays on
  // wave 0 in phase A (moved, they ran 1-9% slower).
  constexpr bool kDecayInB = ROPE && LGR == 0;
  constexpr int kScanWave = kDecayInB ? 3 : 0;
  u32x4 raw[kSets][UPH];
  // theta of one chunk as whole token rows: float4 unit e = token e / NG, group e % NG
  constexpr int kThUnits = Q * NG;
  constexpr int kThU = (kThUnits + kThreads - 1) / kThreads;
  f32x4 rawTh[2][ROPE ? kThU : 1];
  float rdt[2], rlam[2], rAt[2] = {0.f, 0.f};
  // Every wave issues the same loads every chunk (chunks past the end read
  // zeros): with no load behind a branch the wait counters stay exact.
  // row (within the chunk) and column of this lane's 16 bytes in load s
  auto piece_rc = [&](const Piece pc, int& row, int& col) __attribute__((always_inline)) {
    if constexpr (kFL) {
      const int D = pc.kind == 2 ? P : N;
      const int cpr = Lt::cpr(D);
      row = 16 * quad + (64 / cpr) * pc.i + lane / cpr;
      col = 64 * pc.cb + 8 * (lane % cpr);
    } else {
      row = 16 * quad + l16;
      col = 32 * pc.cb + 8 * g;
    }
  };
  auto load_piece = [&](int c, int s, auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    const Piece pc = Lt::piece(kFL, h, s);
    if (pc.kind < 0 || (SO && pc.kind == 1)) return u32x4{0u, 0u, 0u, 0u};  // no load (unrolled away)
    const int D = pc.kind == 2 ? P : N;
    int row, col;
    piece_rc(pc, row, col);
    const uint32_t grow = static_cast<uint32_t>((c * Q + (row >> LGR)) * tsR + (row & (R - 1)));
    const uint32_t off = col < D ? (grow * D + col) * 2u : kBad;
    // whole-line loads stream with the non-temporal policy (7% off the SISO
    // real workload); the half-line loads of the MFMA layout need the L2 to
    // keep each line for its other half (with the policy: +25% at R = 4)
    const rsrc_t rs = pc.kind == 2 ? rX : (pc.kind == 1 ? rC : rB);
    if constexpr (kFL) return bload16_nt(rs, off); else return bload16(rs, off);
  };
  constexpr bool kLateRefill = LGR == 0;
  auto issue_bcx = [&](int c, u32x4 (&dst)[UPH], auto HALF) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < UPH; ++s) dst[s] = load_piece(c, s, HALF);
  };
  auto issue_small = [&](int c, int set) __attribute__((always_inline)) {
    // Delta and lambda feed only the decay scan of wave 0.  The other waves
    // issue the same instructions with an out-of-range offset: no memory
    // request (one strided scalar per lane is one cache-line lookup per lane)
    // and identical wait counts everywhere.
    const uint32_t off = (wave == kScanWave && lane < Q) ? static_cast<uint32_t>((c * Q + lane) * H + hh) * 4u : kBad;
    rdt[set] = bloadf(rDt, off);
    rlam[set] = bloadf(rLam, off);
    rAt[set] = bloadf(rAtok, off);  // an empty range without A_tok: reads 0, no request
    if constexpr (ROPE) {  // consecutive lanes read consecutive 16 bytes of a token's row
#pragma unroll
      for (int s = 0; s < kThU; ++s) {
        const int e = tid + s * kThreads;
        const int tok = e / NG, grp = e % NG;
        const uint32_t off4 =
            e < kThUnits ? (static_cast<uint32_t>((c * Q + tok) * thTok + thHead) + 4 * grp) * 4u : kBad;
        rawTh[set][s] = bloadf4(rTh, off4);
      }
    }
  };
  // decay scalars (log2 units) of chunk c -> SC[c%3] (the scan wave)
  auto stage_decay = [&](int c, int set) __attribute__((always_inline)) {
    if (wave == kScanWave) {
      float* S = sc(c % 3);
      // Delta (softplus of raw + bias with the prologue; tokens past the end
      // have Delta = 0, which the zero-filled loads give without it)
      const float dl = delta_of(rdt[set], proDt, dtBias, lane < Q && c * Q + lane < L);
      const float lamc = seg_scan<64>(dl * (aTok ? rAt[set] * kLog2e : A2));
      const float lamEnd = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lamc), Q - 1));
      // next token's Delta, lambda: lane t + 1, or token 0 of chunk c + 1 (the
      // other register set; zeros past the end, i.e. Delta_L = 0) for t = Q - 1
      const float dNext = dpp<0x130, 0xF, true>(dl), lNext = dpp<0x130, 0xF, true>(rlam[set]);  // lane t + 1 (wave_shl 1)
      const float d0 = delta_of(
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rdt[set ^ 1]), 0)), proDt, dtBias,
          (c + 1) * Q < L);
      const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rlam[set ^ 1]), 0));
      const float gam = rlam[set] * dl;
      const float del = gam + (1.f - (lane == Q - 1 ? l0 : lNext)) * (lane == Q - 1 ? d0 : dNext);
      S[0 * 64 + lane] = lamc;
      S[1 * 64 + lane] = gam;
      S[2 * 64 + lane] = del;
      S[3 * 64 + lane] = __builtin_amdgcn_exp2f(lamEnd - lamc) * del;
      S[4 * 64 + lane] = __builtin_amdgcn_exp2f(lamc);
      if (lane == 0) S[5 * 64] = __builtin_amdgcn_exp2f(lamEnd);
      if constexpr (!kDecayInB) S[6 * 64 + lane] = dl;  // Delta, for angles given as rates (else stage_dt)
    }
  };
  // Delta of chunk c alone -> SC[c%3] (for the angle scan of rates)
  auto stage_dt = [&](int c, int set) __attribute__((always_inline)) {
    if (wave == kScanWave)
      sc(c % 3)[6 * 64 + lane] = delta_of(rdt[set], proDt, dtBias, lane < Q && c * Q + lane < L);
  };
  // raw theta of chunk c -> Phi[c%2] (every thread)
  auto stage_theta = [&](int c, int set) __attribute__((always_inline)) {
    if constexpr (ROPE) {
      float* tab = phiTab(c & 1);
#pragma unroll
      for (int s = 0; s < kThU; ++s) {
        const int e = tid + s * kThreads;
        if (e < kThUnits) *reinterpret_cast<f32x4*>(tab + (e / NG) * PH + 4 * (e % NG)) = rawTh[set][s];
      }
    }
  };
  auto stage_small = [&](int c, int set) __attribute__((always_inline)) {
    if constexpr (kDecayInB)
      if (om) stage_dt(c, set);
    stage_decay(c, set);
    stage_theta(c, set);
  };
  // cumulative angles of chunk c in place in Phi[c%2] (after a barrier since
  // its raw theta was stored): lanes are tokens, a segment of Q lanes per
  // group of four angles, carry across chunks in phiC
  auto scan_angles = [&](int c) __attribute__((always_inline)) {
    if constexpr (ROPE) {
      const int tl = lane % Q, pg = lane / Q;
      float* tab = phiTab(c & 1);
      const float dsc = om ? sc(c % 3)[6 * 64 + tl] : 1.f;  // theta = Delta * omega (exact x 1 otherwise)
      // Scan slots dealt from wave 2 on: with fewer angle groups than waves
      // (R > 1) the work falls on waves 2, 3, ..., not on waves 0 and 1,
      // which compute two masked Gram tiles in the same phase.
      const int sw = (wave + kWaves - 2) & (kWaves - 1);
#pragma unroll
      for (int s = 0; s < TSL; ++s) {
        const int q4 = (s * kWaves + sw) * R + pg;  // uniform within a Q-lane segment
        if ((s * kWaves + sw) * R < NG) {
          constexpr f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
          f32x4 v = q4 < NG ? *reinterpret_cast<const f32x4*>(tab + tl * PH + 4 * q4) : zero4;
          v *= dsc;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = seg_scan<Q>(v[e]);
          if (q4 < NG) {
            // reduced modulo 2 pi: the hardware sin/cos that rotate B and C
            // are accurate only for small arguments, and the running sum of a
            // chunk can reach any size
            const f32x4 cin = *reinterpret_cast<const f32x4*>(phiC + 4 * q4);
            const f32x4 a = v + cin;
            f32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = wrap_angle(a[e]);
            *reinterpret_cast<f32x4*>(tab + tl * PH + 4 * q4) = w;
            if (tl == Q - 1) *reinterpret_cast<f32x4*>(phiC + 4 * q4) = w;
          }
        }
      }
    }
  };
  // raw X row piece (8 columns) -> X rows
  auto store_x = [&](int s2, int row, int col, u32x4 v) __attribute__((always_inline)) {
    if (col < P) *reinterpret_cast<u32x4*>(slotX(s2) + swz<PK>(row, col)) = v;
  };
  // stage this wave's pieces of chunk c into operand slot c%2; each register
  // is refilled with the same piece of chunk c+1 as soon as it is consumed,
  // which spreads the load issue over the staging work.  At R = 1 the upper
  // waves refill in the second phase instead: the loads of a chunk then do not
  // all queue at its start (measured 3-5% faster).
  // ---------------------------------------------------------------- prologue of B, C
  // sum of squares of the 8 bf16 values of one staging piece
  auto sumsq8 = [](u32x4 v) __attribute__((always_inline)) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = __uint_as_float(v[q] << 16), a1 = __uint_as_float(v[q] & 0xffff0000u);
      a += a0 * a0 + a1 * a1;
    }
    return a;
  };
  // Row sums of squares -> 1 / RMS of the B (k = 0) and C (k = 1) rows that
  // this lane stages: the lanes of one row add their pieces, and where the two
  // waves of a row tile hold different columns of a row they swap their sums
  // through LDS (behind a workgroup barrier: both halves call this).
  // `rowOf(s)` is the row index slot of piece s (0 .. NRS-1), `row(slot)` its row.
  auto row_scales = [&](const u32x4 (&src)[UPH], auto HALF, auto NRS_, auto rowOf, auto rowAt, auto reduce,
                        float (&rsc)[2][decltype(NRS_)::value]) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    constexpr int NRS = decltype(NRS_)::value;
    float ss[2][NRS];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < NRS; ++i) ss[k][i] = 0.f;
    if constexpr (Lt::has_bc(kFL, h)) {
#pragma unroll
      for (int s = 0; s < UPH; ++s) {
        const Piece pc = Lt::piece(kFL, h, s);
        if (pc.kind == 0 || (pc.kind == 1 && !SO)) ss[pc.kind][rowOf(pc)] += sumsq8(src[s]);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < NRS; ++i) ss[k][i] = reduce(ss[k][i]);
    }
    if constexpr (Lt::rows_split(kFL)) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < NRS; ++i) proEx[(h * 2 + k) * 64 + rowAt(i)] = ss[k][i];  // same value on a row's lanes
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int i = 0; i < NRS; ++i) ss[k][i] += proEx[((1 - h) * 2 + k) * 64 + rowAt(i)];
    }
    // a row of zeros (tokens past the end) stays zero: a finite scale
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < NRS; ++i) rsc[k][i] = ss[k][i] > 0.f ? rsqrtf(ss[k][i] * (1.f / N) + proEps) : 0.f;
  };
  // Gains and biases of the B / C columns this lane stages: the same in every
  // chunk (one column block per half with whole lines at R = 1; the half's k
  // blocks and the lane's rank in the MFMA layout), so they stay in registers:
  // pw = gain (1 without the normalisation), pb = bias (0 without it; 0 in
  // columns past N as well, which must stay zero).
  constexpr int NBH = Lt::bc_blocks_max(kFL);
  float pw[2][NBH][8], pb[2][NBH][8];
  auto load_pro = [&](auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    const int r = kFL ? 0 : ((16 * quad + l16) & (R - 1));
#pragma unroll
    for (int j = 0; j < NBH; ++j) {
      const int cb = Lt::bc_first(kFL, h) + j;
      const int col = kFL ? 64 * cb + 8 * (lane % Lt::cpr(N)) : 32 * cb + 8 * g;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float* w = k == 0 ? p.pro.B_w : p.pro.C_w;
        const float* b = k == 0 ? p.pro.B_bias : p.pro.C_bias;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool in = col + e < N && j < Lt::bc_blocks(kFL, h);
          pw[k][j][e] = (proNorm && w != nullptr && in) ? w[col + e] : 1.f;
          pb[k][j][e] = (b != nullptr && in) ? b[(static_cast<size_t>(hh) * R + r) * N + col + e] : 0.f;
        }
      }
    }
  };
  // bf16 piece -> 8 fp32 values; B / C pieces (kind < 2) of column block j
  // get gain x scale and bias (one fma each)
  auto unpack_pro = [&](u32x4 v, int kind, int j, float scale, float (&f)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = __uint_as_float(v[q] << 16);
      f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
    }
    if constexpr (PRO) {
      if (kind < 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] * (scale * pw[kind][j][e]) + pb[kind][j][e];
      }
    }
  };
  // rotate 4 pairs of fp32 values and round them to bf16
  auto rotate_pack = [](const float (&f)[8], const float (&cs)[4], const float (&sn)[4]) __attribute__((always_inline)) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = f[2 * q], a1 = f[2 * q + 1];
      o[q] = ROPE ? pack_bf16x2(cs[q] * a0 + sn[q] * a1, cs[q] * a1 - sn[q] * a0) : pack_bf16x2(a0, a1);
    }
    return o;
  };
  auto build_slot_fl = [&](int c, u32x4 (&src)[UPH], auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    constexpr bool kRefill = !(kLateRefill && h == 1);
    const int s2 = c & 1;
    uint16_t* sB = slotB(s2);
    uint16_t* sC = slotC(s2);
    const float* tab = phiTab(c & 1);
    // whole-line pieces: piece i of a unit covers rows 16 quad + (64 / cpr) i + lane / cpr
    constexpr int cprN = Lt::cpr(N), IPN = Lt::ipu(N);
    float rsc[2][IPN];
    if (proNorm)
      row_scales(src, HALF, std::integral_constant<int, IPN>{}, [](const Piece pc) { return pc.i; },
                 [&](int i) { return 16 * quad + (64 / cprN) * i + lane / cprN; },
                 [](float v) {  // the cpr (4 or 8) aligned lanes of a row, by DPP
                   v += dpp<0xB1, 0xF, false>(v);  // quad_perm [1,0,3,2]
                   v += dpp<0x4E, 0xF, false>(v);  // quad_perm [2,3,0,1]
                   if constexpr (cprN == 8) v += dpp<0x141, 0xF, false>(v);  // row_half_mirror
                   return v;
                 },
                 rsc);
    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < UPH; ++s) {
      const Piece pc = Lt::piece(kFL, h, s);
      if (pc.kind < 0 || (SO && pc.kind == 1)) continue;  // unrolled away
      const u32x4 v = src[s];
      int row, col;
      piece_rc(pc, row, col);
      if (pc.kind == 2) {
        store_x(s2, row, col, v);
      } else {
        if constexpr (ROPE) {
          // B precedes C of the same rows and columns: C reuses sin/cos (with
          // B and C on different waves, each computes its own)
          if (pc.kind == 0 || Lt::kByKind) {
            const int q = col < N ? (col >> 1) : 0;
            const f32x4 a = *reinterpret_cast<const f32x4*>(tab + (row >> LGR) * PH + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sn[e] = __sinf(a[e]);
              cs[e] = __cosf(a[e]);
            }
          }
        }
        float f[8];
        unpack_pro(v, pc.kind, pc.cb - Lt::bc_first(kFL, h), proNorm ? rsc[pc.kind][pc.i] : 1.f, f);
        // B and C feed the Gram tiles and the readout, B also the state
        *reinterpret_cast<u32x4*>((pc.kind == 1 ? sC : sB) + swz<NK>(row, col)) = rotate_pack(f, cs, sn);
      }
      if constexpr (kRefill) src[s] = load_piece(c + kSets, s, HALF);
    }
  };
  auto build_slot_mf = [&](int c, u32x4 (&src)[UPH], auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    constexpr bool kRefill = !(kLateRefill && h == 1);
    const int s2 = c & 1;
    uint16_t* sB = slotB(s2);
    uint16_t* sC = slotC(s2);
    const float* tab = phiTab(c & 1);
    // MFMA-layout pieces: every piece of this lane is row 16 quad + l16 (k blocks
    // differ); the four lanes g of a row hold its columns 8 g .. of a k block
    float rsc[2][1];
    if (proNorm)
      row_scales(src, HALF, std::integral_constant<int, 1>{}, [](const Piece) { return 0; },
                 [&](int) { return 16 * quad + l16; },
                 [](float v) {
                   return add_x32(add_x16(v));
                 },
                 rsc);
    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < UPH; ++s) {
      const Piece pc = Lt::piece(kFL, h, s);
      if (pc.kind < 0) {  // padding slot of the smaller half: keep the load count uniform
        if constexpr (kRefill) src[s] = load_piece(c + kSets, s, HALF);
        continue;
      }
      const u32x4 v = src[s];
      const int col = 32 * pc.cb + 8 * g;
      if (pc.kind == 2) {
        store_x(s2, 16 * quad + l16, col, v);
        if constexpr (kRefill) src[s] = load_piece(c + kSets, s, HALF);
        continue;
      }
      if (SO && pc.kind == 1) {  // C is not needed for the state
        if constexpr (kRefill) src[s] = load_piece(c + kSets, s, HALF);
        continue;
      }
      if constexpr (ROPE) {
        if (pc.kind == 0 || Lt::kByKindMf) {  // B comes first for a k-block; C reuses its sin/cos (same wave)
          const int q = (N >= 32 || 16 * pc.cb + 4 * g < N / 2) ? 16 * pc.cb + 4 * g : 0;
          const f32x4 a = *reinterpret_cast<const f32x4*>(tab + ((16 * quad + l16) >> LGR) * PH + q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sn[e] = __sinf(a[e]);
            cs[e] = __cosf(a[e]);
          }
        }
      }
      float f[8];
      unpack_pro(v, pc.kind, pc.cb - Lt::bc_first(kFL, h), proNorm ? rsc[pc.kind][0] : 1.f, f);
      // B and C feed the Gram tiles and the readout, B also the state
      *reinterpret_cast<u32x4*>((pc.kind == 1 ? sC : sB) + swz<NK>(16 * quad + l16, col)) = rotate_pack(f, cs, sn);
      if constexpr (kRefill) src[s] = load_piece(c + kSets, s, HALF);
    }
  };
  auto build_slot = [&](int c, u32x4 (&src)[UPH], auto HALF) __attribute__((always_inline)) {
    if constexpr (kFL)
      build_slot_fl(c, src, HALF);
    else
      build_slot_mf(c, src, HALF);
  };
  // ================================================================ compute state
  // The state H' (N x P) lives in MFMA accumulators: wave (quad, upper) keeps p
  // tiles quad + 4u and, when the pair splits n, n tiles [NTW upper, NTW upper + NTW).
  constexpr bool kSplit = Lt::split_n(ROPE);
  constexpr int NTW = kSplit ? NTH / 2 : NTH;  // n tiles kept per wave
  constexpr int NKW = NTW >= 2 ? NTW / 2 : 1;  // k blocks of the readout over the kept n
  f32x4 acc[UPT][NTW];
  f32x4 zown[UPT][2];  // readout of this wave's two i tiles (own part), phase A -> B
  f32x4* sEx = reinterpret_cast<f32x4*>(smem + Lt::oEx(ROPE));
  constexpr bool kAllPt = NPT % kPGroups == 0;  // every wave owns UPT real p tiles
  constexpr bool kEarly = Lt::early_gram(ROPE);
  // S pieces of chunk c (two buffers with the early Gram tiles)
  auto sSb = [&](int c) __attribute__((always_inline)) {
    return reinterpret_cast<u32x2*>(smem + ((kEarly && (c & 1)) ? Lt::oS2(ROPE) : Lt::oS));
  };
  // causal (j tile, i tile) pairs, numbered (0,0) (0,1) (1,1) (0,2) (1,2) (2,2)
  // (0,3) (1,3) (2,3) (3,3); tile t is computed once, by wave t % 8
  auto tile_id = [](int jt, int it) { return it * (it + 1) / 2 + jt; };
  // phase A: masked Gram tile S^T(jt, it) = M o (B C^T)^T of chunk k -> LDS
  // The operand fragments of a tile are all read before its products start:
  // the scheduler barrier keeps the compiler from interleaving each k block's
  // reads with its product, which made a chain of LDS round trips.
  auto gram_fetch = [&](int k, auto JT, auto IT, bf16x8 (&fb)[NKB], bf16x8 (&fc)[NKB]) __attribute__((always_inline)) {
    constexpr int jt = decltype(JT)::value, it = decltype(IT)::value;
    const uint16_t* tB = slotB(k & 1) + opaque(16 * jt * NK);
    const uint16_t* tC = slotC(k & 1) + opaque(16 * it * NK);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int col = 32 * kb + 4 * g;  // rows of a row tile share their swizzle with l16
      fb[kb] = cat8(*reinterpret_cast<const u32x2*>(tB + swz<NK>(l16, col)),
                    *reinterpret_cast<const u32x2*>(tB + swz<NK>(l16, col + 16)));
      fc[kb] = cat8(*reinterpret_cast<const u32x2*>(tC + swz<NK>(l16, col)),
                    *reinterpret_cast<const u32x2*>(tC + swz<NK>(l16, col + 16)));
    }
  };
  auto gram_mma = [&](const bf16x8 (&fb)[NKB], const bf16x8 (&fc)[NKB]) __attribute__((always_inline)) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) a = mma(fb[kb], fc[kb], a);
    return a;
  };
  auto gram_store = [&](int k, auto JT, auto IT, f32x4 a) __attribute__((always_inline)) {
    constexpr int jt = decltype(JT)::value, it = decltype(IT)::value;
    const float* S = sc(k % 3);
    const int ti = (16 * it + l16) >> LGR;
    const float lamI = S[ti], gamI = S[64 + ti];
    // scalars are read and the decay evaluated on every lane, then selected:
    // keeps the tile free of divergent control flow
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int tj = (16 * jt + 4 * g + jj) >> LGR;
      const float mk = __builtin_amdgcn_exp2f(lamI - S[tj]) * S[2 * 64 + tj];
      if constexpr (jt < it) {  // every token of tile jt precedes every token of tile it
        a[jj] *= mk;
      } else {
        const float sel = tj < ti ? mk : gamI;
        a[jj] *= tj <= ti ? sel : 0.f;
      }
    }
    sSb(k)[tile_id(jt, it) * 64 + lane] = pack4(a);
  };
  auto gram_one = [&](int k, auto JT, auto IT) __attribute__((always_inline)) {
    bf16x8 fb[NKB], fc[NKB];
    gram_fetch(k, JT, IT, fb, fc);
    __builtin_amdgcn_sched_barrier(0);
    gram_store(k, JT, IT, gram_mma(fb, fc));
  };
  // two tiles: the second tile's reads are issued behind the first tile's
  // products and overlap its masking
  auto gram_two = [&](int k, auto JT, auto IT, auto JT2, auto IT2) __attribute__((always_inline)) {
    bf16x8 fb[NKB], fc[NKB], fb2[NKB], fc2[NKB];
    gram_fetch(k, JT, IT, fb, fc);
    __builtin_amdgcn_sched_barrier(0);
    const f32x4 a = gram_mma(fb, fc);
    gram_fetch(k, JT2, IT2, fb2, fc2);
    __builtin_amdgcn_sched_barrier(0);
    gram_store(k, JT, IT, a);
    gram_store(k, JT2, IT2, gram_mma(fb2, fc2));
  };
  auto gram_tiles = [&](int k) __attribute__((always_inline)) {
    if constexpr (SO) return;
    using std::integral_constant;
    switch (wave) {
      case 0: gram_two(k, integral_constant<int, 0>{}, integral_constant<int, 0>{},
                       integral_constant<int, 2>{}, integral_constant<int, 3>{}); break;
      case 1: gram_two(k, integral_constant<int, 0>{}, integral_constant<int, 1>{},
                       integral_constant<int, 3>{}, integral_constant<int, 3>{}); break;
      case 2: gram_one(k, integral_constant<int, 1>{}, integral_constant<int, 1>{}); break;
      case 3: gram_one(k, integral_constant<int, 0>{}, integral_constant<int, 2>{}); break;
      case 4: gram_one(k, integral_constant<int, 1>{}, integral_constant<int, 2>{}); break;
      case 5: gram_one(k, integral_constant<int, 2>{}, integral_constant<int, 2>{}); break;
      case 6: gram_one(k, integral_constant<int, 0>{}, integral_constant<int, 3>{}); break;
      default: gram_one(k, integral_constant<int, 1>{}, integral_constant<int, 3>{}); break;
    }
  };
  // i tiles owned in phase B: {0, 3} (lower waves) and {1, 2} (upper waves)
  auto own_tile = [](int h, int idx) { return h == 0 ? (idx == 0 ? 0 : 3) : (idx == 0 ? 1 : 2); };
  // phase A: readout C^T H'_prev of chunk k from the kept part of the state.
  // With the n split, every wave covers all four i tiles over its n tiles and
  // hands the partner's two to LDS; otherwise it covers its own two over all n.
  auto readout = [&](int k, auto HALF) __attribute__((always_inline)) {
    if constexpr (SO) return;
    constexpr int h = decltype(HALF)::value;
    constexpr int nb = kSplit && h ? NTW : 0;  // first kept n tile
    const uint16_t* sC = slotC(k & 1);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!(kAllPt || quad + kPGroups * u < NPT)) continue;
      bf16x8 hfr[NKW];
#pragma unroll
      for (int kw = 0; kw < NKW; ++kw) {
        constexpr u32x2 zero2 = {0u, 0u};
        if constexpr (NTW >= 2) {
          hfr[kw] = cat8(pack4(acc[u][2 * kw]), pack4(acc[u][2 * kw + 1]));
        } else {  // one kept n tile: the low or high half of k block 0
          hfr[kw] = (nb & 1) ? cat8(zero2, pack4(acc[u][0])) : cat8(pack4(acc[u][0]), zero2);
        }
      }
      constexpr int kb0 = NTW >= 2 ? nb / 2 : 0;
      // all C fragments first (own i tiles, then the partner's), then the products
      constexpr int NI = kSplit ? 4 : 2;
      bf16x8 cf[NI][NKW];
#pragma unroll
      for (int q = 0; q < NI; ++q) {
        const int it = q < 2 ? own_tile(h, q) : own_tile(1 - h, q - 2);
        const uint16_t* tC = sC + opaque(16 * it * NK);
#pragma unroll
        for (int kw = 0; kw < NKW; ++kw) {
          const int col = 32 * (kb0 + kw) + 4 * g;
          cf[q][kw] = cat8(*reinterpret_cast<const u32x2*>(tC + swz<NK>(l16, col)),
                           *reinterpret_cast<const u32x2*>(tC + swz<NK>(l16, col + 16)));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < NI; ++q) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kw = 0; kw < NKW; ++kw) z = mma(hfr[kw], cf[q][kw], z);
        if (q < 2)
          zown[u][q] = z;
        else
          sEx[((wave * UPT + u) * 2 + (q - 2)) * 64 + lane] = z;
      }
    }
  };
  // transposed reads: slot e of k block m holds row 32 m + 4g + e (+16 in
  // the upper four slots), the order of the masked Gram pieces; this lane
  // points at row 32 m + 4g + l16 / 4, columns 4 (l16 % 4) + 0..3
  const int rT = 4 * g + (l16 >> 2), c4 = 4 * (l16 & 3);
  // X^T of p tile quad + 4u, k block m, of the next chunk to compute: read once
  // its slot is visible, a phase before it is used
  bf16x8 xnext[UPT][2];
  auto load_x = [&](int c) __attribute__((always_inline)) {
    const uint16_t* sX = slotX(c & 1);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int pt = quad + kPGroups * u;
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (kAllPt || pt < NPT)
          xnext[u][m] = cat8(lds_read_tr(sX + swz<PK>(32 * m + rT, 16 * pt + c4)),
                             lds_read_tr(sX + swz<PK>(32 * m + 16 + rT, 16 * pt + c4)));
    }
  };
  // phase B: y of this wave's i tiles and p tiles, then the state update
  auto compute_rest = [&](int k, auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    constexpr int nb = kSplit && h ? NTW : 0;
    const int s2 = k & 1;
    const float* S = sc(k % 3);
    const uint16_t* sB = slotB(s2);
    const u32x2* sS = sSb(k);
    const float cdec = S[5 * 64];
    auto& xfr = xnext;  // X^T of chunk k, read during chunk k - 1
    // B^T fragments of the state update are read first; the y products run
    // while they land
    bf16x8 btr[NTW][2];
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        btr[i][m] = cat8(lds_read_tr(sB + swz<NK>(32 * m + rT, 16 * (nb + i) + c4)),
                         lds_read_tr(sB + swz<NK>(32 * m + 16 + rT, 16 * (nb + i) + c4)));
    __builtin_amdgcn_sched_barrier(0);
    auto do_it = [&](auto IT, auto IDX) __attribute__((always_inline)) {
      constexpr int it = decltype(IT)::value, idx = decltype(IDX)::value;
      const int iRow = 16 * it + l16;
      const int ti = iRow >> LGR;
      const float decI = S[4 * 64 + ti];
      f32x4 yacc[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) yacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (2 * m <= it) {
          constexpr u32x2 zero2 = {0u, 0u};
          const u32x2 lo = sS[opaque(tile_id(2 * m, it) * 64) + lane];
          const u32x2 hi = (2 * m + 1 <= it) ? sS[opaque(tile_id(2 * m + 1 <= it ? 2 * m + 1 : 0, it) * 64) + lane] : zero2;
          const bf16x8 sop = cat8(lo, hi);
#pragma unroll
          for (int u = 0; u < UPT; ++u)
            if (kAllPt || quad + kPGroups * u < NPT) yacc[u] = mma(xfr[u][m], sop, yacc[u]);
        }
      }
      const uint32_t yrow = static_cast<uint32_t>((k * Q + ti) * tsR + (iRow & (R - 1))) * P;
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int pt = quad + kPGroups * u;
        if (kAllPt || pt < NPT) {
          f32x4 zz = zown[u][idx];
          if constexpr (kSplit) zz += sEx[(((wave ^ 4) * UPT + u) * 2 + idx) * 64 + lane];
          const f32x4 yv = yacc[u] + decI * zz;
          if constexpr (kStageY)
            sY[iRow * (Lt::PY / 4) + 4 * pt + g] = pack4(yv);
          else
            bstore8(rY, (yrow + 16 * pt + 4 * g) * 2u, pack4(yv));  // rows past L are dropped
        }
      }
    };
    using std::integral_constant;
    if constexpr (!SO) {
      do_it(integral_constant<int, h == 0 ? 0 : 1>{}, integral_constant<int, 0>{});
      do_it(integral_constant<int, h == 0 ? 3 : 2>{}, integral_constant<int, 1>{});
    }
    // H' = exp(Lam_e) H' + B^T (w X) on the kept n tiles, w_j = exp(Lam_e -
    // Lam_j) delta_j applied to the X fragments of the rows this lane holds
    f32x4 wrow[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) wrow[m][hh][e] = S[3 * 64 + ((32 * m + 16 * hh + 4 * g + e) >> LGR)];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int pt = quad + kPGroups * u;
      if (kAllPt || pt < NPT) {
        bf16x8 wfr[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) wfr[m] = scale8(xfr[u][m], wrow[m][0], wrow[m][1]);
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const int nt = nb + i;
          f32x4 a = acc[u][i] * cdec;
#pragma unroll
          for (int m = 0; m < 2; ++m) a = mma(btr[i][m], wfr[m], a);
          acc[u][i] = a;
        }
      }
    }
  };

  // staged y of chunk c -> HBM in whole rows, 16 bytes per lane; every thread
  // issues the same number of stores (rows past the end, or c < 0, are dropped)
  auto flush_y = [&](int c) __attribute__((always_inline)) {
    constexpr int kUnits = kRows * P / 8;
    constexpr int kIter = (kUnits + kThreads - 1) / kThreads;
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int e = tid + it * kThreads;
      const int eu = e < kUnits ? e : e - kUnits;
      const int r = eu / (P / 8), c8 = eu % (P / 8);
      const u32x2* src = sY + r * (Lt::PY / 4) + 2 * c8;
      const u32x2 lo = src[0], hi = src[1];
      const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
      const uint32_t off = (c >= 0 && e < kUnits)
                               ? (static_cast<uint32_t>((c * Q + (r >> LGR)) * tsR + (r & (R - 1))) * P + 8 * c8) * 2u
                               : kBad;
      bstore16_nt(rY, off, v);
    }
  };

  // ================================================================ prologue
  // H'_{-1} = h0 + (1 - lambda_0) Delta_0 sum_r Bprev_rot[r] xprev[r]^T (kept tiles)
  auto init_state = [&](auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    constexpr int nb = kSplit && h ? NTW : 0;
    const size_t o0 = tok0 * H + hh;
    const float coef = (1.f - p.lam[o0]) * delta_of(p.dt[o0], proDt, dtBias, true);
    const bool hasCarry = cBprev != nullptr && cXprev != nullptr;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int pt = quad + kPGroups * u;
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int nt = nb + i;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (pt < NPT) {
          const int pc = 16 * pt + l16;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int n = 16 * nt + 4 * g + jj;
            float v = cH0 != nullptr ? cH0[static_cast<size_t>(bh) * N * P + static_cast<size_t>(n) * P + pc] : 0.f;
            if (hasCarry) {
              float uu = 0.f;
#pragma unroll
              for (int rr = 0; rr < R; ++rr)
                uu += cBprev[(static_cast<size_t>(bh) * R + rr) * N + n] *
                      bf16_to_f32(static_cast<const bf16_t*>(cXprev)[(static_cast<size_t>(bh) * R + rr) * P + pc].bits);
              v += coef * uu;
            }
            a[jj] = v;
          }
        }
        acc[u][i] = a;
      }
    }
  };
  if (!upper)
    init_state(std::integral_constant<int, 0>{});
  else
    init_state(std::integral_constant<int, 1>{});
  if constexpr (ROPE)
    for (int q = tid; q < N / 2; q += kThreads)
      phiC[q] = cPhi0 != nullptr ? cPhi0[static_cast<size_t>(bh) * (N / 2) + q] : 0.f;
  // retire the prologue's state and carry loads here, so no wait on them is
  // left for the loop to repeat every chunk
  __builtin_amdgcn_s_waitcnt(0);
  auto prologue = [&](auto HALF) __attribute__((always_inline)) {
    issue_small(0, 0);
    issue_small(1, 1);
    issue_bcx(0, raw[0], HALF);
    if constexpr (kSets == 2) issue_bcx(1, raw[kSets - 1], HALF);
    stage_small(0, 0);
    issue_small(2, 0);
    __syncthreads();  // angle carry, raw theta(0) visible
    scan_angles(0);
    __syncthreads();  // SC(0), Phi(0) visible
    build_slot(0, raw[0], HALF);  // and issues chunk kSets into raw[0]
    if constexpr (kLateRefill && decltype(HALF)::value == 1) issue_bcx(kSets, raw[0], HALF);
    stage_small(1, 1);
    issue_small(3, 1);
    __syncthreads();  // slot 0, raw theta(1) visible
    scan_angles(1);
    if constexpr (kEarly) gram_tiles(0);
    __syncthreads();  // slot 0, S(0), SC(1), Phi(1) visible
    load_x(0);
  };
  // chunk walk, unrolled by two so the small-load register sets are indexed
  // statically.  Phase A: stage chunk k+1 (`bcx` holds it), refill `bcx` with
  // the loads of chunk k+2, scan the decays and store the raw angles of chunk
  // k+2, issue the small loads of chunk k+4, and compute the readout partials of chunk k
  // (and its masked Gram tiles when they are not computed early); phase B:
  // scan the angles of chunk k+2, products, y and state of chunk k, then the
  // Gram tiles of chunk k+1.
  auto chunk = [&](int k, u32x4 (&bcx)[UPH], int sset, auto HALF) __attribute__((always_inline)) {
    if constexpr (kStageY) flush_y(k - 1);
    build_slot(k + 1, bcx, HALF);  // and issues chunk k+1+kSets into bcx
    if constexpr (!kDecayInB)
      stage_decay(k + 2, sset);
    else if (om)
      stage_dt(k + 2, sset);  // the angle scan of this chunk scales by Delta
    stage_theta(k + 2, sset);
    if constexpr (!kDecayInB) issue_small(k + 4, sset);  // after the reads of its register set
    if constexpr (!kEarly) gram_tiles(k);
    readout(k, HALF);
    __syncthreads();  // S(k), readout partials, slot k+1, raw theta(k+2) visible
    // the upper waves' refill, first thing in phase B: issued after the
    // products instead, its loads were still in flight when phase A staged
    // them (the upper waves' staging took ~1,250 cycles against ~770)
    if constexpr (kLateRefill && decltype(HALF)::value == 1) issue_bcx(k + 1 + kSets, bcx, HALF);
    scan_angles(k + 2);
    compute_rest(k, HALF);
    load_x(k + 1);  // slot k+1 is visible since the first barrier
    if constexpr (kDecayInB) {
      stage_decay(k + 2, sset);  // first read after the next barrier
      issue_small(k + 4, sset);
    }
    if constexpr (kEarly) gram_tiles(k + 1);  // overlaps the tail of chunk k
    __syncthreads();  // S(k+1), SC(k+2), Phi(k+2) visible; slot k free
  };
  auto walk = [&](auto HALF) __attribute__((always_inline)) {
    for (int k = 0; k < nch; k += 2) {
      chunk(k, raw[kSets - 1], 0, HALF);
      if (k + 1 < nch) chunk(k + 1, raw[0], 1, HALF);
    }
  };
  if (!upper) {
    if constexpr (PRO) load_pro(std::integral_constant<int, 0>{});
    prologue(std::integral_constant<int, 0>{});
    walk(std::integral_constant<int, 0>{});
  } else {
    if constexpr (PRO) load_pro(std::integral_constant<int, 1>{});
    prologue(std::integral_constant<int, 1>{});
    walk(std::integral_constant<int, 1>{});
  }

  // ================================================================ epilogue
  if constexpr (kStageY) flush_y(nch - 1);  // the walk ended on a barrier
  if (!lastSeg && !p.outAll) return;
  // with outAll, segment s writes at offset s x (one output's size)
  const size_t so = p.outAll ? static_cast<size_t>(seg) : 0;
  const size_t uAll = static_cast<size_t>(units);
  float* const hOut = p.h_final != nullptr ? p.h_final + so * uAll * N * P : nullptr;
  float* const phiOut = p.phi_out != nullptr ? p.phi_out + so * uAll * (N / 2) : nullptr;
  float* const bOut = p.Bprev_rot_out != nullptr ? p.Bprev_rot_out + so * uAll * R * N : nullptr;
  bf16_t* const xOut = p.xprev_out != nullptr ? static_cast<bf16_t*>(p.xprev_out) + so * uAll * R * P : nullptr;
  // each wave writes its kept n tiles (both waves hold all of them without the split)
  auto write_state = [&](auto HALF) __attribute__((always_inline)) {
    constexpr int h = decltype(HALF)::value;
    constexpr int nb = kSplit && h ? NTW : 0;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int pt = quad + kPGroups * u;
      if (pt < NPT) {
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            hOut[static_cast<size_t>(bh) * N * P + static_cast<size_t>(16 * (nb + i) + 4 * g + jj) * P + 16 * pt + l16] =
                acc[u][i][jj];
      }
    }
  };
  if (hOut != nullptr) {
    if (!upper)
      write_state(std::integral_constant<int, 0>{});
    else if (kSplit)
      write_state(std::integral_constant<int, 1>{});
  }
  if constexpr (ROPE) {
    if (phiOut != nullptr)
      for (int q = tid; q < N / 2; q += kThreads) phiOut[static_cast<size_t>(bh) * (N / 2) + q] = phiC[q];
  }
  // carry-out of token L-1: rotated B (fp32) and x
  {
    const int t = L - 1;
    if (bOut != nullptr) {
      // with the prologue, B_{L-1} normalised (1 / RMS of each rank's row in
      // the exchange area, free after the walk) and biased as when staged
      if (proNorm) {
        if (tid < R) {
          const bf16_t* src = static_cast<const bf16_t*>(p.B) + (row0 + static_cast<size_t>(t) * tsR + tid) * N;
          float ss = 0.f;
          for (int n = 0; n < N; ++n) {
            const float v = bf16_to_f32(src[n].bits);
            ss += v * v;
          }
          proEx[tid] = ss > 0.f ? rsqrtf(ss * (1.f / N) + proEps) : 0.f;
        }
        __syncthreads();
      }
      for (int e = tid; e < R * (N / 2); e += kThreads) {
        const int r = e / (N / 2), q = e % (N / 2);
        const bf16_t* src = static_cast<const bf16_t*>(p.B) + (row0 + static_cast<size_t>(t) * tsR + r) * N;
        float a0 = bf16_to_f32(src[2 * q].bits), a1 = bf16_to_f32(src[2 * q + 1].bits);
        if (proBC) {
          const float* w = p.pro.B_w;
          const float* bb = p.pro.B_bias != nullptr ? p.pro.B_bias + (static_cast<size_t>(hh) * R + r) * N : nullptr;
          const float sc0 = proNorm ? proEx[r] * (w != nullptr ? w[2 * q] : 1.f) : 1.f;
          const float sc1 = proNorm ? proEx[r] * (w != nullptr ? w[2 * q + 1] : 1.f) : 1.f;
          a0 = a0 * sc0 + (bb != nullptr ? bb[2 * q] : 0.f);
          a1 = a1 * sc1 + (bb != nullptr ? bb[2 * q + 1] : 0.f);
        }
        if constexpr (ROPE) {
          // Phi_{L-1} is the final angle carry (reduced modulo 2 pi)
          float sn, cs;
          sincosf(phiC[q], &sn, &cs);
          const float b0 = cs * a0 + sn * a1, b1 = cs * a1 - sn * a0;
          a0 = b0;
          a1 = b1;
        }
        float* dst = bOut + (static_cast<size_t>(bh) * R + r) * N + 2 * q;
        dst[0] = a0;
        dst[1] = a1;
      }
    }
    if (xOut != nullptr)
      for (int e = tid; e < R * P; e += kThreads)
        xOut[static_cast<size_t>(bh) * R * P + e] =
            static_cast<const bf16_t*>(p.x)[(row0 + static_cast<size_t>(t) * tsR) * P + e];
  }
}

}  // namespace pc
}  // namespace m3
