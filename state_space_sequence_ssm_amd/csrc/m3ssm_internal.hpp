// Kernel parameter blocks and launcher entry points shared between the C-ABI
// layer (api.hip) and the kernels.  Plain pointers and sizes only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace m3 {

// A kernel that uses more than 64 KB of dynamic LDS must be cleared for it,
// per device, before its first launch there.  `cleared` (one per kernel) has
// bit d set once device d is done; the attribute is always set to the same
// value (the most the kernel ever asks for), so concurrent first calls from
// several host threads at worst repeat an idempotent call.
inline hipError_t allow_lds(const void* fn, size_t max_bytes, std::atomic<uint64_t>& cleared) {
  if (max_bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
  if (bit != 0 && (cleared.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(max_bytes));
  if (e == hipSuccess && bit != 0) cleared.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Steps fused in front of the core (all off when zero / null):
//   Delta = softplus(dt + dt_bias[h]) when dt_softplus (dt is then the raw
//   value); each (token, head, rank) row of B and of C RMS-normalised over N,
//   row / sqrt(mean(row^2) + eps) times the gain w[N], when bc_norm; then the
//   head-specific biases [H, R, N] added to B and C.
struct Prologue {
  int bc_norm, dt_softplus;
  float eps;
  const float* B_w;     // [N] or null (gain 1)
  const float* C_w;     // [N] or null
  const float* B_bias;  // [H, R, N] or null
  const float* C_bias;  // [H, R, N] or null
  const float* dt_bias; // [H] or null
};

struct DecodeParams {
  int Bt, H, P, N, R;
  bool bf16;
  float* h;
  float* phi;
  float* Bprev_rot;
  void* xprev;
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* A;
  const float* theta;
  void* y;
  const float* A_tok;  // [Bt, H] A of this token, or null (then A [H])
  const float* omega;  // [Bt, N/2] rates shared by the heads (theta = dt * omega), or null
  Prologue pro;
};

struct PrefillParams {
  int Bt, L, H, P, N, R;
  int log2R;
  int chunk;  // tokens per chunk, 0: 64 / R (the fp32 kernel also takes a smaller power of two)
  bool bf16;
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* A;
  const float* theta;
  // omega [Bt, L, N/2] (bf16 path): per-token angular rates shared by the
  // heads; when set (theta is then null), theta = Delta * omega on chip
  const float* omega;
  // A_tok [Bt, L, H]: A per token, or null (then A [H] for every token)
  const float* A_tok;
  const float* h0;
  const float* Bprev_rot;
  const void* xprev;
  const float* phi0;
  void* y;
  float* h_final;
  float* Bprev_rot_out;
  void* xprev_out;
  float* phi_out;
  // Sequence segments (bf16 path).  Tokens of batch item b start at
  // b * Lfull; this launch covers tokens [0, L) of each item, cut into nseg
  // segments of segLen tokens (the last one takes the rest), one workgroup per
  // (segment, batch, head).  Segment 0 takes the carry-in above; segment s > 0
  // takes the *_mid carry (the state after the previous segment).  Only the
  // last segment writes h_final and the carry-out.
  int Lfull, nseg, segLen;
  // outAll: every segment writes its end state and carry-out, segment s at
  // offset s x (the size of one such output)
  int outAll;
  const float* h_mid;
  const float* Bprev_mid;
  const void* xprev_mid;
  const float* phi_mid;
  // x, B, C, y head-major [Bt, H, L, R, .] instead of token-major (bf16 path)
  int headMajor;
  Prologue pro;
};

// Backward of the bf16 prefill (backward.hip): forward inputs, upstream
// gradients, gradient outputs and the workspace of chunk-entry states.
struct BackwardParams {
  int Bt, L, H, P, N, R, log2R;
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* A;      // [H] or null
  const float* A_tok;  // [Bt, L, H] or null
  const float* theta;  // [Bt, L, H, N/2] or null
  const float* h0;
  const float* Bprev_rot;
  const void* xprev;
  const float* phi0;
  const void* dy;        // [Bt, L, H, R, P] bf16
  const float* dh_final; // [Bt, H, N, P] or null
  void* dx;
  void* dB;
  void* dC;
  float* ddt;
  float* dlam;
  float* dA_tok;    // [Bt, L, H] when A_tok is given
  float* dA_part;   // [Bt * H] per-unit sums of dA (workspace) when A is per head
  float* dtheta;    // [Bt, L, H, N/2] or null
  float* dh0;
  float* dBprev_rot;
  void* dxprev;
  float* dphi0;
  void* states;     // [Bt * H][chunks][N * P] shifted state entering each chunk (bf16, accumulator tile order)
  float* phis;      // [Bt * H][chunks][N/2] angle entering each chunk
  // sequence split at chunk cm (0: none); dA_part is then [2][Bt * H]
  int cm;
  float* sH;        // [Bt * H][N * P] shifted state entering chunk cm
  float* sPhiM;     // [Bt * H][N/2] angle entering chunk cm
  float* sG;        // [Bt * H][N * P] segment 1's relative part of the gradient entering chunk cm
  float* sDc;       // [Bt * H] decay over segment 1
  float* sDth;      // [Bt * H][N/2] dtheta at token cm Q
  float* sTok;      // [2][Bt * H][2] the two segments' parts of token cm Q's Delta and lambda gradients
};
// one walk per (batch, head), or with cm > 0 the split's pre, main and join launches
hipError_t launch_backward(const BackwardParams& p, hipStream_t s);
hipError_t launch_backward_pre(const BackwardParams& p, hipStream_t s);
hipError_t launch_backward_main(const BackwardParams& p, hipStream_t s);
// dA [H] = sum over the batch of the per-unit sums
hipError_t launch_backward_dA(const float* part, float* dA, int Bt, int H, hipStream_t s);
size_t backward_lds_bytes(int N, int P, bool rope);

struct AnglesParams {
  const float* theta;
  const float* phi0;
  float* phi;
  int Bt, L, H, J;  // J = number of angle pairs per head
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
// decode step on the matrix cores: bf16, N in {32, 64, 128}, P in {64, 128}, R <= 16
bool decode_mma_supported(const DecodeParams& p);
hipError_t launch_decode_mma(const DecodeParams& p, hipStream_t s);
// state_only: the walk that produces the state and carry only (no y)
hipError_t launch_prefill_bf16(const PrefillParams& p, bool state_only, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t s);
hipError_t launch_angles(const AnglesParams& p, hipStream_t s);
// Joins the end states of two consecutive segments into the state after the
// second (see split.hip): in place in the workspace buffers.
struct CombineParams {
  int Bt, H, N, P, R, Lfull;
  int t1, t2;  // the second segment covers tokens [t1, t2) of each batch item
  const float* dt;
  const float* lam;
  const float* A;
  const float* A_tok;  // [Bt, L, H] or null
  int dt_softplus;     // dt holds raw values: Delta = softplus(dt + dt_bias[h])
  const float* dt_bias;
  float* h;        // [2][Bt*H][N][P]: segment 0 end state -> joined state
  float* Bprev;    // [2][Bt*H][R][N]: segment 1's (relative frame) -> rotated in place
  const void* x0;  // [Bt*H][R][P] bf16: segment 0's last x
  float* phi;      // [2][Bt*H][N/2] or null: segment 1's relative angle -> absolute
};
hipError_t launch_split_combine(const CombineParams& c, hipStream_t s);
// LDS bytes the prefill kernel needs for (N, P, rope) and, with `pro_bc`
// (B / C normalisation), for the row-sum exchange of its prologue; 0 if not
// compiled.
size_t prefill_lds_bytes_bf16(int N, int P, int R, bool rope, bool pro_bc);
size_t prefill_lds_bytes_f32(int N, int P, bool rope);

}  // namespace m3
