// Kernel parameter blocks and launcher entry points shared between the C-ABI
// layer (api.hip) and the kernels.  Plain pointers and sizes only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

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
};

struct PrefillParams {
  int Bt, L, H, P, N, R;
  int log2R;
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
};

struct AnglesParams {
  const float* theta;
  const float* phi0;
  float* phi;
  int Bt, L, H, J;  // J = number of angle pairs per head
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
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
  float* h;        // [2][Bt*H][N][P]: segment 0 end state -> joined state
  float* Bprev;    // [2][Bt*H][R][N]: segment 1's (relative frame) -> rotated in place
  const void* x0;  // [Bt*H][R][P] bf16: segment 0's last x
  float* phi;      // [2][Bt*H][N/2] or null: segment 1's relative angle -> absolute
};
hipError_t launch_split_combine(const CombineParams& c, hipStream_t s);
// LDS bytes the prefill kernel needs for (N, P, rope); 0 if not compiled.
size_t prefill_lds_bytes_bf16(int N, int P, bool rope);
size_t prefill_lds_bytes_f32(int N, int P, bool rope);

}  // namespace m3
