// C ABI of the Mamba-3 SSM core: host-side validation and dispatch.
// Every check runs on the host before any HIP call, so invalid arguments are
// rejected without a GPU (the contract of include/m3ssm.h).
#include <stdint.h>

#include "m3ssm.h"
#include "m3ssm_internal.hpp"

namespace {

constexpr size_t kMaxLds = 160 * 1024;

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool tile_dim(int v) { return v == 16 || v == 32 || v == 64 || v == 128; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool al16(const void* p) { return p == nullptr || aligned(p, 16); }
bool al4(const void* p) { return p == nullptr || aligned(p, 4); }

int hip_status(hipError_t e) { return e == hipSuccess ? M3_OK : M3_ERR_HIP; }

// Compute units of the current device (cached per device; 256, the MI355X
// count, when no device can be queried).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 256;
    }
    cache[dev] = v;
  }
  return cache[dev];
}

// Sequence split of the bf16 prefill: with fewer (batch, head) units than
// half the compute units, a state-only walk over the first half of every
// sequence hands its end state to the second half, and both halves then run
// at once (twice the workgroups).  Workspace: the state and carry in the
// middle of each sequence.
constexpr int kMinSegChunks = 4;  // both halves keep at least this many chunks
struct SplitPlan {
  bool on = false;
  int segLen = 0;  // tokens of the first half
  int segA = 0;    // > 0: the first half's state-only walk runs as two parts of segA and the rest
  size_t oH = 0, oB = 0, oX = 0, oPhi = 0, bytes = 0;
};
size_t up256(size_t v) { return (v + 255) & ~size_t(255); }
SplitPlan split_plan(const m3_prefill_args* a) {
  SplitPlan s;
  if (a->in_dtype != M3_BF16 || a->R < 1 || a->R > 8) return s;
  const int Q = 64 / a->R;
  const long units = long(a->Bt) * a->H;
  if (2 * units > device_cus() || a->L < 2 * kMinSegChunks * Q) return s;
  const size_t u = size_t(units);
  s.on = true;
  s.segLen = (((a->L + 1) / 2 + Q - 1) / Q) * Q;
  if (s.segLen >= 2 * kMinSegChunks * Q) s.segA = (((s.segLen + 1) / 2 + Q - 1) / Q) * Q;
  // state and carry of two segments: [2][units][...] each
  s.oH = 0;
  s.oB = up256(s.oH + 2 * u * a->N * a->P * 4);
  s.oX = up256(s.oB + 2 * u * a->R * a->N * 4);
  s.oPhi = up256(s.oX + 2 * u * a->R * a->P * 2);
  const bool rope = a->theta != nullptr || a->omega != nullptr;
  s.bytes = up256(s.oPhi + (rope ? 2 * u * (a->N / 2) * 4 : 0));
  return s;
}

}  // namespace

extern "C" {

const char* m3_status_string(int status) {
  switch (status) {
    case M3_OK: return "ok";
    case M3_ERR_INVALID_ARG: return "invalid argument";
    case M3_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case M3_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* m3_version(void) { return "0.1.0"; }

size_t m3_ssm_prefill_workspace_size(const m3_prefill_args* args) {
  if (args == nullptr) return 0;
  const SplitPlan s = split_plan(args);
  return s.on ? s.bytes : 0;
}

int m3_ssm_prefill(const m3_prefill_args* a, void* stream) {
  if (a == nullptr) return M3_ERR_INVALID_ARG;
  if (a->Bt < 1 || a->L < 1 || a->H < 1 || a->R < 1 || a->N < 1 || a->P < 1) return M3_ERR_INVALID_ARG;
  if (a->in_dtype != M3_F32 && a->in_dtype != M3_BF16) return M3_ERR_UNSUPPORTED;
  if (a->layout != M3_TOKEN_MAJOR && a->layout != M3_HEAD_MAJOR) return M3_ERR_INVALID_ARG;
  if (!a->x || !a->B || !a->C || !a->dt || !a->lam || (!a->A && !a->A_tok) || !a->y) return M3_ERR_INVALID_ARG;
  if ((a->Bprev_rot == nullptr) != (a->xprev == nullptr)) return M3_ERR_INVALID_ARG;
  if (a->theta != nullptr && a->omega != nullptr) return M3_ERR_INVALID_ARG;  // one angle source
  const bool rope = a->theta != nullptr || a->omega != nullptr;
  if (!rope && (a->phi0 != nullptr || a->phi_out != nullptr)) return M3_ERR_INVALID_ARG;
  if (rope && (a->N % 2) != 0) return M3_ERR_INVALID_ARG;
  if (!pow2(a->R) || a->R > 64) return M3_ERR_UNSUPPORTED;
  if (!tile_dim(a->N) || !tile_dim(a->P)) return M3_ERR_UNSUPPORTED;
  if (a->chunk != 0 && a->chunk != 64 / a->R) return M3_ERR_UNSUPPORTED;
  const void* v16[] = {a->x, a->B, a->C, a->y, a->theta, a->omega, a->h0, a->Bprev_rot, a->xprev,
                       a->phi0, a->h_final, a->Bprev_rot_out, a->xprev_out, a->phi_out};
  for (const void* p : v16)
    if (!al16(p)) return M3_ERR_INVALID_ARG;
  if (!al4(a->dt) || !al4(a->lam) || !al4(a->A) || !al4(a->A_tok)) return M3_ERR_INVALID_ARG;
  const double elems = double(a->Bt) * a->L * a->H * a->R * (a->N > a->P ? a->N : a->P);
  if (elems > 4.0e18 || double(a->Bt) * a->H > 2147483647.0) return M3_ERR_INVALID_ARG;
  const bool bf16 = a->in_dtype == M3_BF16;
  if (bf16) {
    // the bf16 kernel is compiled for R <= 8 and addresses one batch item with
    // 32-bit buffer offsets
    if (a->R > 8) return M3_ERR_UNSUPPORTED;
    const double item = double(a->L) * a->H * a->R * (a->N > a->P ? a->N : a->P) * 2.0;
    const double itemTh = double(a->L) * a->H * (a->N / 2) * 4.0;
    if (item > 2147483000.0 || itemTh > 2147483000.0) return M3_ERR_UNSUPPORTED;
  }
  const size_t lds = bf16 ? m3::prefill_lds_bytes_bf16(a->N, a->P, rope)
                          : m3::prefill_lds_bytes_f32(a->N, a->P, rope);
  if (lds == 0 || lds > kMaxLds) return M3_ERR_UNSUPPORTED;

  m3::PrefillParams p{};
  p.Bt = a->Bt; p.L = a->L; p.H = a->H; p.P = a->P; p.N = a->N; p.R = a->R;
  int lg = 0;
  while ((1 << lg) < a->R) ++lg;
  p.log2R = lg;
  p.bf16 = bf16;
  p.x = a->x; p.B = a->B; p.C = a->C; p.dt = a->dt; p.lam = a->lam; p.A = a->A; p.theta = a->theta;
  p.omega = a->omega;
  p.A_tok = a->A_tok;
  p.h0 = a->h0; p.Bprev_rot = a->Bprev_rot; p.xprev = a->xprev; p.phi0 = a->phi0;
  p.y = a->y; p.h_final = a->h_final; p.Bprev_rot_out = a->Bprev_rot_out; p.xprev_out = a->xprev_out;
  p.phi_out = a->phi_out;
  p.Lfull = a->L;
  p.nseg = 1;
  p.segLen = a->L;
  p.headMajor = a->layout == M3_HEAD_MAJOR;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!bf16) return hip_status(m3::launch_prefill_f32(p, st));

  const SplitPlan sp = split_plan(a);
  if (!sp.on || a->workspace == nullptr) return hip_status(m3::launch_prefill_bf16(p, false, st));
  if (a->workspace_bytes < sp.bytes || !aligned(a->workspace, 256)) return M3_ERR_INVALID_ARG;
  unsigned char* ws = static_cast<unsigned char*>(a->workspace);
  const size_t u = size_t(a->Bt) * a->H;
  float* hMid = reinterpret_cast<float*>(ws + sp.oH);
  float* bMid = reinterpret_cast<float*>(ws + sp.oB);
  unsigned char* xMid = ws + sp.oX;
  float* phiMid = rope ? reinterpret_cast<float*>(ws + sp.oPhi) : nullptr;
  // 1) state and carry after the first segLen tokens (carry-in of the call)
  m3::PrefillParams pa = p;
  pa.L = sp.segLen;
  pa.segLen = sp.segLen;
  pa.y = nullptr;
  pa.h_final = hMid;
  pa.Bprev_rot_out = bMid;
  pa.xprev_out = xMid;
  pa.phi_out = phiMid;
  if (sp.segA > 0) {
    // as two parts at once, the second from a zero start, then joined
    pa.nseg = 2;
    pa.segLen = sp.segA;
    pa.outAll = 1;
  }
  hipError_t e = m3::launch_prefill_bf16(pa, true, st);
  if (e != hipSuccess) return hip_status(e);
  const float* hCarry = hMid;
  const float* bCarry = bMid;
  const void* xCarry = xMid;
  const float* phiCarry = phiMid;
  if (sp.segA > 0) {
    m3::CombineParams c{};
    c.Bt = a->Bt; c.H = a->H; c.N = a->N; c.P = a->P; c.R = a->R; c.Lfull = a->L;
    c.t1 = sp.segA;
    c.t2 = sp.segLen;
    c.dt = a->dt; c.lam = a->lam; c.A = a->A; c.A_tok = a->A_tok;
    c.h = hMid;
    c.Bprev = bMid;
    c.x0 = xMid;
    c.phi = phiMid;
    e = m3::launch_split_combine(c, st);
    if (e != hipSuccess) return hip_status(e);
    // joined state in part 0's slot; B, x and angle carries of part 1
    bCarry = bMid + u * a->R * a->N;
    xCarry = xMid + u * a->R * a->P * 2;
    phiCarry = phiMid != nullptr ? phiMid + u * (a->N / 2) : nullptr;
  }
  // 2) both halves at once; the second starts from that carry
  m3::PrefillParams pb = p;
  pb.nseg = 2;
  pb.segLen = sp.segLen;
  pb.h_mid = hCarry;
  pb.Bprev_mid = bCarry;
  pb.xprev_mid = xCarry;
  pb.phi_mid = phiCarry;
  return hip_status(m3::launch_prefill_bf16(pb, false, st));
}

int m3_ssm_decode_step(const m3_decode_args* a, void* stream) {
  if (a == nullptr) return M3_ERR_INVALID_ARG;
  if (a->Bt < 1 || a->H < 1 || a->R < 1 || a->N < 1 || a->P < 1) return M3_ERR_INVALID_ARG;
  if (a->in_dtype != M3_F32 && a->in_dtype != M3_BF16) return M3_ERR_UNSUPPORTED;
  if (!a->h || !a->Bprev_rot || !a->xprev || !a->x || !a->B || !a->C || !a->dt || !a->lam || (!a->A && !a->A_tok) ||
      !a->y)
    return M3_ERR_INVALID_ARG;
  if (a->theta != nullptr && a->omega != nullptr) return M3_ERR_INVALID_ARG;  // one angle source
  const bool rope = a->theta != nullptr || a->omega != nullptr;
  if (rope != (a->phi != nullptr)) return M3_ERR_INVALID_ARG;
  if (rope && (a->N % 2) != 0) return M3_ERR_INVALID_ARG;
  if (a->R > 16) return M3_ERR_UNSUPPORTED;
  if (!tile_dim(a->N) || !tile_dim(a->P)) return M3_ERR_UNSUPPORTED;
  const void* v16[] = {a->h, a->Bprev_rot, a->xprev, a->x, a->B, a->C, a->y, a->phi, a->theta, a->omega};
  for (const void* p : v16)
    if (!al16(p)) return M3_ERR_INVALID_ARG;
  if (!al4(a->dt) || !al4(a->lam) || !al4(a->A) || !al4(a->A_tok)) return M3_ERR_INVALID_ARG;
  if (double(a->Bt) * a->H > 2147483647.0) return M3_ERR_INVALID_ARG;
  m3::DecodeParams p{};
  p.Bt = a->Bt; p.H = a->H; p.P = a->P; p.N = a->N; p.R = a->R;
  p.bf16 = a->in_dtype == M3_BF16;
  p.h = a->h; p.phi = a->phi; p.Bprev_rot = a->Bprev_rot; p.xprev = a->xprev;
  p.x = a->x; p.B = a->B; p.C = a->C; p.dt = a->dt; p.lam = a->lam; p.A = a->A; p.theta = a->theta;
  p.y = a->y;
  p.A_tok = a->A_tok;
  p.omega = a->omega;
  return hip_status(m3::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int m3_rope_angles_cumsum(const float* theta, const float* phi0, float* phi, int32_t Bt, int32_t L,
                          int32_t H, int32_t npairs, void* stream) {
  if (theta == nullptr || phi == nullptr) return M3_ERR_INVALID_ARG;
  if (Bt < 1 || L < 1 || H < 1 || npairs < 1) return M3_ERR_INVALID_ARG;
  if ((int64_t(H) * npairs) % 4 != 0) return M3_ERR_UNSUPPORTED;
  if (!al16(theta) || !al16(phi) || !al16(phi0)) return M3_ERR_INVALID_ARG;
  if (theta == phi) return M3_ERR_INVALID_ARG;
  const int64_t tiles = (int64_t(H) * npairs / 4 + 7) / 8;
  if (tiles * Bt > 2147483647LL || double(Bt) * L * H * npairs > 4.0e18) return M3_ERR_INVALID_ARG;
  m3::AnglesParams p{theta, phi0, phi, Bt, L, H, npairs};
  return hip_status(m3::launch_angles(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
