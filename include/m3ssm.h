/*
 * m3ssm.h -- C ABI of the Mamba-3 SSM core for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are web pages on Mamba-3, cited by title/section):
 *   "Znakomstvo s Mamba-3" (chernovdev.ru), sec. 1, the displayed recurrence:
 *       h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1}^T + gamma_t B_t x_t^T,
 *       alpha_t = exp(Delta_t A), beta_t = (1 - lambda_t) Delta_t alpha_t,
 *       gamma_t = lambda_t Delta_t;
 *   same page, sec. 2: complex dynamics as data-dependent cumulative RoPE on
 *       B and C (angles aggregated over all time steps);
 *   same page, sec. 3, and "La dualita: Mamba-2 e Mamba-3" (book.paithon.it),
 *       sec. "Mamba-3": rank-R MIMO, B_t, C_t in R^{N x R}, x_t in R^{P x R},
 *       the update is a sum of R outer products on an unchanged N x P state;
 *   "La dualita", sec. "State Space Duality" / "Perche conviene": the chunked
 *       evaluation (intra-chunk masked product, chunk states, inter-chunk
 *       recurrence, readout of the previous state).
 *
 * Conventions fixed by this library (the pages leave them open):
 *   - Rotation pairs are adjacent state entries (2j, 2j+1).  With the inclusive
 *     cumulative angle Phi_t = Phi_{-1} + sum_{s<=t} theta_s, the kernels use
 *     Btil = R(Phi)^T B and Ctil = R(Phi)^T C, R(phi) = [[cos,-sin],[sin,cos]].
 *   - y_t[r] = h_t^T Ctil_t[r] (state after the update, no skip term).
 *   - The carried previous-token term uses the previous token's rotated B.
 *   - The state h is the real state in the rotated frame, fp32, [N][P] per head.
 *
 * Layouts: every tensor is dense row-major (C order), innermost dimension
 * last, with the shapes given below.  Base pointers of x, B, C, y, xprev,
 * xprev_out, h0, h_final, h, Bprev_rot, Bprev_rot_out must be 16-byte
 * aligned; theta / phi pointers must be 16-byte aligned.
 * All pointers are device pointers (hipMalloc'd or equivalent) unless noted.
 * The caller owns every buffer, including the optional prefill workspace; the
 * library allocates nothing.  Between calls it keeps only per-device caches,
 * each safe under concurrent first calls from several host threads: the
 * compute-unit count (atomics), which kernels have had their dynamic-LDS
 * limit raised (an atomic bit mask per kernel) and the address of the
 * no-allocation scratch (under a mutex).  Calls on different streams are
 * independent given separate workspaces (m3_ssm_prefill_noalloc shares its
 * scratch per device).
 * `stream` is a hipStream_t (NULL = the null stream).  All calls are
 * asynchronous with respect to the host; results are visible after the
 * stream is synchronised.  Results are deterministic (no atomics).
 *
 * Errors: every entry point validates its arguments on the host before any
 * launch and returns a negative m3_status without touching the GPU when they
 * are invalid.  No exception crosses the ABI.
 */
#ifndef M3SSM_H
#define M3SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum m3_status {
  M3_OK = 0,
  M3_ERR_INVALID_ARG = -1, /* null required pointer, bad size, misalignment  */
  M3_ERR_UNSUPPORTED = -2, /* shape/dtype outside the compiled kernel tiles  */
  M3_ERR_HIP = -3,         /* a HIP launch or runtime error was reported     */
  M3_ERR_SCRATCH = -4      /* m3_ssm_prefill_noalloc: the call needs more
                              scratch than M3_NOALLOC_SCRATCH_BYTES          */
} m3_status;

typedef enum m3_dtype {
  M3_F32 = 0,  /* IEEE float32 */
  M3_BF16 = 1  /* bfloat16 stored as uint16 bit patterns */
} m3_dtype;

/* Order of the token and head axes of the prefill's x, B, C and y. */
typedef enum m3_layout {
  M3_TOKEN_MAJOR = 0, /* [Bt, L, H, R, .] (the default) */
  M3_HEAD_MAJOR = 1   /* [Bt, H, L, R, .]: each head's rows one contiguous run */
} m3_layout;

/*
 * Prefill (chunked, whole sequence per (batch, head)).
 *
 *   x       [Bt, L, H, R, P]  in_dtype   inputs x_t (R columns of length P)
 *   B, C    [Bt, L, H, R, N]  in_dtype   input / output projections
 *   dt      [Bt, L, H]        float32    Delta_t (> 0, already positive)
 *   lam     [Bt, L, H]        float32    lambda_t in [0, 1]
 *   A       [H]               float32    per-head scalar A (< 0); may be NULL
 *                                        when A_tok is given
 *   A_tok   [Bt, L, H]        float32    A per token (< 0), or NULL: the decay
 *                                        rate itself depending on the token
 *                                        ("La dualita", sec. "Mamba-3");
 *                                        alpha_t = exp(Delta_t A_tok_t)
 *   theta   [Bt, L, H, N/2]   float32    per-token rotation angles, or NULL
 *                                        for the real-valued SSM (no RoPE)
 *   omega   [Bt, L, N/2]      float32    alternative to theta: rotation
 *                                        rates per token and pair, shared by
 *                                        all heads; the angle
 *                                        is then theta_t = Delta_t * omega_t
 *                                        (the step times the rate, per head),
 *                                        formed on chip, which saves reading
 *                                        the per-head theta tensor.  Setting
 *                                        both theta and omega is
 *                                        M3_ERR_INVALID_ARG.
 *   Carry-in, each nullable (NULL = zeros, i.e. a fresh sequence):
 *   h0        [Bt, H, N, P]   float32    state before the first token
 *   Bprev_rot [Bt, H, R, N]   float32    rotated B of the token before
 *   xprev     [Bt, H, R, P]   in_dtype   x of the token before
 *   phi0      [Bt, H, N/2]    float32    cumulative angle before the first token
 *   Outputs:
 *   y         [Bt, L, H, R, P] in_dtype  required
 *   h_final   [Bt, H, N, P]   float32    state after token L-1 (nullable)
 *   Bprev_rot_out [Bt,H,R,N]  float32    rotated B_{L-1} (nullable)
 *   xprev_out [Bt, H, R, P]   in_dtype   x_{L-1} (nullable)
 *   phi_out   [Bt, H, N/2]    float32    Phi_{L-1} reduced modulo 2*pi into
 *                                        [-pi, pi] (nullable; needs theta or
 *                                        omega)
 * Sizes: Bt, L, H >= 1; N, P in {16, 32, 64, 128}; R a power of two <= 64;
 * combinations whose chunk tiles exceed the 160 KB LDS of a CU return
 * M3_ERR_UNSUPPORTED (fp32 with RoPE at N = 128, and fp32 at N = P = 128);
 * chunk = tokens per chunk Q of the chunked evaluation, 0 selects 64 / R.
 * A chunk tile holds 64 (token, rank) rows: the bf16 path takes only
 * Q = 64 / R; the fp32 path also any smaller power of two (the tile's rows
 * past Q R then stay empty).  Results do not depend on Q beyond rounding.
 * Outputs must not alias inputs.  Passing the carry-out of one call as the
 * carry-in of the next continues the sequence exactly.
 * workspace: optional, see m3_ssm_prefill_workspace_size; a non-NULL
 * workspace smaller than that size (or not 256-byte aligned) is
 * M3_ERR_INVALID_ARG.
 * layout: M3_TOKEN_MAJOR (0, the shapes above) or M3_HEAD_MAJOR (1): x, B, C
 * and y as [Bt, H, L, R, .] (dt, lam, A_tok, theta and omega keep the shapes
 * above).  The arithmetic is the same, so both layouts give identical bits;
 * head-major reads each (batch, head) walk as one contiguous run.  Other
 * values are M3_ERR_INVALID_ARG.
 * Prologue (optional steps fused in front of the core; all off when zero /
 * NULL), see m3_prologue below: the B and C given are then the raw
 * projections and dt the raw step.
 */
/*
 * The steps just before the SSM core, computed on chip ("Znakomstvo s
 * Mamba-3" (chernovdev.ru), sec. "Architecture and normalisation": RMS
 * normalisation of the B and C projections, by analogy with QK normalisation,
 * then learnable head-specific biases added to B and C after it; "Mamba-3:
 * un modello a spazio di stato progettato per l'inferenza" (cartesia.ai),
 * "Normalizzazioni" and "Addio convoluzione corta"):
 *   bc_norm      0 or 1: each (token, head, rank) row of B and of C, an
 *                N-vector, becomes row / sqrt(mean(row^2) + bc_eps) times the
 *                gain B_norm_w / C_norm_w [N] (NULL = 1); a row of zeros stays
 *                zero.  bc_eps >= 0.
 *   B_bias, C_bias  [H, R, N] float32 added after the normalisation (or to
 *                the raw B / C without it), or NULL.
 *   dt_softplus  0 or 1: Delta = softplus(dt + dt_bias[h]) (dt_bias [H] or
 *                NULL; needs dt_softplus), the step made positive on chip.
 * The rotation (RoPE) applies to the normalised and biased B and C, and the
 * carried B (Bprev_rot, Bprev_rot_out) is that rotated B.  Gains and biases
 * must be 4-byte aligned.  Other values are M3_ERR_INVALID_ARG.
 */
typedef struct m3_prologue {
  int32_t bc_norm;
  int32_t dt_softplus;
  float bc_eps;
  const float* B_norm_w;
  const float* C_norm_w;
  const float* B_bias;
  const float* C_bias;
  const float* dt_bias;
} m3_prologue;

typedef struct m3_prefill_args {
  int32_t Bt, L, H, P, N, R, chunk;
  int32_t in_dtype; /* m3_dtype */
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* A;
  const float* theta;
  const float* h0;
  const float* Bprev_rot;
  const void* xprev;
  const float* phi0;
  void* y;
  float* h_final;
  float* Bprev_rot_out;
  void* xprev_out;
  float* phi_out;
  void* workspace;        /* device scratch of workspace_bytes (256-byte aligned), or NULL */
  size_t workspace_bytes;
  const float* omega;     /* [Bt, L, N/2] angular rates, or NULL (see above) */
  const float* A_tok;     /* [Bt, L, H] A per token, or NULL (see above) */
  int32_t layout;         /* m3_layout of x, B, C, y (see above) */
  m3_prologue pro;        /* steps fused in front of the core (zeros = none) */
} m3_prefill_args;

int m3_ssm_prefill(const m3_prefill_args* args, void* stream);

/* Device scratch that lets m3_ssm_prefill use more of the GPU; 0 when it
 * would not (fp32 inputs, or at least half as many (batch, head) units as the
 * device has compute units, or sequences shorter than 8 chunks).
 *   With fewer units than that, a bf16 prefill given a workspace of this size
 * first walks the first half of every sequence for its state only (the
 * chunked evaluation of "La dualita: Mamba-2 e Mamba-3", sec. "Perche
 * conviene", needs only the state to hand over), then computes both halves at
 * once, the second one starting from that state -- the same carry that
 * continues a sequence across calls.  When the first half has at least 8
 * chunks, its state walk itself runs as two parts at once, the second from a
 * zero state and zero angle, and a small kernel joins them (the recurrence is
 * linear in the state and the rotations compose).  Results agree with the
 * unsplit call to rounding (the handed-over carry is exact fp32, where the
 * unsplit walk passes the pending term through bf16).  With workspace == NULL
 * the call runs unsplit.
 * The workspace holds the state and carry of two segments
 * (Bt*H*2*(4NP + 4RN + 2RP + 2N) bytes, rounded); it is overwritten by every
 * call, so concurrent calls need their own.  Depends only on the shape
 * fields (and the current device), not on pointers. */
size_t m3_ssm_prefill_workspace_size(const m3_prefill_args* args);

/*
 * m3_ssm_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and kernels as m3_ssm_prefill, except that
 * `workspace` must be NULL and `workspace_bytes` 0: where the call would use
 * the optional workspace (m3_ssm_prefill_workspace_size > 0) it uses instead
 * a static device buffer of M3_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends.  Nothing is allocated
 * by the call (the buffer's address is looked up once per device, with the
 * device current, on the first call there).  A call whose workspace size
 * exceeds M3_NOALLOC_SCRATCH_BYTES (16 MiB) returns M3_ERR_SCRATCH without
 * launching: on a 256-CU device every split shape with N * P <= 128 * 64
 * fits (at most ~8.6 MB); at N = P = 128 calls with more than ~120 (batch,
 * head) units do not (they can use m3_ssm_prefill with a workspace).  The
 * buffer needs no clearing (each call writes what it reads), but every call
 * on one device shares it: calls that overlap in time on one device (two
 * streams, two host threads) race and give undefined results; serialise
 * them, or use m3_ssm_prefill with a workspace per stream.
 */
#define M3_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int m3_ssm_prefill_noalloc(const m3_prefill_args* args, void* stream);

/*
 * One decode token against a resident state (the same token update as the
 * prefill, "La dualita", sec. "Mamba-3": MIMO update on an unchanged state).
 *
 *   In/out (updated in place):
 *   h         [Bt, H, N, P]   float32    state
 *   phi       [Bt, H, N/2]    float32    cumulative angle (NULL iff neither
 *                                        theta nor omega is given);
 *                                        stored reduced modulo 2*pi
 *   Bprev_rot [Bt, H, R, N]   float32    rotated B of the previous token
 *   xprev     [Bt, H, R, P]   in_dtype   x of the previous token
 *   In:
 *   x [Bt,H,R,P], B, C [Bt,H,R,N] (in_dtype); dt, lam [Bt,H] float32;
 *   A [H] float32, or A_tok [Bt,H] float32 (A per (batch, head) for this
 *   token; then A may be NULL); theta [Bt,H,N/2] float32 or NULL, or instead
 *   omega [Bt,N/2] float32 (rates shared by the heads: theta = dt * omega).
 *   Out: y [Bt, H, R, P] in_dtype.
 * Sizes: N, P in {16, 32, 64, 128}; R in 1..16.  A fresh sequence starts with
 * h = 0 (or any state), Bprev_rot = 0, xprev = 0, phi = 0.
 * With bf16 inputs, N in {32, 64, 128} and P in {64, 128} the rank-2R update
 * and the readout run on the matrix cores ("Znakomstvo s Mamba-3", sec. 3: with
 * MIMO the update is a matrix product); other shapes and fp32 inputs on the
 * vector ALUs.  Both keep the state in fp32.
 * pro: the same prologue as the prefill's (B, C, dt raw), so that a decode
 * continues a prefill that used it.
 */
typedef struct m3_decode_args {
  int32_t Bt, H, P, N, R;
  int32_t in_dtype; /* m3_dtype */
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
  const float* A_tok; /* [Bt, H] A of this token, or NULL */
  const float* omega; /* [Bt, N/2] rotation rates shared by the heads, or NULL */
  m3_prologue pro;    /* steps fused in front of the core (zeros = none) */
} m3_decode_args;

int m3_ssm_decode_step(const m3_decode_args* args, void* stream);

/*
 * Backward pass of the prefill: gradients of a loss that reaches the core
 * through y (upstream gradient dy) and the final state (dh_final), by reverse-
 * mode differentiation of the chunked evaluation ("La dualita: Mamba-2 e
 * Mamba-3", sec. "Perche conviene: i tensor core") of the recurrence
 * ("Znakomstvo s Mamba-3", sec. 1-3); the pages print no backward pass.  The
 * carry-out (rotated B, x, angle) is not differentiated.
 *
 *   Forward inputs (as given to m3_ssm_prefill, token-major): x, B, C [Bt, L,
 *   H, R, .] bf16; dt, lam [Bt, L, H]; A [H] or A_tok [Bt, L, H]; theta [Bt, L,
 *   H, N/2] or NULL; carry-in h0, Bprev_rot, xprev, phi0 (nullable).
 *   Upstream: dy [Bt, L, H, R, P] bf16; dh_final [Bt, H, N, P] float32 or NULL.
 *   Gradients (outputs): dx, dB, dC (bf16, shapes of x, B, C); ddt, dlam [Bt,
 *   L, H] float32; dA: [H] when A is given (summed over batch and tokens),
 *   [Bt, L, H] when A_tok is given; dtheta [Bt, L, H, N/2] (required iff
 *   theta); dh0 [Bt, H, N, P], dBprev_rot [Bt, H, R, N] (float32), dxprev
 *   [Bt, H, R, P] (bf16), dphi0 [Bt, H, N/2]: each nullable.
 *   workspace: required, m3_ssm_prefill_backward_workspace_size bytes,
 *   256-byte aligned (the shifted state, in bf16, and the angle entering
 *   every chunk of every (batch, head), written by the kernel's forward
 *   state walk; with at most half as many (batch, head) units as the
 *   device has compute units and at least 8 chunks the sequence is split in
 *   two walked at once, and the workspace also holds the values joined at
 *   the split: so its size depends on the current device).
 * Sizes: bf16 only (M3_ERR_UNSUPPORTED for float32); N, P in {16, 32, 64,
 * 128} whose tiles fit the LDS of a CU (N = P = 128 does not:
 * M3_ERR_UNSUPPORTED); R a power of two <= 8; chunks of 64 / R tokens.
 * Gradients are deterministic (no atomics).
 */
typedef struct m3_backward_args {
  int32_t Bt, L, H, P, N, R;
  int32_t in_dtype;       /* m3_dtype: M3_BF16 */
  const void* x;
  const void* B;
  const void* C;
  const float* dt;
  const float* lam;
  const float* A;
  const float* A_tok;
  const float* theta;
  const float* h0;
  const float* Bprev_rot;
  const void* xprev;
  const float* phi0;
  const void* dy;
  const float* dh_final;
  void* dx;
  void* dB;
  void* dC;
  float* ddt;
  float* dlam;
  float* dA;
  float* dtheta;
  float* dh0;
  float* dBprev_rot;
  void* dxprev;
  float* dphi0;
  void* workspace;
  size_t workspace_bytes;
} m3_backward_args;

size_t m3_ssm_prefill_backward_workspace_size(const m3_backward_args* args);
int m3_ssm_prefill_backward(const m3_backward_args* args, void* stream);

/*
 * Inclusive cumulative rotation angle ("Znakomstvo s Mamba-3", sec. 2: the
 * rotations are aggregated over all time steps):
 *   phi[b, t, h, j] = phi0[b, h, j] + sum_{s <= t} theta[b, s, h, j].
 * theta, phi: [Bt, L, H, npairs] float32; phi0: [Bt, H, npairs] or NULL.
 * H * npairs must be a multiple of 4.  phi is the plain fp32 running sum
 * (no modular reduction).  phi must not alias theta.
 */
int m3_rope_angles_cumsum(const float* theta, const float* phi0, float* phi,
                          int32_t Bt, int32_t L, int32_t H, int32_t npairs,
                          void* stream);

/* Static description of a status code (never NULL). */
const char* m3_status_string(int status);

/* Library version, e.g. "0.1.0". */
const char* m3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M3SSM_H */
