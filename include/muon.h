/*
 * muon.h - C ABI of the MI355X (gfx950) Muon step library, libmuon.so.
 *
 * The Muon step for a GPT's 2-D weight matrices, as described by page 1
 * (web3.cnoyu.systems review of karpathy/autoresearch's train.py, paragraph
 * on the Muon half of MuonAdamW): Nesterov momentum on the gradient, then a
 * 5-step Newton-Schulz iteration towards the orthogonal polar factor
 * (tall: A = X^T X, X <- aX + X(bA + cA^2); wide: A = X X^T,
 * X <- aX + (bA + cA^2)X; per-step coefficients from a precomputed table),
 * whose result is the update direction for the weights.  Page 1 also says
 * the momentum buffer has the parameter's shape and is stacked per shape
 * group; this library groups the matrices of a call by oriented shape.
 *
 * Conventions shared by every entry point:
 *  - Matrices are dense row-major; "rows x cols" is the parameter's shape.
 *    The oriented shape is m = min(rows, cols), n = max(rows, cols).
 *  - Device pointers are caller-owned device memory; host pointers (shape
 *    arrays, pointer arrays, scales, coefficient tables) are read during the
 *    call only.  The library allocates no device memory: scratch comes from
 *    the caller's workspace, sized by the matching *_workspace_bytes query
 *    (muon_step_static instead uses a fixed area the library holds).
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *    results are valid once the caller synchronises that stream.  The
 *    library never synchronises the device.
 *  - All argument checks run on the host before anything is enqueued, so a
 *    call that returns MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED or
 *    MUON_ERR_WORKSPACE had no side effect.  MUON_ERR_HIP means a launch
 *    failed; part of the work may already be enqueued.
 *  - Non-finite values in the data propagate; they are not checked.
 *  - Range: the 1/(||u|| + eps) normalisation is applied inside the first
 *    Newton-Schulz products, so those accumulate products of the raw
 *    entries of u (the momentum-corrected gradient) in fp32: entries of
 *    magnitude between about 1e-18 and 1e16 keep full accuracy (the tests
 *    cover 2^-60 to 2^55); far larger ones can overflow fp32 in the first
 *    Gram matrix, far smaller ones lose precision to fp32's normal range.
 *  - Repeated calls on the same inputs give bitwise-identical results (all
 *    reductions use a fixed order; there are no floating-point atomics).
 *  - Calls are re-entrant when they use distinct workspaces.
 *  - A step whose chunks are all small runs them concurrently: on the
 *    caller's stream and up to three library-owned streams per device
 *    (default priority), forked off the caller's stream with an event and
 *    joined back to it before the call returns, so stream order and graph
 *    capture see one step as usual.
 *  - The step entry points (muon_step, muon_step_ex, muon_step_static) work
 *    on the calling thread's current device, whose library streams and
 *    static scratch they use: a `stream` that belongs to another device
 *    returns MUON_ERR_INVALID_ARG before anything is enqueued.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  MUON_BF16 is bfloat16 (round-to-nearest-even on every
 * fp32 -> bf16 conversion), MUON_FP32 is IEEE binary32. */
typedef enum { MUON_BF16 = 0, MUON_FP32 = 1 } muon_dtype;

/* One row of the Newton-Schulz coefficient table: step k computes
 * X <- a_k X + (b_k A + c_k A^2) X in the wide form. */
typedef struct { float a, b, c; } muon_coeff;

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, aliasing */
  MUON_ERR_UNSUPPORTED = -2, /* valid request the library does not implement */
  MUON_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned */
  MUON_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} muon_status;

#define MUON_MAX_STEPS 64          /* n_steps must lie in [1, MUON_MAX_STEPS] */
#define MUON_MAX_ELEMENTS (1LL << 31) /* per matrix, after padding to the tile grid */
#define MUON_WORKSPACE_ALIGN 256   /* required alignment of `workspace`, bytes */
#define MUON_PTR_ALIGN 16          /* required alignment of every matrix pointer */

/* ---------------------------------------------------------------- queries */

/* Text for a muon_status value (static storage; never NULL). */
const char* muon_status_string(int status);

/* Bytes of workspace muon_orthogonalize needs for `batch` matrices of
 * rows x cols with the given compute precision.  0 for invalid sizes. */
size_t muon_orthogonalize_workspace_bytes(int batch, int rows, int cols, int compute);

/* Bytes of workspace muon_step needs for the n matrices rows[i] x cols[i]:
 * the largest of its chunks (matrices of one oriented shape, at most 64 per
 * chunk) when the chunks run one after the other, their sum when a small
 * step runs them concurrently (every chunk small enough to leave most of the
 * chip idle on its own).  0 for invalid sizes or n == 0. */
size_t muon_step_workspace_bytes(int n, const int* rows, const int* cols, int compute);

/* The grouping muon_step uses (page 1: momentum stacked per shape group).
 * Matrices are grouped by oriented shape (min(rows,cols), max(rows,cols)),
 * groups numbered in order of first appearance.  Writes group_of[i] for
 * i < n and, for g < *n_groups, group_m[g], group_n[g], group_count[g];
 * the group arrays must hold n entries.  Pure host code; no HIP call. */
int muon_plan_groups(int n, const int* rows, const int* cols, int* group_of,
                     int* group_m, int* group_n, int* group_count, int* n_groups);

/* ---------------------------------------------------------- computations */

/* Orthogonalise a batch of same-shape matrices: for each matrix G,
 *   X_0 = G / (||G||_F + eps);  for k < n_steps:  X_{k+1} = a_k X_k + (b_k A_k + c_k A_k^2) X_k
 * with A_k = X_k X_k^T (wide or square) and the transposed forms for tall
 * matrices (page 1, Newton-Schulz paragraph), and writes out = X_{n_steps}.
 *   in, out       device, `batch` matrices rows x cols, matrix i at
 *                 element offset i * batch_stride (batch_stride >= rows*cols);
 *                 out may alias in exactly (same pointer and same dtype); any
 *                 other overlap returns MUON_ERR_INVALID_ARG.
 *   in_dtype      MUON_BF16 or MUON_FP32; out_dtype likewise.
 *   coeffs        host, n_steps rows (copied during the call).
 *   eps           >= 0, finite (the step's default is 1e-7).
 *   compute       MUON_BF16: bf16 MFMA operands with fp32 accumulation; X is
 *                 carried between steps as hi = bf16(x) and one signed byte,
 *                 x - hi in 1/256 of hi's bf16 spacing (16 significant bits,
 *                 3 bytes) for the a*X term; for matrices whose
 *                 padded shape has n >= 4m and m >= 2048, the A of steps 1
 *                 and 3 is formed as Q A Q from the step before (Q = aI + B;
 *                 equal to X X^T in exact arithmetic).  MUON_FP32: fp32
 *                 throughout, A = X X^T at every step.
 *   workspace     device, >= muon_orthogonalize_workspace_bytes(...) bytes,
 *                 MUON_WORKSPACE_ALIGN-aligned; contents on entry are ignored.
 * batch == 0 returns MUON_OK with nothing enqueued. */
int muon_orthogonalize(const void* in, int in_dtype, void* out, int out_dtype,
                       int batch, int rows, int cols, long long batch_stride,
                       const muon_coeff* coeffs, int n_steps, float eps, int compute,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One Muon step on n matrices of any mix of shapes (page 1: Nesterov
 * momentum, Newton-Schulz orthogonalisation, the orthogonal factor as the
 * update direction).  For each matrix i, in place:
 *   momentum[i] <- mu * momentum[i] + g_i
 *   u           =  g_i + mu * momentum[i]
 *   O           =  the muon_orthogonalize result for u
 *   params[i]   <- params[i] - lr * scale[i] * O
 *   rows, cols     host arrays of n shapes.
 *   params         host array of n device pointers, fp32 rows x cols, in/out.
 *   param_dtype    MUON_FP32 (bf16 parameters return MUON_ERR_UNSUPPORTED).
 *   grads          host array of n device pointers, read only.
 *   grad_dtype     MUON_BF16 or MUON_FP32.
 *   momentum       host array of n device pointers, fp32 rows x cols, in/out.
 *   scale          host array of n per-matrix multipliers of lr.
 *   coeffs, n_steps, eps, compute, workspace: as for muon_orthogonalize,
 *                  with the workspace from muon_step_workspace_bytes.
 * params[i], grads[i] and momentum[i] must not overlap one another or the
 * workspace, and no params or momentum buffer may overlap any other
 * matrix's buffers (gradients may share memory with each other)
 * (MUON_ERR_INVALID_ARG).
 * n == 0 returns MUON_OK with nothing enqueued. */
int muon_step(int n, const int* rows, const int* cols,
              void* const* params, int param_dtype,
              const void* const* grads, int grad_dtype,
              float* const* momentum, float mu, float lr, const float* scale,
              const muon_coeff* coeffs, int n_steps, float eps, int compute,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Page 1, in the paragraph after the Muon one, adds two things on top of the
 * plain step.  NorMuon: after orthogonalisation, per-row (or, by the aspect
 * ratio, per-column) second-moment estimates of the update, kept as an
 * exponential moving average, give each output dimension its own step size.
 * Cautious weight decay: only parameters whose update direction agrees in
 * sign with the parameter decay, mask = (update * param) >= 0.  The page
 * gives no constants; this library takes them from the caller and reads:
 *   - NorMuon statistics on the shorter side of the matrix (per row of a wide
 *     or square matrix, per column of a tall one), the second moment being
 *     the mean of O^2 along the longer side;
 *     v' = beta2 * v + (1 - beta2) * mean(O^2), no bias correction;
 *     O' = O / (sqrt(v') + normuon_eps);
 *   - decoupled decay on the parameter before the update:
 *     W' = W - lr*scale*O' - lr*weight_decay*mask*W, mask = (O'*W >= 0) when
 *     cautious, 1 otherwise. */
typedef struct {
  float weight_decay;  /* finite, >= 0; 0 disables the decay */
  int cautious;        /* 0 or 1 */
  int normuon;         /* 0 or 1: NorMuon scaling with `second_moment` */
  float beta2;         /* NorMuon EMA factor, in [0, 1] */
  float normuon_eps;   /* NorMuon: finite, >= 0.  With 0, a row whose v' is 0
                          (a zero row of O and a zero v, or beta2 = 1 and a
                          zero v) divides by zero and its values become
                          non-finite, as the formula gives; a positive value
                          avoids that */
} muon_options;

/* Workspace bytes of muon_step_ex for these shapes and options (NULL
 * options: as muon_step_workspace_bytes).  0 for invalid sizes or n == 0. */
size_t muon_step_ex_workspace_bytes(int n, const int* rows, const int* cols, int compute,
                                    const muon_options* options);

/* muon_step with page 1's additions.  Arguments as for muon_step, plus:
 *   second_moment  host array of n device pointers, fp32, min(rows[i], cols[i])
 *                  elements each, in/out (read and written only when
 *                  options->normuon; may be NULL otherwise).  Each is
 *                  4-byte aligned and overlaps none of params[i], grads[i],
 *                  momentum[i] and the workspace.
 *   options        NULL: exactly muon_step.
 * For each matrix i: momentum and orthogonalisation as in muon_step, then
 * (normuon) O' and v' as above, then the decayed weight update with O'.
 * Invalid options (negative or non-finite weight_decay or normuon_eps,
 * beta2 outside [0, 1], flags other than 0/1, missing second moments)
 * return MUON_ERR_INVALID_ARG before anything is enqueued. */
int muon_step_ex(int n, const int* rows, const int* cols,
                 void* const* params, int param_dtype,
                 const void* const* grads, int grad_dtype,
                 float* const* momentum, float* const* second_moment,
                 float mu, float lr, const float* scale,
                 const muon_coeff* coeffs, int n_steps, float eps, int compute,
                 const muon_options* options,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * muon_step with no workspace argument: its scratch is a fixed area of
 * MUON_STATIC_SCRATCH_BYTES of device memory inside the library, one per GPU
 * (the calling thread's current device; `stream` must belong to it), held
 * from the first call on that GPU until the process ends.  The call itself
 * allocates nothing.  It runs the step's chunks (up to 64 matrices of one
 * oriented shape each) one after the other, never concurrently, so the area
 * must hold the largest chunk: muon_orthogonalize_workspace_bytes of that
 * chunk's count and oriented shape (at compute), which for a step with a
 * single chunk is its muon_step_workspace_bytes.  A step with a larger chunk
 * returns MUON_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses that GPU's one area, which keeps the
 * last call's contents (the step reads none of them): calls that overlap in
 * time on one GPU (several streams, or host threads, at once) race and must
 * be serialised by the caller.  Otherwise exactly muon_step: the same checks,
 * the same kernels, bitwise the same results. */
#define MUON_STATIC_SCRATCH_BYTES (256ull << 20)
int muon_step_static(int n, const int* rows, const int* cols,
                     void* const* params, int param_dtype,
                     const void* const* grads, int grad_dtype,
                     float* const* momentum, float mu, float lr, const float* scale,
                     const muon_coeff* coeffs, int n_steps, float eps, int compute,
                     hipStream_t stream);

/* ------------------------------------------------------------ measurement */

/* Kernel classes reported by the timing log. */
typedef enum {
  MUON_K_PREP = 0,   /* momentum (or input read), norm partials, oriented X_0 */
  MUON_K_NORM = 1,   /* per-matrix 1 / (||u||_F + eps) */
  MUON_K_GRAM = 2,   /* A = X X^T, one triangle, mirrored */
  MUON_K_POLY = 3,   /* B = b A + c A^2 */
  MUON_K_UPDATE = 4, /* X <- a X + B X, steps before the last */
  MUON_K_FINAL = 5,  /* last step's a X + B X, written to the weights or output */
  MUON_K_NORMUON = 6, /* NorMuon row statistics and second-moment update */
  MUON_K_APPLY = 7,  /* weight update as its own pass (after NorMuon) */
  MUON_K_GRAMQ = 8   /* one of the two launches forming A as Q A Q, Q = aI + B */
} muon_kernel_kind;

typedef struct {
  int kind;        /* muon_kernel_kind */
  int m, n;        /* oriented shape of the launch's matrices */
  int batch;       /* matrices in the launch */
  int step;        /* Newton-Schulz step, -1 for PREP and NORM */
  float ms;        /* elapsed time between HIP events around the launch */
  double flops;    /* counted flops: GRAM 2m^2n, POLY 2m^3, UPDATE/FINAL 2m^2n per matrix
                      (GRAMQ: m^2n per launch, the Gram's count split over its two) */
  double bytes;    /* algorithmic HBM bytes of the launch: each operand, input
                      and output of the launch read or written once */
  double exec_flops; /* flops the launch's MFMAs execute: its tiles over the
                        padded shape (lower-triangle tiles for GRAM, POLY and
                        GRAMQ) */
} muon_timing_record;

/* Turn per-launch HIP-event timing on (1) or off (0) for later calls in
 * this process.  Events are recorded on the call's stream around every
 * kernel launch.  Returns the previous setting. */
int muon_timing_enable(int on);

/* Wait for the recorded events, write up to `cap` records (oldest first)
 * to `out`, set *n_out to the number written, and clear the log.
 * Returns MUON_OK or MUON_ERR_HIP. */
int muon_timing_read(muon_timing_record* out, int cap, int* n_out);

/* Probes of what the chip sustains, timed by the caller next to the step
 * (HIP events on `stream`, around the one kernel each call enqueues).  Not
 * part of the Muon step; they compute nothing of it.
 *   muon_probe_mfma_bf16  `blocks` workgroups of 8 waves, each wave running
 *       `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16 on register
 *       operands, no memory traffic: the launch performs exactly
 *       blocks * 8 * iters * 4 * 32768 flops.  `sink` is device memory of
 *       blocks * 512 floats (overwritten; the values mean nothing).
 *   muon_probe_copy  copies `bytes` (a multiple of 16; src and dst device
 *       pointers, 16-byte aligned, not overlapping) in 16-byte accesses with
 *       `blocks` workgroups of 256 threads: 2 * bytes of HBM traffic.
 * Both return MUON_ERR_INVALID_ARG for bad arguments (nothing enqueued) and
 * MUON_ERR_HIP if the launch fails. */
int muon_probe_mfma_bf16(int blocks, int iters, float* sink, hipStream_t stream);
int muon_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MUON_H */
