/*
 * dion.h -- C ABI of the MI355X (gfx950) Gram Newton-Schulz orthogonalization
 * library: the orthogonalization of momentum matrices inside a Muon-style
 * optimizer step, done the Dion3 way.
 *
 * What is computed, and where it is stated
 *   "Dion3: Full-Stack Orthogonal Updates" (arXiv abstract): Gram
 *   Newton-Schulz cuts the FLOPs of orthogonalization, symmetric kernels
 *   exploit the symmetry of the Gram products, megabatching groups the
 *   matrices, and the update rule orthogonalizes only a fraction of the
 *   momentum matrix's rows each step.
 *   "Dion3：全栈正交更新" (Chinese summary), section 方法 / 核心模块: the Gram
 *   form with restarts and safety factors; upper-triangle-only symmetric GEMM
 *   with a transpose epilogue and fused GEMM+add; the row rule (e.g. 1/8 of
 *   the rows) where the other rows keep the raw momentum update, with error
 *   feedback and finite-precision handling.  Section 输入输出流程: momentum
 *   update, then row selection, then Gram Newton-Schulz, then the weight
 *   update (the weight update is not part of this library).
 *
 * Per matrix M (R x C, row-major, densely packed), with k = ceil(row_frac*R)
 * (clamped to [1, R]; x = row_frac*R is shrunk by a relative 1e-6 first):
 *   1. rows are ranked by squared L2 norm: the exact sum of the squares of
 *      the stored values, rounded once to the nearest double (ties to even),
 *      which no summation order changes; larger first, equal keys to the
 *      lower row index; the top k are selected and kept in ascending row
 *      order (all rows when row_frac = 1);
 *   2. S = M[selected]; if S is tall (k > C) it is transposed so that the
 *      Gram matrix is formed on the smaller side m = min(k, C);
 *   3. X = S / ||S||_F (a zero S gives zero output rows);
 *   4. K iterations of X <- (a I + b A + c A^2) X with A = X X^T, run in Gram
 *      form on G = X X^T and the accumulated factor Q; the safety factor s
 *      rescales the argument at every iteration, (a, b, c) -> (a/s, b/s^3,
 *      c/s^5); a restart after iteration k (never after the last) re-forms G
 *      from the current iterate and resets Q;
 *   5. out[selected] = the result (transposed back if tall),
 *      out[other rows] = M[other rows], cast to the output dtype
 *      (round to nearest even for bf16).  No learning-rate or shape scaling.
 *
 * Conventions for every entry point
 *   - Matrix arguments are HOST arrays of `batch` DEVICE pointers.  Every
 *     device buffer is owned by the caller.  The library allocates no device
 *     memory and keeps no device state between calls: all scratch lives in
 *     the caller's `workspace` (device memory, at least
 *     dion_workspace_size() bytes, 256-byte aligned).  The one exception is
 *     dion_orth_batched_noalloc, whose scratch is a fixed array that each
 *     device holds for the life of the process.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work on it and return without waiting for the device: the plan header
 *     goes up through a ring of pinned host buffers, each refilled only once
 *     its copy has completed, or as kernel arguments while all of them are in
 *     flight.  Host arrays are only read during the call.  Two calls must not
 *     share a workspace concurrently.
 *   - Errors are detected on the host before any launch and returned as a
 *     negative dion_status; dion_last_error() gives a message for the calling
 *     thread.  NaN/Inf inputs are not checked: the output is unspecified.
 */
#ifndef DION_H
#define DION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DION_OK = 0,
  DION_E_INVAL = -1,        /* bad argument (shape, count, fraction, aliasing ...) */
  DION_E_UNSUPPORTED = -2,  /* valid but not implemented combination */
  DION_E_WORKSPACE = -3,    /* workspace NULL, too small or misaligned */
  DION_E_HIP = -4           /* a HIP runtime call or kernel launch failed */
} dion_status;

/* Storage dtype of the momentum / gradient / output matrices.  DION_FP16 is
 * accepted by dion_orth_batched and the phase entry points (inputs and
 * outputs in fp16, processed like bf16: the values are exact in one fp16
 * term); the row-subset step takes bf16 or fp32 gradients. */
typedef enum { DION_BF16 = 0, DION_FP32 = 1, DION_FP16 = 2 } dion_dtype;

/* Arithmetic of the iteration.
 *   DION_PREC_MFMA16: fp16 MFMA with fp32 accumulation; operands carry
 *     power-of-two scales, and every product whose rounding the iteration
 *     amplifies uses a two-term (hi + lo) fp16 split.  Relative Frobenius
 *     error against the exact result: a few 1e-3 on low-rank-plus-noise
 *     momentum at 5 to 8 iterations (gate 2e-2); it grows with n_iter, as
 *     each iteration amplifies the rounding in the small singular directions
 *     (about 1.4e-2 at 12 and 2e-2 at 16 iterations on small blocks).  A
 *     call that would run a matrix on this path with more than 12 iterations,
 *     with slopes a_k / s multiplying to more than 3.4445^12, or with
 *     keep_schedule and a run of more than two iterations between restarts
 *     where a run is longer than 5 iterations or the slopes multiply to more
 *     than 3.4445^6 is refused (DION_E_UNSUPPORTED); DION_PREC_FP64 takes
 *     it.  Matrices with a Gram side of at most 64 and a long side of at
 *     most 1024, or a Gram side of at most 16, run in fp64 in one launch on
 *     every precision setting.
 *   DION_PREC_FP64: fp64 arithmetic throughout (error ~1e-12; gate 1e-4).
 *   DION_PREC_AUTO: FP64 for DION_FP32 inputs of dion_orth_batched, MFMA16
 *     otherwise (bf16 and fp16). */
typedef enum { DION_PREC_AUTO = 0, DION_PREC_MFMA16 = 1, DION_PREC_FP64 = 2 } dion_precision;

typedef struct {
  int32_t rows;
  int32_t cols;
} dion_shape;

/* Hyper-parameters of the orthogonalization (shared by the whole batch).
 *   ns_coeffs     host array of n_coeff_sets * 3 floats (a, b, c); NULL means
 *                 the fixed quintic (3.4445, -4.7750, 2.0315)
 *   n_coeff_sets  1 (same triple every iteration) or n_iter
 *   n_iter        K >= 1 (at most 64; see DION_PREC_MFMA16 for that path's range)
 *   restart_every restart after every restart_every-th iteration (0 = none)
 *   restart_mask  if nonzero, bit (k-1) set = restart after iteration k;
 *                 overrides restart_threshold and restart_every.  Never
 *                 applied after iteration K.
 *   safety        s > 0
 *   row_frac      in (0, 1]
 *   precision     a dion_precision value
 *   ef_carry      row-subset steps only: 0 = the buffer keeps the momentum and
 *                 unselected rows apply it raw (the pages' "raw momentum
 *                 update"); 1 = the carry form of error feedback: the buffer
 *                 takes the gradient undecayed, B = fl32(E + G), only the
 *                 selected (captured) rows decay to fl32(beta * B), and
 *                 unselected rows contribute a zero update.  Ignored elsewhere.
 *   restart_threshold  tau >= 0 (0 = off); with no mask it overrides
 *                 restart_every: a restart follows the iteration at which the
 *                 product of (a_k / s)^2 since the last restart first reaches
 *                 tau.  (a_k/s)^2 is the factor by which one iteration scales
 *                 an error of the Gram matrix in its smallest singular
 *                 directions, where the spurious negative eigenvalues that
 *                 restarts remove appear (Dion3 summary, 局限: restart
 *                 threshold).  With the fixed quintic, tau = 100 restarts
 *                 every 2 iterations.  Evaluated on the host from the
 *                 coefficients: no device synchronization.
 *   keep_schedule MFMA16 path only.  0 (default): a run of more than two
 *                 iterations between restarts is cut by an extra restart after
 *                 every second iteration of the run.  A restart gives the same
 *                 result in exact arithmetic; the short runs take one-term
 *                 fp16 operands in the m x m chain (with the fixed quintic and
 *                 bf16 Llama-shaped inputs, relative error about 5e-3).
 *                 1: run the schedule as given; runs longer than two
 *                 iterations take two-term operands (about 1e-3 without
 *                 restarts, at about three times the MFMA work of those
 *                 runs).  Two terms hold the rounding of such a run only
 *                 while few iterations follow it: the slopes a_k / s of the
 *                 whole schedule must multiply to at most 3.4445^6 (six
 *                 iterations of the fixed quintic) and no run may exceed 5
 *                 iterations, else the call is refused.  dion_restart_points and the useful-FLOP count
 *                 follow the schedule as given either way. */
typedef struct {
  const float* ns_coeffs;
  int32_t n_coeff_sets;
  int32_t n_iter;
  int32_t restart_every;
  uint32_t restart_mask;
  float safety;
  float row_frac;
  int32_t precision;
  float restart_threshold;
  int32_t ef_carry;
  int32_t keep_schedule;
} dion_ns_params;

/* The iterations after which this parameter set restarts (host only, no
 * device work): writes up to `cap` 1-based iteration indices, ascending, to
 * `after` (may be NULL when cap = 0) and returns how many there are, or a
 * negative dion error code for invalid parameters. */
int dion_restart_points(const dion_ns_params* p, int32_t* after, int32_t cap);

/* Bytes of device workspace needed by dion_orth_batched for this batch
 * (pure function of its arguments; 0 on invalid arguments).  For
 * dion_rowsubset_step pass dtype = DION_FP32 and precision MFMA16 or AUTO. */
size_t dion_workspace_size(const dion_shape* shapes, int32_t batch, int32_t dtype,
                           const dion_ns_params* p);

/* Workspace for running the batch within at most `cap` bytes (the megabatch
 * of the Dion3 abstract, sized to fit beside the model's own memory): the
 * full size when it fits, else the largest of the waves the call will run
 * (see dion_orth_batched); 0 if one matrix alone needs more than `cap`, or on
 * invalid arguments.  Like dion_workspace_size it also covers the row-subset
 * step for dtype = DION_FP32. */
size_t dion_workspace_size_capped(const dion_shape* shapes, int32_t batch, int32_t dtype,
                                  const dion_ns_params* p, size_t cap);

/* Orthogonalize a batch of momentum matrices in one megabatched pass.
 * Workspace: dion_workspace_size() bytes run the batch as one wave (one
 * grouped launch per phase over every matrix).  A smaller workspace runs it as
 * consecutive waves of matrices, each wave's plan fitting workspace_bytes, one
 * after another on the stream, with the same kernels and tile sizes: the
 * results are bit-identical.  DION_E_WORKSPACE if one matrix alone does not
 * fit (dion_workspace_size_capped gives the size a cap leads to).
 *   M[i]     device, R_i x C_i of `dtype`, read only
 *   out[i]   device, R_i x C_i of `dtype`, must not overlap any M[j]
 *   sel_idx  optional device int32 buffer of sum_i k_i entries: receives each
 *            matrix's selected rows (ascending), matrices in batch order
 * Pages: Dion3 abstract (Gram Newton-Schulz, symmetric kernels, megabatching,
 * row fraction); Dion3 summary, 方法 / 核心模块. */
int dion_orth_batched(const void* const* M, void* const* out, const dion_shape* shapes,
                      int32_t batch, int32_t dtype, const dion_ns_params* p,
                      int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as dion_orth_batched, with its scratch in a fixed array inside the
 * library instead of a caller's workspace.  It calls no allocating routine:
 * the plan header reaches the device as kernel arguments.
 *   Limit: the batch's dion_workspace_size() must not exceed
 *   DION_NOALLOC_SCRATCH_BYTES (256 MiB), else DION_E_WORKSPACE before any
 *   launch.  Each device the library runs on holds one such array until the
 *   process ends, shared by every call on that device: calls that overlap in
 *   time on one device (other streams, other threads) race on it and must be
 *   serialized by the caller.  Nothing in it needs to start at zero.
 *   Arguments as dion_orth_batched. */
#define DION_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int dion_orth_batched_noalloc(const void* const* M, void* const* out, const dion_shape* shapes, int32_t batch,
                              int32_t dtype, const dion_ns_params* p, int32_t* sel_idx, void* stream);

/* Same operation with a flat parameter list: one coefficient triple (NULL =
 * the fixed quintic), restarts every restart_every iterations, AUTO precision. */
int dion_orth_batched_simple(const void* const* M, void* const* out, const dion_shape* shapes,
                             int32_t batch, int32_t dtype, const float* ns_coeffs,
                             int32_t n_iter, int32_t restart_every, float safety,
                             float row_frac, void* workspace, size_t workspace_bytes,
                             void* stream);

/* One step of the row-subset rule with its fp32 momentum / error-feedback
 * buffer (Dion3 summary, 核心模块 "Dion3 更新规则" bullet and 输入输出流程):
 *   E[i]     device fp32 R x C, updated in place:
 *            E <- fl32(fl32(beta * E) + grad), two separately rounded fp32
 *            operations (no fused multiply-add)
 *   grad[i]  device R x C of grad_dtype (bf16 or fp32), read only
 *   out[i]   device bf16 R x C: the orthogonalized selected rows of the new E,
 *            the raw new E (rounded to bf16) in the other rows
 *   p        as above; p->precision must be AUTO or MFMA16
 * Workspace: dion_workspace_size(shapes, batch, DION_FP32, p), or less for
 * waves as in dion_orth_batched. */
int dion_rowsubset_step(float* const* E, const void* const* grad, void* const* out,
                        const dion_shape* shapes, int32_t batch, int32_t grad_dtype, float beta,
                        const dion_ns_params* p, int32_t* sel_idx, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The same step followed by the weight update, fused: the flow of the Dion3
 * summary (输入输出流程: update the momentum, select rows, Gram Newton-Schulz,
 * update the weights), with the optimizer's last step in the final apply:
 *   E, grad, shapes, grad_dtype, beta, p, sel_idx  as dion_rowsubset_step
 *   W[i]          device R x C of w_dtype (bf16 or fp32), updated in place:
 *                 W <- fl32(fl32(W * (1 - weight_decay)) - fl32(alpha[i] * U)),
 *                 rounded to nearest even for bf16, where U is the step's
 *                 update: the orthogonalized selected rows (fp32, before any
 *                 rounding) and the new momentum E in the other rows
 *   alpha         host array of `batch` floats: the learning rate times the
 *                 matrix's shape scale (chosen by the caller)
 *   weight_decay  decoupled weight decay factor (0 = none)
 * No separate output is written.  Workspace: dion_workspace_size(shapes,
 * batch, DION_FP32, p), or less for waves as in dion_orth_batched. */
int dion_rowsubset_step_update(float* const* E, const void* const* grad, void* const* W,
                               const dion_shape* shapes, int32_t batch, int32_t grad_dtype, int32_t w_dtype,
                               float beta, const float* alpha, float weight_decay, const dion_ns_params* p,
                               int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Low-rank update: Dion and Orth-Dion (Orth-Dion explainer, technical
 * summary: Problem Statement, Methodology "The Geometric Insight" and
 * "Orth-Dion", Error Feedback Analysis).  One step per matrix, with
 * r = min(rank, R, C):
 *   B = fl32(M + G)            the residual buffer takes the gradient
 *   P = orth(B Q)              one power-iteration step from the previous Q
 *   W = B^T P
 *   M <- B - beta P W^T        error feedback (beta = 1 removes the captured part)
 *   Q <- orth(W)  (DION_LOWRANK_QR, Orth-Dion)  or  W / column norms
 *                              (DION_LOWRANK_COLNORM, Dion)
 *   out = P Q^T                unscaled (the caller applies lr and shape factors)
 * orth(F) is the reduced QR factor with a positive triangular diagonal,
 * computed as shifted CholeskyQR3 (Gram in fp32, Cholesky factor and its
 * inverse in fp64; the first of three passes factors the Gram matrix plus
 * 1e-3 times its largest diagonal entry), which keeps the factor
 * orthonormal to working precision for F of condition number up to about
 * 1e7, where plain CholeskyQR2 in fp32 needs about 4e3 at most.  The
 * factor itself is fixed by fp32-accurate data only to about
 * cond(F) * 2^-24 (relative error about 1e-6 for a well-conditioned F; a
 * first step from a square random Q can reach cond(B Q) = 1e5).  Inputs for
 * which B Q or W has rank below r are outside the method's contract (the
 * factor is not unique): the output is finite but unspecified.
 *   M[i]      device R x C fp32 buffer, updated in place
 *   grad[i]   device R x C of grad_dtype (bf16, fp32 or fp16), read only;
 *             must not overlap M[i]
 *   Q[i]      device C x r fp32 right factor: read as the previous one,
 *             overwritten with the new one; must not overlap M[i]
 *   out[i]    device R x C of out_dtype; must not overlap M[i]
 *   rank      1 .. 512 (DION_E_UNSUPPORTED above)
 * The rank-r products run in this library's GEMM kernel (one launch per
 * distinct (R, C, r) and product, with device pointer arrays from the
 * uploaded header), with fp32 accumulation: B Q on fp32 operands split into
 * three bf16 terms (six MFMA products, fp32 accuracy: its error is amplified
 * by the orthogonalization that follows), every other product on two fp16
 * terms under a power-of-two scale taken from the operand's largest |value|
 * (three MFMA products, 22 significant bits).  With a 16-bit gradient, B is
 * never stored: the products that read it add M and G as they load them
 * (the same single rounding), and M takes the new buffer in the last of
 * them.  The update is written in out_dtype by the last product (round to
 * nearest even).  All memory is the
 * caller's workspace; no handle or other state is kept.  Asynchronous on
 * `stream`. */
typedef enum { DION_LOWRANK_QR = 0, DION_LOWRANK_COLNORM = 1 } dion_lowrank_mode;

/* Bytes of workspace for dion_lowrank_step (0 on invalid arguments). */
size_t dion_lowrank_workspace_size(const dion_shape* shapes, int32_t batch, int32_t rank, int32_t out_dtype);

int dion_lowrank_step(float* const* M, const void* const* grad, float* const* Q, void* const* out,
                      const dion_shape* shapes, int32_t batch, int32_t grad_dtype, int32_t out_dtype,
                      int32_t rank, float beta, int32_t mode, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ------------------------------------------------------------------------
 * Phase entry points: one step of the path on its own, with the same kernels,
 * operand layout and precision as inside dion_orth_batched, for kernel-level
 * checks.  Conventions as above; each takes its own workspace of
 * dion_phase_workspace_size(phase, ...) bytes.  "Gram side" means the
 * orientation of the iteration: a wide matrix (R <= C) is X itself, a tall
 * one is processed as X^T, and m = min(R, C).
 * precision: DION_PREC_MFMA16 (fp16 MFMA, fp32 accumulation), DION_PREC_FP64,
 * or DION_PREC_AUTO (FP64 for DION_FP32 inputs, MFMA16 otherwise).
 * ------------------------------------------------------------------------ */
typedef enum {
  DION_PHASE_ROWKEYS_TOPK = 1,
  DION_PHASE_SYRK = 2,
  DION_PHASE_SYMPOLY = 3,
  DION_PHASE_APPLY = 4
} dion_phase;

/* Workspace bytes of one phase entry point (0 on invalid arguments).  For
 * DION_PHASE_SYMPOLY pass shapes {m_i, m_i} (dtype is ignored); row_frac is
 * used by DION_PHASE_ROWKEYS_TOPK only. */
size_t dion_phase_workspace_size(int32_t phase, const dion_shape* shapes, int32_t batch, int32_t dtype,
                                 int32_t precision, float row_frac);

/* Row keys and top-k selection (the row rule of the Dion3 abstract and of the
 * Dion3 summary, 核心模块, "Dion3 更新规则" bullet), as step 1 above:
 *   keys     optional device fp64 buffer of sum_i R_i entries: the squared L2
 *            norm of every row, matrices in batch order
 *   sel_idx  optional device int32 buffer of sum_i k_i entries: the selected
 *            rows of each matrix, ascending (larger key first, ties to the
 *            lower row index, k = dion_selected_rows(R, row_frac)) */
int dion_rowkeys_topk_batched(const void* const* M, const dion_shape* shapes, int32_t batch, int32_t dtype,
                              float row_frac, double* keys, int32_t* sel_idx, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Gram matrix on the Gram side (Dion3 summary, 核心模块, "Gram Newton-Schulz"
 * and CuteDSL bullets: the symmetric product computed on the upper triangle
 * and mirrored):
 *   X[i]  device R x C of dtype, read only
 *   G[i]  device m x m fp32, row-major: X X^T (wide) or X^T X (tall)
 * MFMA16 runs on one fp16 term of X / ||X||_F (exact for bf16 input, an fp16
 * rounding of fp32 input), fp32 accumulation, result kept in two fp16 terms
 * and scaled back by ||X||_F^2. */
int dion_syrk_batched(const void* const* X, float* const* G, const dion_shape* shapes, int32_t batch,
                      int32_t dtype, int32_t precision, void* workspace, size_t workspace_bytes, void* stream);

/* Gram polynomial of one iteration (the same bullet; the polynomial is fused
 * into the epilogue of G * G):
 *   G[i]    device m_i x m_i fp32, symmetric, spectral norm <= 1 (the Gram
 *           matrix of a Frobenius-normalized iterate); only G^T is read, so
 *           the result is exact for the transpose of a nonsymmetric input
 *   P[i]    device m_i x m_i fp32: a I + b G + c G^2
 *   coeffs  host (a, b, c); NULL = the fixed quintic
 * MFMA16 takes G in two fp16 terms; a spectral norm above 1 may overflow its
 * fixed fp16 scale (output unspecified). */
int dion_sympoly_batched(const float* const* G, float* const* P, const int32_t* m, int32_t batch,
                         const float* coeffs, int32_t precision, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Apply of an m x m factor on the Gram side (the final apply of the path):
 *   Q[i]  device m x m fp32 (m = min(R, C)), read only
 *   X[i]  device R x C of dtype, read only
 *   Y[i]  device R x C of dtype: Q X when R <= C, X Q when R > C (rounded to
 *         nearest even for bf16)
 * MFMA16 takes Q in two fp16 terms and X in one (bf16) or two (fp32). */
int dion_apply_batched(const float* const* Q, const void* const* X, void* const* Y, const dion_shape* shapes,
                       int32_t batch, int32_t dtype, int32_t precision, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Useful floating-point operations of one dion_orth_batched call on this
 * batch, in the executed formulation, symmetric products counted once:
 * per matrix and restart segment of length L,
 *   n*m*(m+1) [Gram] + 2*m*m*n [apply] + (4L-3)*m*m*(m+1) [m x m chain]. */
double dion_useful_flops(const dion_shape* shapes, int32_t batch, const dion_ns_params* p);

/* Rows selected from a matrix of `rows` rows: ceil(row_frac * rows) with the
 * 1e-6 relative shrink described above, clamped to [1, rows]; 0 if invalid. */
int32_t dion_selected_rows(int32_t rows, float row_frac);

/* Profiling for benchmarks.  While enabled, every phase that a call of the
 * calling thread enqueues is bracketed by two hipEvents recorded on the
 * call's own stream, so the durations are those of the kernels on that
 * stream.  dion_profile_enable clears the records and returns the previous
 * state.  Record i carries the phase name ("rowkeys", "momentum", "select",
 * "pack", "syrk", "gram_poly", "sym_product", "apply", "transpose", "final",
 * "copy_rows"), the kernel instance it launched (as profilers print it, e.g.
 * "dion::k_gemm16<256, 2, 2, 0, true>"), its elapsed milliseconds (waits for
 * its end event), its useful FLOPs (symmetric products counted once), the
 * MFMA FLOPs it executes (split terms and full diagonal tiles included) and
 * its algorithmic HBM bytes (streaming phases).  Strings stay valid until the
 * thread exits.  Any output pointer may be NULL. */
int dion_profile_enable(int enable);
int dion_profile_count(void);
int dion_profile_get(int index, const char** name, const char** kernel, float* ms,
                     double* useful_flops, double* mfma_flops, double* bytes);
/* Algorithmic FLOPs of record `index`: the per-unit formulas of its useful
 * count (Gram n m (m+1), m x m chain product m^2 (m+1), apply 2 m^2 n) over
 * every product the launch runs, including those outside the caller's
 * schedule (the accumulated restart factor S = Q_2 Q_1 of a restart from X0,
 * and the applies and Grams of the restarts the planner adds to cut long
 * runs), which the useful count leaves out.  Diagonal tiles, padding and
 * split terms are not counted.  Does not wait for the device.  NULL output
 * allowed; DION_E_INVAL for an index out of range. */
int dion_profile_get_algorithmic(int index, double* algorithmic_flops);

/* Static message for a status code. */
const char* dion_strerror(int status);
/* Message describing the last error on the calling thread ("" if none). */
const char* dion_last_error(void);
/* ABI version (major * 100 + minor). */
int dion_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DION_H */
