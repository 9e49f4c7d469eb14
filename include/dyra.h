/*
 * dyra.h -- C-ABI of libdyra.so: the DyRA layer forward on AMD MI355X (gfx950).
 *
 * DyRA (arXiv 2610.02882, "DyRA: Dynamic Residual Approximation for Efficient
 * Matrix Multiplication in DNNs") splits a dense weight W (c1 x c2) into a
 * structured approximation W_hat (low-rank, Monarch or BLAST) and a dense
 * residual, W = W_hat + W_res, and corrects the residual product X W_res of
 * each input with one alternating-least-squares step at inference time:
 *
 *   L = X P                     P = W_res R0^T, R0 = top-r right singular
 *                               vectors of W_res (prepared offline)
 *   R = (L^T L + lambda I)^-1 (L^T X) W_res
 *   Y = X W_hat + L R + bias    (the n x c2 product X W_res is never formed)
 *
 * Sources (page title + section):
 *   nanless.github.io DyRA digest post: the split equations W = W_hat + W_res
 *   and XW = X W_hat + X W_res; the residual-product objective
 *   min ||X W_res - L R||_F^2 and the cheap ALS ordering; the one-iteration
 *   form XW ~ X W_hat + L1 R1 with L1 = X times a precomputable thin matrix;
 *   the offline/online split; the structured-matrix definitions.
 *   paperlayer.ai summary: 2.2 (ALS, ridge), 2.4 (fused merge, Cholesky for
 *   small r, Newton-Schulz for large r), App. A (offline + online stages),
 *   App. B (structured matrices).
 *
 * Conventions (every entry point):
 *   - Returns int: DYRA_OK (0) or a negative DYRA_E* code.  No C++ exception
 *     crosses the ABI.  dyra_status_string() names a code.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call touches no device state.
 *   - The caller owns every buffer (host and device).  The library allocates
 *     no device memory.  Its only process-wide state, created on first use and
 *     kept until the process ends: the compute-unit count of each device
 *     (queried once, to size the persistent kernels' grids); per device, one
 *     side stream with two events, on which a bf16 Newton-Schulz solve runs
 *     beside the token reduction (the caller's stream waits for it before
 *     the forward goes on; not created while the caller's stream is being
 *     captured, nor by dyra_forward_noalloc); and, for dyra_forward_noalloc
 *     only, that entry point's static device workspace.  Calls on distinct
 *     streams with distinct workspaces are independent.
 *   - Matrices are row-major and contiguous.  Device pointers must be 16-byte
 *     aligned.  "stream" is a hipStream_t passed as void* (NULL = default);
 *     it must belong to the current device (grid sizes and the side stream
 *     are taken from that device).
 *   - dtype: DYRA_F32 (fp32 storage, fp32 arithmetic) or DYRA_BF16 (bf16
 *     storage, fp32 accumulation); the r x r solves run in fp64 (Cholesky),
 *     fp32 with an fp64 pass where a pivot needs it (sweep), or at fp32
 *     accuracy (Newton-Schulz) for both.
 *   - Size constraints: c1, c2, k, r multiples of 8; 1 <= r <= min(c1, c2);
 *     r <= 128.  Low-rank: k + r <= min(c1, c2).  Monarch: c1 == c2 ==
 *     mblk^2 with mblk == 32 (bf16 only).  BLAST: nb divides c1 and c2,
 *     rb <= min(c1, c2) / nb, rb multiple of 8, c2 / nb multiple of 128
 *     (bf16 only); BLAST_DIAG also nb rb <= 32768.
 */
#ifndef DYRA_H
#define DYRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DYRA_OK          0
#define DYRA_EINVAL     -1   /* null pointer, negative ridge, unknown enum   */
#define DYRA_ESHAPE     -2   /* sizes violate the constraints above         */
#define DYRA_EWORKSPACE -3   /* workspace smaller than dyra_workspace_size  */
#define DYRA_EHIP       -4   /* a HIP launch or copy reported an error      */
#define DYRA_ENOCONV    -5   /* host eigensolver did not converge           */
#define DYRA_EDTYPE     -6   /* dtype not supported for this structure      */

/* static structure */
#define DYRA_LOWRANK 0
#define DYRA_MONARCH 1
#define DYRA_BLAST   2
#define DYRA_BLAST_DIAG 3   /* BLAST with diagonal couplings S_ij = diag(s_ij) */

/* storage / arithmetic type */
#define DYRA_F32  0
#define DYRA_BF16 1

/* r x r solver choice for dyra_forward */
#define DYRA_SOLVER_AUTO 0   /* the sweep (the faster solver on MI355X at every r <= 128) */
#define DYRA_SOLVER_CHOL 1   /* Cholesky: G + lambda I = C C^T, W = C^-1, Ginv = W^T W (fp64) */
#define DYRA_SOLVER_NS   2   /* Newton-Schulz, falling back to the sweep where it stalls   */

/* per-segment solver status words (dyra_solver_status) */
#define DYRA_SOLVE_OK        0
#define DYRA_SOLVE_NOT_SPD   1   /* a pivot <= 0, a non-finite G_b (a NaN or Inf in X_b), or */
                                 /* at ridge_eps = 0 a pivot <= 2^-16 of its diagonal:       */
                                 /* R_b := 0, Y_b = X_b W_hat + bias (a row of X_b that is   */
                                 /* not finite still gives a non-finite row of Y_b)           */
#define DYRA_SOLVE_NOCONV    2   /* reserved: an iterative solve without a usable result */
#define DYRA_SOLVE_ZERO      3   /* trace(G_b) == 0 (X_b P == 0): R_b := 0               */
#define DYRA_SOLVE_FALLBACK  4   /* Newton-Schulz did not reach its tolerance;            */
                                 /* R_b solved by the sweep instead (result valid)        */

typedef struct {
  int32_t kind;   /* DYRA_LOWRANK / DYRA_MONARCH / DYRA_BLAST / DYRA_BLAST_DIAG */
  int32_t k;      /* low-rank: static rank                                     */
  int32_t mblk;   /* Monarch: block count == block size m, c1 == c2 == m*m     */
  int32_t nb;     /* BLAST: nb x nb block grid                                 */
  int32_t rb;     /* BLAST: rank of the shared row / column bases              */
  int32_t r;      /* residual (dynamic) rank                                   */
  int64_t c1;     /* input features                                            */
  int64_t c2;     /* output features                                           */
} dyra_spec;

/* Element counts of each host factor array (0 = unused by this structure). */
typedef struct {
  int64_t U, V;        /* low-rank                                      */
  int64_t B1, B2;      /* Monarch                                       */
  int64_t Ub, S, Vb;   /* BLAST                                         */
  int64_t P, R0, Wres, res_sv;
} dyra_sizes;

/*
 * Host float64 factors written by dyra_prepare (caller-allocated, sizes from
 * dyra_prepare_sizes; pointers of unused arrays may be NULL):
 *   U  [c1][k], V [k][c2]                      W_hat = U V, sqrt(sigma) on each side
 *   B1 [m][m][m] (block a, row i, col j), B2 [m][m][m] (block j, row a, col l):
 *        W_hat[a*m+i][j*m+l] = B1[a][i][j] * B2[j][a][l]
 *        (= blockdiag(B1) . Pi . blockdiag(B2), Pi the reshape-transpose)
 *   Ub [nb][c1/nb][rb], S [nb][nb][rb][rb], Vb [nb][c2/nb][rb]:
 *        block (i, j) of W_hat = Ub[i] S[i][j] Vb[j]^T
 *        (DYRA_BLAST_DIAG: S [nb][nb][rb], the diagonals:
 *        block (i, j) = Ub[i] diag(S[i][j]) Vb[j]^T)
 *   P [c1][r] = W_res R0^T,  R0 [r][c2] (orthonormal rows),  Wres [c1][c2],
 *   res_sv [r] = top singular values of W_res (descending).
 */
typedef struct {
  double* U;  double* V;
  double* B1; double* B2;
  double* Ub; double* S; double* Vb;
  double* P;  double* R0; double* Wres; double* res_sv;
} dyra_host_factors;

/* Element counts of the factor arrays for a spec.  Errors: EINVAL, ESHAPE. */
int dyra_prepare_sizes(const dyra_spec* spec, dyra_sizes* out);

/*
 * Offline preparation on the host (float64, not part of the timed forward).
 * Fits W_hat by structure (low-rank: truncated SVD; Monarch: rank-1 SVD of
 * each m x m block; BLAST: shared bases from block-row / block-column SVDs
 * and least-squares couplings, for BLAST_DIAG the least-squares diagonal
 * couplings for those bases, diag(Ub[i]^T W_ij Vb[j])), forms
 * W_res = W - W_hat, takes R0 = top-r right singular vectors of W_res and
 * P = W_res R0^T.
 *   W: host [c1][c2] float64 (read only).  out: caller-allocated arrays.
 *   nthreads: host worker threads (<= 0: hardware concurrency).
 * Errors: EINVAL, ESHAPE, ENOCONV.
 * Source: nanless.github.io DyRA digest, "overall DyRA flow" and "offline
 * preparation and online computation" sections; paperlayer.ai App. A, App. B.
 */
int dyra_prepare(const dyra_spec* spec, const double* W, dyra_host_factors* out,
                 int32_t nthreads);

/*
 * Offline preparation with an input-aware static start (low-rank only): the
 * static factors minimise the output error on calibration rows instead of
 * the weight error.  A transform S (c1 x c1) is built from the rows, and
 * W_hat = S^-1 SVD_k(S W), split as U = S^-1 U_k sqrt(sigma),
 * V = sqrt(sigma) V_k^T; the residual, R0 and P follow from W_hat as in
 * dyra_prepare, and the device forward is unchanged.
 *   X_cal: host [n_cal][c1] float64 calibration rows (read only, finite).
 *   mode:  DYRA_INPUT_AWARE_DIAG: S = diag(channel RMS over the rows), each
 *          raised to at least 1e-6 of the largest;
 *          DYRA_INPUT_AWARE_CHOL: S = C^T with C C^T = X_cal^T X_cal / n_cal
 *          + delta I, delta = 1e-6 trace(X_cal^T X_cal / n_cal) / c1, so that
 *          ||S (W - W_hat)||_F = ||X_cal (W - W_hat)||_F / sqrt(n_cal) up to
 *          delta: W_hat is the best rank-k fit in that norm.
 *   out:   as for dyra_prepare (U, V, P, R0, Wres, res_sv).
 * Errors: EINVAL (null pointer, structure not low-rank, unknown mode,
 * non-finite or all-zero X_cal), ESHAPE (n_cal <= 0 or spec sizes),
 * ENOCONV.
 * Source: paperlayer.ai App. B (input-aware decomposition with activation-
 * based diagonal scaling or a Cholesky factor of the input covariance) and
 * nanless.github.io DyRA digest, "how the existing structured-matrix
 * methods differ" (transform from calibration activations, truncated SVD
 * of the transformed weight) and its input-aware x DyRA paragraph.
 */
#define DYRA_INPUT_AWARE_DIAG 1
#define DYRA_INPUT_AWARE_CHOL 2
int dyra_prepare_input_aware(const dyra_spec* spec, const double* W, const double* X_cal, int64_t n_cal,
                             int32_t mode, dyra_host_factors* out, int32_t nthreads);

/* Bytes of the packed device plan for (spec, dtype).  Errors: EINVAL, ESHAPE, EDTYPE. */
int dyra_plan_size(const dyra_spec* spec, int32_t dtype, size_t* bytes);

/*
 * Packs host float64 factors into the device plan layout (a host buffer of
 * dyra_plan_size bytes that the caller copies to device memory once).
 * Values are rounded fp64 -> fp32 (RNE), then to bf16 (RNE) for DYRA_BF16.
 * The layout is internal to the library (weights stored output-major so
 * every GEMM operand is contiguous along its reduction axis).
 * Errors: EINVAL, ESHAPE, EDTYPE.
 */
int dyra_plan_pack(const dyra_spec* spec, const dyra_host_factors* f, int32_t dtype,
                   void* host_plan);

/* Bytes of device workspace dyra_forward needs for B segments of s rows. */
int dyra_workspace_size(const dyra_spec* spec, int64_t B, int64_t s, int32_t dtype,
                        size_t* bytes);

/*
 * Byte offsets of the forward's intermediates inside the workspace, for
 * inspection and per-stage testing (the layout is otherwise internal):
 *   A      [n][wa]      stage-1 output: low-rank [T | L] (wa = k + r)
 *   Lt     [r][lt_pitch] L transposed (token-contiguous), dtype
 *   G      [B][r][r]    fp32  L_b^T L_b
 *   M      [B][r][c1]   fp32  L_b^T X_b
 *   Ginv   [B][r][r]    fp64  (G_b + lambda_b I)^-1
 *   Mp     [B][r][c1]   dtype Ginv_b M_b
 *   Rt     [c2][B r]    dtype R_b^T, R_b = Mp_b W_res
 *   status [B]          int32 solver status words
 *   prec   [B]          int32 1 where Mp_b was formed in fp64 (the sweep or
 *                       Cholesky solve met a relative pivot below 2^-5),
 *                       0 where in fp32 (Newton-Schulz inverses included)
 * Errors: EINVAL, ESHAPE, EDTYPE.
 */
typedef struct {
  int64_t A, Wp, Lt, G, M, Ginv, Mp, Rt, status, total, wa, lt_pitch, prec;
} dyra_ws_offsets;

int dyra_workspace_offsets(const dyra_spec* spec, int64_t B, int64_t s, int32_t dtype,
                           dyra_ws_offsets* out);

/*
 * The DyRA layer forward (asynchronous on `stream`; no host synchronisation).
 *   plan:      device, packed by dyra_plan_pack for the same spec and dtype.
 *   X:         device [B*s][c1], dtype.   Segment b = rows [b*s, (b+1)*s):
 *              each segment gets its own ALS solve (L_b, G_b, M_b, R_b).
 *   bias:      device [c2], dtype, or NULL.
 *   Y:         device [B*s][c2], dtype (written; must not alias X).
 *   ridge_eps: lambda_b = ridge_eps * trace(G_b) / r (>= 0; 1e-6 typical).
 *              0 means no ridge: a G_b whose pivot falls to 2^-16 of its
 *              diagonal (rank-deficient L_b, e.g. s < r) counts as singular
 *              and segment b gets status NOT_SPD and R_b = 0.
 *   solver:    DYRA_SOLVER_*.
 *   workspace: device, >= dyra_workspace_size bytes; holds the per-segment
 *              solver status words read by dyra_solver_status.
 * Errors (before any HIP call): EINVAL, ESHAPE, EDTYPE, EWORKSPACE; EHIP if
 * a launch fails.  Per-segment numerical trouble is not an error: see the
 * DYRA_SOLVE_* status words.
 * Source: nanless.github.io DyRA digest, equations XW = X W_hat + X W_res,
 * min_{L,R} ||X W_res - L R||_F^2 and XW ~ X W_hat + L1 R1; paperlayer.ai
 * 2.2 and 2.4.
 */
int dyra_forward(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                 void* Y, int64_t B, int64_t s, int32_t dtype, float ridge_eps,
                 int32_t solver, void* workspace, size_t ws_bytes, void* stream);

/*
 * More ALS iterations than the default one.  half_steps = 2 t: 2 is exactly
 * dyra_forward (t = 1: L from the precomputed thin matrix, then R); 3 is
 * t = 1.5 (then L again, L_b = X_b (W_res R_b^T)(R_b R_b^T + lambda I)^-1,
 * lambda = ridge_eps * trace(R_b R_b^T) / r, solved by the sweep); 4 is
 * t = 2 (then R again from the new L).  Y uses the last L and R.  Every
 * structure (the left step does not involve the static branch) in every
 * storage type it takes, uniform segments (ragged ones:
 * dyra_forward_varlen_als): EINVAL for half_steps outside 2..4.
 * The workspace must hold
 * dyra_workspace_size_als bytes for the same half_steps; otherwise the
 * arguments, ownership and errors are those of dyra_forward.
 * Source: nanless.github.io DyRA digest, "what the low-rank objective of the
 * residual product is" (alternating least squares, the fix-R solve for L
 * and the fix-L solve for R); paperlayer.ai 2.2 and E.3 (more iterations
 * lower the error).
 */
int dyra_workspace_size_als(const dyra_spec* spec, int64_t B, int64_t s, int32_t dtype, int32_t half_steps,
                            size_t* bytes);
int dyra_forward_als(const dyra_spec* spec, const void* plan, const void* X, const void* bias, void* Y,
                     int64_t B, int64_t s, int32_t dtype, float ridge_eps, int32_t solver, int32_t half_steps,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * dyra_forward with stage-boundary events, a profiling aid.  events[i] are
 * caller-created hipEvent_t handles (passed as void*; NULL entries skipped;
 * nevents <= 6 used): events[0] is recorded on `stream` before the first
 * kernel, events[i] after stage i -- 1: the stage-1 pass over X ([T | L] or
 * the structured first stage and L), 2: the token reductions M_b, G_b,
 * 3: the r x r solve and M'_b, 4: the right-factor GEMM R (and the BLAST
 * coupling GEMM), 5: the fused output GEMM.  Same arguments, results and
 * errors as dyra_forward (EINVAL also for nevents < 0 or events == NULL with
 * nevents > 0).
 */
int dyra_forward_events(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                        void* Y, int64_t B, int64_t s, int32_t dtype, float ridge_eps,
                        int32_t solver, void* workspace, size_t ws_bytes, void* stream,
                        void* const* events, int32_t nevents);

/*
 * dyra_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * static device array inside the library of DYRA_NOALLOC_MAX_WORKSPACE
 * bytes (64 MiB: enough for B = 32 segments of 1029 tokens at 1024 -> 4096,
 * k = 256, r = 64); a call whose dyra_workspace_size exceeds it returns
 * DYRA_EWORKSPACE before any HIP call.  Each GPU holds its own copy from the
 * first call made with that device current until the process ends; the
 * library takes the copy's address then (hipGetSymbolAddress) and calls no
 * allocating routine.  `stream` must belong to the current device.
 *   status_out: device int32[B] receiving the per-segment solver status
 *               words (DYRA_SOLVE_*), or NULL.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams or threads) race and give undefined results;
 * serialise them.  Every byte a call reads from the array is written earlier
 * in the same call, so nothing needs clearing between calls.  Other
 * arguments, results and errors as for dyra_forward.
 */
#define DYRA_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
int dyra_forward_noalloc(const dyra_spec* spec, const void* plan, const void* X, const void* bias, void* Y,
                         int64_t B, int64_t s, int32_t dtype, float ridge_eps, int32_t solver,
                         int32_t* status_out, void* stream);

/*
 * Ragged segments: dyra_forward over B segments of different lengths, one
 * per input of a batch that was concatenated token-wise (each input gets its
 * own low-rank correction, as for uniform segments).
 *   offsets:     host int64[B + 1], offsets[0] = 0, strictly increasing
 *                (every segment at least one row), offsets[B] = n < 2^31;
 *                segment b = rows [offsets[b], offsets[b + 1]).
 *   offsets_dev: device int32[B + 1] holding the same values (4-byte
 *                aligned; read by the kernels, never written).
 *   X: device [n][c1]; Y: device [n][c2]; status_out: device int32[B] that
 *   receives the per-segment DYRA_SOLVE_* words, or NULL.
 *   workspace: device, >= dyra_workspace_size_varlen bytes.
 * Other arguments as for dyra_forward.  Errors (before any HIP call):
 * EINVAL (NULL offsets or offsets_dev, misaligned pointers), ESHAPE
 * (offsets[0] != 0, an empty segment, n >= 2^31), EDTYPE, EWORKSPACE; EHIP
 * if a launch fails.  The host and device offsets must agree: the library
 * does not compare them.
 * Source: nanless.github.io DyRA digest (the per-input correction L1 R1);
 * paperlayer.ai 2.2.
 */
int dyra_workspace_size_varlen(const dyra_spec* spec, int64_t B, const int64_t* offsets,
                               int32_t dtype, size_t* bytes);
int dyra_forward_varlen(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                        void* Y, int64_t B, const int64_t* offsets, const int32_t* offsets_dev,
                        int32_t dtype, float ridge_eps, int32_t solver, int32_t* status_out,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * Ragged segments with more ALS iterations: dyra_forward_varlen with
 * half_steps = 2 t as for dyra_forward_als (2: t = 1, exactly
 * dyra_forward_varlen; 3: t = 1.5; 4: t = 2), each segment's left and right
 * steps on its own rows.  The workspace must hold
 * dyra_workspace_size_varlen_als bytes for the same offsets and half_steps.
 * Errors as for dyra_forward_varlen, and EINVAL for half_steps outside 2..4.
 * Source: nanless.github.io DyRA digest, "what the low-rank objective of the
 * residual product is" (the alternating solves); paperlayer.ai 2.2, E.3.
 */
int dyra_workspace_size_varlen_als(const dyra_spec* spec, int64_t B, const int64_t* offsets,
                                   int32_t dtype, int32_t half_steps, size_t* bytes);
int dyra_forward_varlen_als(const dyra_spec* spec, const void* plan, const void* X, const void* bias,
                            void* Y, int64_t B, const int64_t* offsets, const int32_t* offsets_dev,
                            int32_t dtype, float ridge_eps, int32_t solver, int32_t half_steps,
                            int32_t* status_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Copies the B per-segment solver status words of the last dyra_forward on
 * this workspace to host_out[B] (synchronises `stream`).  Errors: EINVAL, EHIP.
 */
int dyra_solver_status(const dyra_spec* spec, const void* workspace, int64_t B, int64_t s,
                       int32_t dtype, int32_t* host_out, void* stream);

/*
 * Dense comparator Y = X W + bias on the same GEMM core (asynchronous).
 *   X: device [n][c1]; Wt: device [c2][c1] (W transposed, i.e. the weight in
 *   output-major order as a linear layer stores it); bias: device [c2] or
 *   NULL; Y: device [n][c2].  Errors: EINVAL, ESHAPE, EDTYPE, EHIP.
 */
int dyra_dense_ref(const void* X, const void* Wt, const void* bias, void* Y, int64_t n,
                   int64_t c1, int64_t c2, int32_t dtype, void* stream);

/* Static string naming a status code. */
const char* dyra_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* DYRA_H */
