/*
 * bakron.h - C ABI of the MI355X (gfx950) BaKron solver.
 *
 * BaKron quantises a weight matrix W (m x n) with GPTQ run on vec(W) under a
 * two-sided Kronecker-factored Hessian A (x) B: A is n x n (input side), B is
 * m x m (output side), both symmetric positive definite. Source: "BaKron:
 * Efficient Quantization with Kronecker-Factored Hessians" (arXiv
 * 2608.06291), §3 (Algorithms 2-6, Theorem 3.2) and Appendix B (recurrence
 * (2), the order-free definition of the result).
 *
 * Conventions for every call:
 *  - All matrices are row-major with an explicit leading dimension (ld >= the
 *    number of columns). The column-major vec of §3.1 is an indexing
 *    convention of the math only; by the symmetry of the dependency order a
 *    column-major caller can pass (n, m, W^T, B, A) with column scales.
 *  - Every pointer except `bad_pivot` is a device pointer owned by the
 *    caller. The library allocates and frees no device memory and keeps no
 *    global state (but for bakron_solve_noalloc's scratch and the poll bound
 *    of bakron_debug_set_wait_polls); scratch memory is the caller's
 *    `workspace` of at least
 *    the size the matching *_workspace_bytes query returns (256-byte
 *    aligned). The synchronous factor calls are the one place that creates
 *    HIP objects: when m != n, or an order exceeds 8192, bakron_factor and
 *    bakron_factor_batched create helper streams and events for the call
 *    and destroy them before returning (every return path, errors included,
 *    first waits for all work the call enqueued). bakron_solve_timed
 *    creates and destroys its timing events the same way.
 *  - There is no out-of-memory status: no call allocates device memory, so
 *    none can run out of it. A workspace smaller than its query is
 *    BAKRON_EINVAL.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *    asynchronous unless stated otherwise; argument errors are reported
 *    before anything is enqueued. Calls on different streams with distinct
 *    workspaces may run concurrently.
 *  - `dtype` selects the element type of every floating-point array of the
 *    call: BAKRON_F32 (float) or BAKRON_F64 (double). Codes are int32.
 *  - m = 0 or n = 0 is accepted and does nothing.
 */
#ifndef BAKRON_H_
#define BAKRON_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BAKRON_OK 0
#define BAKRON_EINVAL (-1)  /* bad argument: null pointer, size, leading dimension,
                               mode, alphabet, or workspace too small */
#define BAKRON_ENOTSPD (-2) /* A or B is not numerically positive definite */
#define BAKRON_EHIP (-3)    /* a HIP runtime call or kernel launch failed */
#define BAKRON_EWAIT (-4)   /* a solve's bounded wait inside a leaf block gave up
                               (bakron_solve_status): its outputs are invalid */

/* Element types. */
#define BAKRON_F32 0
#define BAKRON_F64 1

/* Scale modes of the quantizer (§3.1: one scale per row and/or column). */
#define BAKRON_SCALE_NONE 0 /* s = 1 */
#define BAKRON_SCALE_ROW 1  /* s_i for row i, length m */
#define BAKRON_SCALE_COL 2  /* s_j for column j, length n */

/* Human-readable text for a status code (static storage). */
const char *bakron_status_string(int status);

/* ABI revision of this header; bumped on any incompatible change. */
int bakron_abi_version(void);

/* Tile edge (16) of the tiling of W the solver works on, for `dtype`.
 * Returns 0 for an invalid dtype. */
int bakron_tile_size(int dtype);

/* ------------------------------------------------------------------------
 * Factor: the first two steps of Algorithms 2, 3, 5 and 6 (§3.2-§3.5).
 *
 * L^A = Cholesky(A^-1) and L^B = Cholesky(B^-1) (§3.1: lower triangular,
 * L L^T = A^-1, positive diagonal), then every column divided by its
 * diagonal entry. Computed as L = RevCholesky(A)^-1 (if A = R^T R with R
 * lower, A^-1 = R^-1 R^-T, so R^-1 is the Cholesky factor of A^-1), in
 * float64 internally for both dtypes, and rounded once to `dtype`.
 *
 * A      n x n (lda >= n), B m x m (ldb >= m); only the lower triangles are
 *        read.
 * LA     out, n x n (ldla >= n): unit lower triangular, strict upper part
 *        written as 0. LB likewise, m x m (ldlb >= m).
 * dA, dB out (nullable), length n / m: the diagonals of Cholesky(A^-1) and
 *        Cholesky(B^-1) before normalisation.
 * bad_pivot  HOST pointer to int64[2] (nullable). On BAKRON_ENOTSPD it
 *        receives {side, index}: side 0 = A, 1 = B, and the first pivot of
 *        the reversed Cholesky that was not positive and finite, counted
 *        from the last row (index k refers to row n-1-k of A). Otherwise
 *        {-1, -1}.
 *
 * SYNCHRONOUS: waits for `stream` to read the pivot check. On
 * BAKRON_ENOTSPD the outputs are unspecified.
 * ------------------------------------------------------------------------ */
size_t bakron_factor_workspace_bytes(int dtype, int64_t m, int64_t n);
int bakron_factor(int dtype, int64_t m, int64_t n,
                  const void *A, int64_t lda, const void *B, int64_t ldb,
                  void *LA, int64_t ldla, void *LB, int64_t ldlb,
                  void *dA, void *dB,
                  void *workspace, size_t workspace_bytes,
                  int64_t *bad_pivot, void *stream);

/* ------------------------------------------------------------------------
 * Batched factor: bakron_factor on `batch` pairs (A, B) of the same orders
 * (n, m) in one sequence of launches (every linear module of a model has its
 * own pair, §3.6; factoring small pairs one at a time leaves the GPU idle).
 * Pair b uses A + b * stride_a, B + b * stride_b and writes LA + b * stride_la,
 * LB + b * stride_lb, dA + b * stride_da, dB + b * stride_db (element
 * strides). Input strides may be 0 (a shared matrix); for batch > 1 the
 * output strides must keep the outputs of different pairs apart
 * (stride_la >= (n - 1) * ldla + n, stride_da >= n, and likewise for B).
 * Each pair's result is bit-identical to bakron_factor on it.
 * bad_pivot  HOST int64[3] (nullable): on BAKRON_ENOTSPD, {pair, side,
 *        index} of the first failing pivot (pairs in order, A before B),
 *        as for bakron_factor; otherwise {-1, -1, -1}.
 * 0 <= batch <= 32767. SYNCHRONOUS, like bakron_factor.
 * ------------------------------------------------------------------------ */
size_t bakron_factor_batched_workspace_bytes(int dtype, int64_t batch, int64_t m, int64_t n);
int bakron_factor_batched(int dtype, int64_t batch, int64_t m, int64_t n,
                          const void *A, int64_t lda, int64_t stride_a,
                          const void *B, int64_t ldb, int64_t stride_b,
                          void *LA, int64_t ldla, int64_t stride_la,
                          void *LB, int64_t ldlb, int64_t stride_lb,
                          void *dA, int64_t stride_da, void *dB, int64_t stride_db,
                          void *workspace, size_t workspace_bytes,
                          int64_t *bad_pivot, void *stream);

/* ------------------------------------------------------------------------
 * Solve: BaKron (Algorithm 6, §3.5) on a tiling of W, which yields the codes
 * of BaKron-naive (Algorithm 2) by Theorem 3.2 / Appendix B.
 *
 * W      m x n (ldw >= n), never modified.
 * LA, LB the normalised factors (as bakron_factor writes them): only the
 *        strict lower triangles are read, the diagonal is taken as 1.
 * alpha_lo, alpha_hi, unbounded
 *        the alphabet {alpha_lo, ..., alpha_hi} (alpha_lo <= alpha_hi), or
 *        all integers when unbounded != 0 (§3.1).
 * scale_mode, scales
 *        BAKRON_SCALE_NONE (scales must be NULL), ROW (length m) or COL
 *        (length n). Scales must be finite and > 0; other values give
 *        unspecified codes.
 * V      out, m x n int32 codes (ldv >= n): clamp(rint(x / s), lo, hi) at the
 *        value x each entry has when it is rounded; ties go to even.
 *        Unbounded codes must fit int32 (|x / s| < 2^31).
 * Wt     out (nullable), m x n (ldwt >= n): the value x of each entry at the
 *        moment it was rounded (Appendix B: the workspace keeps it).
 *
 * Asynchronous. Deterministic: the same inputs give bit-identical outputs.
 * Non-finite inputs give unspecified codes.
 *
 * Inside a leaf block (a launch that solves G consecutive tile
 * anti-diagonals, one workgroup per tile row) each row waits for the rows
 * above it through the workspace. Every wait is for a running workgroup and
 * is bounded (about 0.1 s); one that gives up lets the launch finish with
 * invalid outputs and marks the workspace: bakron_solve_status reports it.
 * ------------------------------------------------------------------------ */
size_t bakron_solve_workspace_bytes(int dtype, int64_t m, int64_t n);
int bakron_solve(int dtype, int64_t m, int64_t n,
                 const void *W, int64_t ldw,
                 const void *LA, int64_t ldla, const void *LB, int64_t ldlb,
                 int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded,
                 int scale_mode, const void *scales,
                 int32_t *V, int64_t ldv,
                 void *Wt, int64_t ldwt,
                 void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * BaKron-antidiagonal: Algorithm 3 (§3.3) on the whole matrix, the solver
 * the paper compares BaKron with (§6 Table 3; equivalent to YAQA). For each
 * anti-diagonal i + j = k in turn, every entry on it is rounded at once and
 * the errors are applied to all later entries as one rank-d product
 * (Appendix C: O(m^2 n^2) total work, m + n - 1 sequential steps). Same
 * arguments, codes (Theorem 3.2: all four algorithms give the same V),
 * values at rounding and asynchrony as bakron_solve; its own workspace
 * (bakron_solve_antidiag_workspace_bytes). One kernel launch per
 * anti-diagonal.
 * ------------------------------------------------------------------------ */
size_t bakron_solve_antidiag_workspace_bytes(int dtype, int64_t m, int64_t n);
int bakron_solve_antidiag(int dtype, int64_t m, int64_t n,
                          const void *W, int64_t ldw,
                          const void *LA, int64_t ldla, const void *LB, int64_t ldlb,
                          int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded,
                          int scale_mode, const void *scales,
                          int32_t *V, int64_t ldv,
                          void *Wt, int64_t ldwt,
                          void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * No-allocation solve, for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, result and asynchrony as
 * bakron_solve minus the workspace: the scratch is a device array of
 * BAKRON_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held by
 * that GPU until the process ends (the first call on a device looks up its
 * address; no call allocates or frees anything). A problem whose
 * bakron_solve_workspace_bytes exceeds BAKRON_NOALLOC_SCRATCH_BYTES is
 * BAKRON_EINVAL (checked before any HIP call): 96 MiB holds up to 2496 x
 * 2496 in float32, or 1024 x 2048 in float64.
 * All calls on one GPU share its scratch, and it keeps the last call's
 * contents (no part needs to start at zero: the solve writes every word
 * before reading it): calls that may overlap on one GPU (different streams,
 * or host threads) race and must be serialised by the caller. The device
 * is the current one (hipGetDevice), and `stream` must belong to it.
 * ------------------------------------------------------------------------ */
#define BAKRON_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int bakron_solve_noalloc(int dtype, int64_t m, int64_t n,
                         const void *W, int64_t ldw,
                         const void *LA, int64_t ldla, const void *LB, int64_t ldlb,
                         int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded,
                         int scale_mode, const void *scales,
                         int32_t *V, int64_t ldv,
                         void *Wt, int64_t ldwt, void *stream);

/* The launch schedule bakron_solve uses for (dtype, m, n), for measurement:
 * writes up to `max_ops` records of 4 int32 {kind, a, b, c} to the HOST
 * array `ops` (nullable) and returns the total number of records, or a
 * negative status. kind 0 = leaf block: tile anti-diagonals [a, b), solved in
 * order with the updates between them (§3.5 Algorithm 6's leaf, one
 * launch); kinds 2 and 3 = the two band products of an internal node, tile
 * anti-diagonals [a, b) -> [b, c). Host only. */
int64_t bakron_solve_schedule(int dtype, int64_t m, int64_t n, int32_t *ops, int64_t max_ops);

/* Measurement variant of bakron_solve: same arguments and result, and it
 * also times every leaf and band-product launch. For every record i of
 * bakron_solve_schedule, op_ms[i] receives that kernel's execution time in
 * milliseconds, from HIP events stamped by its own dispatch on `stream`
 * (hipExtLaunchKernel start/stop events; 0 for a launch with no work);
 * on an error every slot receives -1. `op_ms` is a HOST
 * array of `n_ops` doubles and n_ops must equal the schedule length.
 * SYNCHRONOUS (waits for the last event), and also returns BAKRON_EWAIT as
 * bakron_solve_status would. Creates and destroys its events; returns
 * BAKRON_EHIP if that fails. */
int bakron_solve_timed(int dtype, int64_t m, int64_t n,
                       const void *W, int64_t ldw,
                       const void *LA, int64_t ldla, const void *LB, int64_t ldlb,
                       int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded,
                       int scale_mode, const void *scales,
                       int32_t *V, int64_t ldv,
                       void *Wt, int64_t ldwt,
                       void *workspace, size_t workspace_bytes, void *stream,
                       double *op_ms, int64_t n_ops);

/* Status of the last solve(s) run on `workspace`: waits for `stream`, then
 * returns BAKRON_EWAIT if a wait inside a leaf block of any of the `batch`
 * problems gave up (their outputs are invalid), else BAKRON_OK. The
 * arguments are those of the solve: (dtype, 1, m, n, workspace,
 * workspace_bytes) for bakron_solve, (dtype, batch, m, n, ...) for
 * bakron_solve_batched, (dtype, heads, m / heads, n, ...) for
 * bakron_solve_blockdiag; workspace = NULL reads the current device's
 * scratch of bakron_solve_noalloc (batch 1). SYNCHRONOUS. */
int bakron_solve_status(int dtype, int64_t batch, int64_t m, int64_t n, const void *workspace,
                        size_t workspace_bytes, void *stream);

/* Test hook: sets the poll bound of the leaf blocks' waits for solves
 * enqueued from now on, process-wide (polls < 0 restores the default,
 * 65536; 0 makes any wait that finds its data not yet written give up at
 * once); returns the previous bound. Host only. */
int32_t bakron_debug_set_wait_polls(int32_t polls);

/* ------------------------------------------------------------------------
 * Batched solve: bakron_solve on `batch` problems of the same shape (m x n)
 * in one sequence of launches, for many small matrices: every linear module
 * of a model is its own problem (§3.6 costs the solve per module), and a
 * small problem alone leaves most of the GPU idle (a 1024 x 2048 matrix has
 * at most 64 tiles per tile anti-diagonal). Problem b uses W + b * stride_w, LA + b * stride_la,
 * LB + b * stride_lb, scales + b * stride_s and writes V + b * stride_v,
 * Wt + b * stride_wt; strides are in elements. Input strides may be 0 (one
 * array shared by every problem, e.g. a common factor); for batch > 1 the
 * output strides must be at least (m - 1) * ld + n, so that the outputs of
 * different problems do not overlap. Each problem's result is bit-identical
 * to bakron_solve on the same inputs (same kernels, same order of
 * operations). 0 <= batch <= 65535. The workspace is batch times that of
 * bakron_solve (bakron_solve_batched_workspace_bytes). Other arguments,
 * errors and asynchrony as for bakron_solve.
 * ------------------------------------------------------------------------ */
size_t bakron_solve_batched_workspace_bytes(int dtype, int64_t batch, int64_t m, int64_t n);
int bakron_solve_batched(int dtype, int64_t batch, int64_t m, int64_t n,
                         const void *W, int64_t ldw, int64_t stride_w,
                         const void *LA, int64_t ldla, int64_t stride_la,
                         const void *LB, int64_t ldlb, int64_t stride_lb,
                         int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded,
                         int scale_mode, const void *scales, int64_t stride_s,
                         int32_t *V, int64_t ldv, int64_t stride_v,
                         void *Wt, int64_t ldwt, int64_t stride_wt,
                         void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Loss: tr(B (W - Q) A (W - Q)^T) with Q = s (.) V, the quadratic form of
 * vec(W - Q) under A (x) B (Proposition 3.1, §3.1). Evaluated in float64 as
 * sum_ij (B D)_ij (D A)_ij with D = W - Q (A symmetric).
 *
 * W (ldw), V (ldv) m x n; A n x n, B m x m, lower triangles read;
 * scale_mode/scales as for bakron_solve.
 * loss   out: DEVICE pointer to one double.
 *
 * Asynchronous.
 * ------------------------------------------------------------------------ */
size_t bakron_loss_workspace_bytes(int dtype, int64_t m, int64_t n);
int bakron_loss(int dtype, int64_t m, int64_t n,
                const void *W, int64_t ldw, const int32_t *V, int64_t ldv,
                int scale_mode, const void *scales,
                const void *A, int64_t lda, const void *B, int64_t ldb,
                double *loss, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Batched loss: bakron_loss on `batch` problems of one shape in the same
 * launches (the companion of bakron_factor_batched / bakron_solve_batched).
 * Problem b uses W + b * stride_w, V + b * stride_v, scales + b * stride_s,
 * A + b * stride_a, B + b * stride_b (element strides; 0 shares an array)
 * and writes loss[b] (DEVICE array of batch doubles). Same definition and
 * float64 arithmetic as bakron_loss; the products are reduced per 64 x 64
 * block instead of per stream-K range, so results agree with bakron_loss to
 * float64 rounding, not bit for bit. 0 <= batch <= 65535. Asynchronous.
 * ------------------------------------------------------------------------ */
size_t bakron_loss_batched_workspace_bytes(int dtype, int64_t batch, int64_t m, int64_t n);
int bakron_loss_batched(int dtype, int64_t batch, int64_t m, int64_t n,
                        const void *W, int64_t ldw, int64_t stride_w,
                        const int32_t *V, int64_t ldv, int64_t stride_v,
                        int scale_mode, const void *scales, int64_t stride_s,
                        const void *A, int64_t lda, int64_t stride_a,
                        const void *B, int64_t ldb, int64_t stride_b,
                        double *loss, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Block-diagonal output factor (Appendix D, experimental setup: the
 * attention-local Hessians of the query, key and value projections, whose
 * per-head output-side Grams are assembled into one block-diagonal matrix
 * over the whole projection; Table 4). B = blockdiag(B_0, ..., B_{h-1}),
 * `heads` = h blocks of order b = m / h (m % h == 0). B^-1 and its Cholesky
 * factor are then block-diagonal, an error reaches only rows of its own
 * block, and the problem splits exactly into h problems of b x n sharing
 * L^A: the calls below run all heads in the same launches (the batched
 * machinery), never touching the zero blocks. Results equal the dense calls
 * on the assembled block-diagonal B (codes, in exact arithmetic; float64
 * codes bit for bit in the tests).
 *
 * Block h of B is at B + h * stride_b (b x b, ldb >= b; lower triangle
 * read); block h of L^B at LB + h * stride_lb (stride_lb >= (b-1) ldlb + b);
 * dB (nullable) is length m, block h at dB + h * b.
 *
 * bakron_factor_blockdiag: L^A (n x n) and dA as bakron_factor, and the h
 * blocks of L^B, each the normalised Cholesky(B_h^-1). bad_pivot (HOST
 * int64[3], nullable): on BAKRON_ENOTSPD {side, block, index} (side 0 = A
 * with block -1, side 1 = B), index as for bakron_factor; else {-1,-1,-1}.
 * SYNCHRONOUS.
 * bakron_solve_blockdiag: the solve of bakron_solve with L^B given by its
 * blocks; W, V, Wt, scales as for bakron_solve (row scales length m, column
 * scales length n). Asynchronous.
 * bakron_loss_blockdiag: tr(B (W - Q) A (W - Q)^T) = sum_h tr(B_h D_h A
 * D_h^T) in float64 (the per-head sums added in head order); *loss is a
 * DEVICE double. Asynchronous.
 * 1 <= heads <= 32767.
 * ------------------------------------------------------------------------ */
size_t bakron_factor_blockdiag_workspace_bytes(int dtype, int64_t heads, int64_t m, int64_t n);
int bakron_factor_blockdiag(int dtype, int64_t heads, int64_t m, int64_t n,
                            const void *A, int64_t lda,
                            const void *B, int64_t ldb, int64_t stride_b,
                            void *LA, int64_t ldla,
                            void *LB, int64_t ldlb, int64_t stride_lb,
                            void *dA, void *dB,
                            void *workspace, size_t workspace_bytes,
                            int64_t *bad_pivot, void *stream);
size_t bakron_solve_blockdiag_workspace_bytes(int dtype, int64_t heads, int64_t m, int64_t n);
int bakron_solve_blockdiag(int dtype, int64_t heads, int64_t m, int64_t n,
                           const void *W, int64_t ldw,
                           const void *LA, int64_t ldla,
                           const void *LB, int64_t ldlb, int64_t stride_lb,
                           int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded,
                           int scale_mode, const void *scales,
                           int32_t *V, int64_t ldv,
                           void *Wt, int64_t ldwt,
                           void *workspace, size_t workspace_bytes, void *stream);
size_t bakron_loss_blockdiag_workspace_bytes(int dtype, int64_t heads, int64_t m, int64_t n);
int bakron_loss_blockdiag(int dtype, int64_t heads, int64_t m, int64_t n,
                          const void *W, int64_t ldw, const int32_t *V, int64_t ldv,
                          int scale_mode, const void *scales,
                          const void *A, int64_t lda,
                          const void *B, int64_t ldb, int64_t stride_b,
                          double *loss, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Per-row scales: s_i = max_j |W_ij| / hi (1 for an all-zero row), the
 * per-output-feature absmax rule of Appendix D with hi the largest code
 * (7 for {-8..7}, 3 for {-4..3}). Computed in `dtype`.
 *
 * W m x n (ldw); scales out, length m; hi > 0. Asynchronous.
 * ------------------------------------------------------------------------ */
int bakron_row_scales(int dtype, int64_t m, int64_t n, const void *W, int64_t ldw,
                      int32_t hi, void *scales, void *stream);

/* ------------------------------------------------------------------------
 * Per-row scale search: the absmax scale of bakron_row_scales, optionally
 * shrunk by an MSE search (Appendix D, experimental setup: shrink by up to a
 * factor of 2, i.e. max_shrink = 0.5). The pages leave the search open;
 * this call evaluates grid + 1 candidates
 *   s_k = (dtype)(s_max * f_k),  f_k = 1 - (max_shrink * k) / grid  (float64),
 * k = 0..grid, s_max = max_j |W_ij| / alpha_hi, and returns for each row the
 * candidate with the smallest round-to-nearest error
 *   sum_j (W_ij - s_k c_j)^2,  c_j = clamp(rint(W_ij / s_k), lo, hi)
 * (division in dtype; terms and sum in float64); ties go to the smaller k.
 * An all-zero row gets scale 1. grid = 0 or max_shrink = 0 give exactly
 * bakron_row_scales.
 *
 * W m x n (ldw); scales out, length m. alpha_lo <= alpha_hi, alpha_hi > 0;
 * 0 <= grid <= 1024; 0 <= max_shrink < 1. BAKRON_EINVAL otherwise.
 * Asynchronous. Deterministic.
 * ------------------------------------------------------------------------ */
int bakron_row_scales_mse(int dtype, int64_t m, int64_t n, const void *W, int64_t ldw,
                          int32_t alpha_lo, int32_t alpha_hi, int32_t grid, double max_shrink,
                          void *scales, void *stream);

/* ------------------------------------------------------------------------
 * Kronecker factors from samples (§4.2 and Appendix A.2): for a Hessian
 * H = E[a a^T (x) b b^T] over N samples (a in R^n on the input side, b in
 * R^m on the output side),
 *   K-FAC style   (independence):        A = E[a a^T],          B = E[b b^T];
 *   Shampoo style (one power-iteration step from A = I, B = I):
 *                                        A = E[|b|^2 a a^T],    B = E[|a|^2 b b^T].
 * bakron_gram computes one such factor,
 *   G = (1/N) sum_k w_k x_k x_k^T  +  damp_rel * mean(diag) * I,
 * the damping applied after the mean of the undamped diagonal (the
 * experiments regularise each Gram by a multiple of its mean diagonal).
 * X      N x d (ldx >= d), row k = sample x_k (a for A, b for B).
 * weights  length N (nullable = all 1): 1 for K-FAC, the other side's
 *        bakron_sample_sqnorms for Shampoo.
 * G      out, d x d (ldg >= d), both triangles written (exactly symmetric);
 *        must not overlap X (BAKRON_EINVAL if the two ranges intersect).
 * Accumulates in `dtype` on MFMA (float32 or float64 sums over the samples).
 * N = 0 gives G = 0. damp_rel >= 0. Asynchronous.
 *
 * bakron_sample_sqnorms: out[k] = sum_j X[k][j]^2 (float64 sum, rounded
 * once to `dtype`), length N. Asynchronous.
 * ------------------------------------------------------------------------ */
int bakron_gram(int dtype, int64_t N, int64_t d, const void *X, int64_t ldx,
                const void *weights, double damp_rel, void *G, int64_t ldg, void *stream);
int bakron_sample_sqnorms(int dtype, int64_t N, int64_t d, const void *X, int64_t ldx,
                          void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BAKRON_H_ */
