/*
 * flashsk.h -- C ABI of the streaming log-domain Sinkhorn library for AMD
 * Instinct MI355X (gfx950).
 *
 * Problem (entropic optimal transport between weighted point clouds under the
 * squared Euclidean cost; "FlashSinkhorn: IO-Aware Entropic Optimal Transport
 * on GPU", abstract, and its replication review, Summary):
 *
 *   x_i (i < n), y_j (j < m) in R^d, weights a_i >= 0, b_j >= 0, eps > 0
 *   C_ij = |x_i - y_j|^2 = |x_i|^2 + |y_j|^2 - 2 x_i.y_j
 *   P_ij = a_i b_j exp((f_i + g_j - C_ij) / eps)                 (transport plan)
 *   F(g)_i = -eps LSE_j( log b_j + (g_j - |y_j|^2 + 2 x_i.y_j)/eps ) + |x_i|^2
 *   G(f)_j = -eps LSE_i( log a_i + (f_i - |x_i|^2 + 2 x_i.y_j)/eps ) + |y_j|^2
 *
 * F and G are the stabilized log-domain Sinkhorn updates written as row-wise
 * log-sum-exp reductions of biased dot-product scores (review, Summary: the
 * cost has the form alpha_i + beta_j - Q_i.K_j). The library evaluates them
 * tile by tile on the GPU; the n x m cost and plan matrices are never stored.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless stated otherwise. Arrays are dense and
 *    row-major: x is n x d, y is m x d, V/U/out are (rows x k), grad_x is n x d.
 *    x and y are float32 (SK_F32) or bfloat16 bit patterns (SK_BF16); every
 *    other array is float32. x, y, V need 16-byte alignment.
 *  - The caller owns all memory. The library allocates nothing and keeps no
 *    state between calls apart from loaded code objects and a thread-local
 *    error string. Scratch memory is the caller's workspace `ws` of at least
 *    sk_workspace_bytes(...) bytes (256-byte aligned); its contents on entry
 *    are ignored and on exit are unspecified.
 *  - `stream` is a hipStream_t (NULL: the default stream). All work is enqueued
 *    on it asynchronously; outputs are valid once the stream has synchronized.
 *    Calls on the same workspace must not overlap.
 *  - Return value: SK_OK (0) or a negative SK_ERR_* code. Arguments are
 *    validated on the host before anything is enqueued; on a validation error
 *    nothing is enqueued and no output is touched. sk_last_error() gives the
 *    message of the calling thread's last failure.
 *  - NaN or Inf inputs propagate to the outputs; they are not detected.
 *    A weight vector that sums to zero makes the potentials +Inf.
 */
#ifndef FLASHSK_H
#define FLASHSK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SK_VERSION 1

/* return codes */
#define SK_OK 0
#define SK_ERR_INVALID_ARG (-1) /* a size, pointer, eps, mode or flag is invalid  */
#define SK_ERR_UNSUPPORTED (-2) /* a valid combination the library does not handle */
#define SK_ERR_WORKSPACE (-3)   /* ws is NULL, misaligned or too small            */
#define SK_ERR_HIP (-4)         /* the HIP runtime reported an error              */

/* storage type of x and y */
#define SK_F32 0
#define SK_BF16 1

/* schedules (review, Strengths: "symmetric-vs-alternating comparisons") */
#define SK_ALTERNATING 0 /* f <- F(g); then g <- G(f) with the new f            */
#define SK_SYMMETRIC 1   /* (f, g) <- ((f + F(g))/2, (g + G(f))/2) at the old pair */

/* solve flags */
#define SK_WARM_START 1u /* f and g hold the starting potentials (else zeros)  */
#define SK_NO_CENTER 2u  /* do not translate the clouds toward the origin     */
#define SK_CHECK_FINITE 4u /* screen the inputs first (see sk_sinkhorn_solve)    */

/* operations, for sk_workspace_bytes */
#define SK_OP_SOLVE 0
#define SK_OP_APPLY 1
#define SK_OP_GRAD 2
#define SK_OP_DIVERGENCE 3
#define SK_OP_APPLY_HADAMARD 4
#define SK_OP_SOLVE_TOL 5
#define SK_OP_HVP 6
#define SK_OP_NEWTON 7 /* float32 points only */

/*
 * Fixed-budget Sinkhorn solve (FlashSinkhorn abstract; review, Summary and
 * Weaknesses: fixed iteration budgets).
 *   iters      number of full iterations (each is an F half-pass and a G
 *              half-pass); iters = 0 returns the starting potentials and
 *              their cost.
 *   mode       SK_ALTERNATING or SK_SYMMETRIC.
 *   flags      SK_WARM_START, SK_NO_CENTER, SK_CHECK_FINITE.
 *   f, g       out (in/out with SK_WARM_START): n and m float32 potentials.
 *   cost       out: one double, <a, f> + <b, g> at the final pair.
 * Requirements: n, m, d >= 1; eps finite and > 0; iters >= 0. The values
 * themselves are not checked by default: a NaN or infinity in x, y, a, b (or
 * in f, g under SK_WARM_START) propagates into the results. SK_CHECK_FINITE
 * screens them on the device first and waits for the verdict (one host
 * synchronization of `stream`): a NaN or infinity, a negative weight, or an
 * a or b with no positive weight returns SK_ERR_INVALID_ARG before anything
 * that writes f, g or cost is enqueued (the screening writes one workspace
 * word). Nonzero weights are never renormalized.
 */
int sk_sinkhorn_solve(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                      const float* a, const float* b, double eps, int32_t iters, int mode,
                      uint32_t flags, float* f, float* g, double* cost, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Solve to a marginal tolerance (the review's Weaknesses note that iterations
 * to convergence grow sharply at small eps, 2000-5000 in its Table 21).
 * Runs iterations as sk_sinkhorn_solve does, and every `check_every`
 * iterations measures the marginal error of the current pair (f, g),
 *   err = ||P 1 - a||_1 + ||P^T 1 - b||_1,
 * from the iteration that follows it (F(g) normalizes the rows exactly, so the
 * row sums of P(f, g) are a_i exp((f_i - F(g)_i)/eps); after an alternating
 * g-step the column sums are b, so in that schedule a check of the starting
 * pair itself is skipped). It stops after that iteration once err <= tol, or
 * after max_iters iterations (err is then the last one measured, or +Inf).
 *   eps_start  eps-scaling: when eps_start > eps, one iteration at each of
 *              eps_start, eps_start/2, ... while above eps runs first (these
 *              count in iters_done); 0 (or <= eps) disables it.
 *   max_iters, check_every   >= 1.
 *   tol        >= 0, finite. float32 potentials put a floor near
 *              1e-7 * max|f| / eps under the measurable error.
 *   iters_done out (host): iterations run.
 *   err        out (host): the last error measured (of the pair before the
 *              last iteration; the returned pair is one iteration further).
 *   flags      SK_WARM_START, SK_NO_CENTER, SK_CHECK_FINITE (as for the solve).
 * BLOCKING: synchronizes `stream` at every check. The iterations at eps run in
 * one workspace lifetime (one prep; every pass after each side's first uses
 * the shifted sweep), so without eps-scaling the returned pair is bitwise the
 * one sk_sinkhorn_solve returns for iters = iters_done.
 * Workspace: sk_workspace_bytes(SK_OP_SOLVE_TOL, dtype, n, m, d, 0).
 */
int sk_sinkhorn_solve_tol(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                          const float* a, const float* b, double eps, double eps_start, int32_t max_iters,
                          int mode, uint32_t flags, double tol, int32_t check_every, float* f, float* g,
                          double* cost, int32_t* iters_done, double* err, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Matrix-free transport application (review, Summary item ii: transport-vector
 * and transport-matrix applications): with the plan P formed from the given
 * (f, g) as they are (no renormalization),
 *   transpose = 0:  out (n x k) = P V,    V is m x k
 *   transpose = 1:  out (m x k) = P^T V,  V is n x k
 * Requirements: 1 <= k <= 4096 (SK_ERR_UNSUPPORTED above), as for the solve
 * otherwise. Widths above 64 on large d (bf16 d > 128, float32 d > 21) run on
 * the wide kernel (scores once per 512 values); on small d the scores are
 * recomputed once per 64 values.
 * Precision of the plan entries in the value products (bf16 d <= 128,
 * float32 d <= 21, any d for k > 64, float32 points for k <= 32): bf16
 * points, one float16 per entry
 * (relative error <= 2^-11, inside the 1e-3 bound of bf16 inputs); float32
 * points, two float16 parts per entry (2^-22); in both, two float16 parts of
 * each value after an exact power-of-two scale per value column (values
 * below 2^-29 of their column's largest magnitude fall into float16's
 * subnormal range). Otherwise (larger d, k <= 64; float32 points with
 * 32 < k <= 64): bf16 points two bf16 parts of each entry (2^-16) and value,
 * float32 points three (float32 accuracy).
 */
int sk_transport_apply(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                       const float* a, const float* b, const float* f, const float* g, double eps,
                       int transpose, const float* V, int64_t k, float* out, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * Gradient of the EOT cost with respect to x as a barycentric projection (the
 * review's Summary item i: the gradient as a residual attention output):
 *   grad_x_i = 2 a_i (x_i - sum_j pi_ij y_j),
 *   pi_ij = softmax over j of (log b_j + (g_j - C_ij)/eps),
 * using g only. This is the exact derivative of x -> <a, F_x(g)> + <b, g>;
 * it equals the derivative of the cost at a converged pair. The weights pi
 * enter the weighted sum with the precision sk_transport_apply states (their
 * normalizing sum is accumulated in float32), the points y exactly.
 * Requirements as for the solve.
 */
int sk_eot_grad_x(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                  const float* a, const float* b, const float* g, double eps, float* grad_x,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * Hadamard-weighted transport application (review, Summary item ii: the
 * released primitives include Hadamard-weighted transport applications; the
 * pages do not define the weight matrix, so it is taken in the low-rank form
 * that streams): W = A B^T with A (n x r) and B (m x r), float32 row-major,
 *   transpose = 0:  out (n x k) = (P o W) V,     V is m x k
 *   transpose = 1:  out (m x k) = (P o W)^T V,   V is n x k
 * where o is the entrywise product and P is formed from (f, g) as in
 * sk_transport_apply. Evaluated as sum_s diag(A_s) P diag(B_s) V: ranks are
 * taken in groups of floor(64 / k), one matrix-free application per group.
 * Requirements: 1 <= k <= 64 (SK_ERR_UNSUPPORTED above), r >= 1, as for
 * sk_transport_apply otherwise. Workspace: sk_workspace_bytes(SK_OP_APPLY_HADAMARD,
 * dtype, n, m, d, k) (independent of r).
 */
int sk_transport_apply_hadamard(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                                const float* a, const float* b, const float* f, const float* g, double eps,
                                int transpose, const float* A, const float* B, int64_t r, const float* V,
                                int64_t k, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Hessian-vector product of OT_eps with respect to x (the replication review,
 * Summary and Strengths: Theorem 5 reduces the HVP to a Schur solve over
 * streaming plan products, checked against a dense Moore-Penrose reference;
 * the pages print no formula). At the pair (f, g), for a tangent V (n x d):
 *   dC_ij = 2 (x_i - y_j).v_i; (df, dg) keep both marginals of P fixed:
 *   [diag(r) P; P^T diag(c)] [df; dg] = [(P o dC) 1; (P o dC)^T 1],
 *   r = P 1, c = P^T 1, solved by conjugate gradients (preconditioned by
 *   diag(c)) on the Schur
 *   complement diag(c) - P^T diag(1/r) P (relative residual cg_tol, at most
 *   cg_max_iters iterations); dP_ij = P_ij (df_i + dg_j - dC_ij)/eps;
 *   out_i = 2 r_i v_i - 2 sum_j dP_ij y_j.
 * At a converged pair this is the Hessian of OT_eps in x applied to V. All
 * plan products are matrix-free applications (O((n + m) d) memory); the
 * CG's take two bf16 parts per plan entry for bf16 points (2^-16) and, for
 * float32 points, the float16 form of sk_transport_apply (2^-22).
 *   V, out     n x d float32 (V 16-byte aligned).
 *   cg_iters, cg_resid   out (host): CG iterations and final relative residual.
 * The term (P o dC) Y is one weighted application (each plan entry times
 * v_i.y_j, on the matrix cores), and the CG scalars stay on the device.
 * BLOCKING: synchronizes `stream` once per batch of 8 CG iterations (an
 * iteration after convergence in a batch changes nothing).
 * Requirements: d <= 4096 (SK_ERR_UNSUPPORTED above), as for the solve otherwise.
 * Workspace: sk_workspace_bytes(SK_OP_HVP, dtype, n, m, d, 0).
 */
int sk_ot_hvp_x(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                const float* b, const float* f, const float* g, double eps, const float* V, float* out,
                double cg_tol, int32_t cg_max_iters, int32_t* cg_iters, double* cg_resid, void* ws,
                size_t ws_bytes, void* stream);

/*
 * Newton-CG on the points x of the first measure: minimizes
 *   F(x) = OT_eps(sum_i a_i delta_{x_i}, sum_j b_j delta_{y_j})
 * over x (n x d) with y, a, b, eps fixed (the replication review's Summary and
 * Strengths: the streaming HVP makes Newton-CG on OT_eps possible in
 * O((n + m) d) memory; the pages print no algorithm, so the textbook
 * line-search Newton-CG is used). Each iterate's potentials are solved to the
 * marginal error sk_tol (sk_sinkhorn_solve_tol, alternating, a check every 10
 * iterations, at most sk_max_iters; warm from the previous iterate's), F is
 * <a, f> + <b, g>, its gradient sk_eot_grad_x and its Hessian sk_ot_hvp_x
 * (inner Schur CG to 1e-6, at most 500 iterations). The CG on H p = -grad
 * stops at the forcing term min(1/2, sqrt|grad|) |grad|, at cg_max_iters, or
 * at the first direction of non-positive curvature (the first one gives
 * p = -grad); the step t halves from 1 until the Armijo condition
 * F(x + t p) <= F(x) + 1e-4 t grad.p holds (at most 30 halvings, else stop).
 *   x0         n x d float32 start (may equal x).
 *   y          m x d float32 (the points are float32 on both sides).
 *   newton_iters   at most this many steps; grad_tol >= 0 stops earlier once
 *              |grad|_2 <= grad_tol.
 *   x          out: n x d float32, the last iterate.
 *   costs      out (host, newton_iters + 1 doubles, or NULL): F at iterates 0..steps.
 *   grad_norms out (host, newton_iters + 1 doubles, or NULL): |grad|_2 at the
 *              iterates whose gradient was formed (0..steps).
 *   steps_done out (host): steps taken.
 * BLOCKING (host decisions on every CG and line-search step).
 * Requirements: d <= 4096 (SK_ERR_UNSUPPORTED above); sk_tol > 0; as for the
 * solve otherwise. Workspace: sk_workspace_bytes(SK_OP_NEWTON, SK_F32, n, m, d, 0).
 */
int sk_ot_newton_x(const float* x0, const float* y, int64_t n, int64_t m, int64_t d, const float* a,
                   const float* b, double eps, double sk_tol, int32_t sk_max_iters, int32_t newton_iters,
                   double grad_tol, int32_t cg_max_iters, float* x, double* costs, double* grad_norms,
                   int32_t* steps_done, void* ws, size_t ws_bytes, void* stream);

/*
 * Debiased Sinkhorn divergence (the replication review names a
 * "debiased-Sinkhorn" sweep among the OTDD drivers, Weaknesses, "Downstream
 * drivers absent"; the pages print no formula, so the textbook form is used):
 *   S = OT(x,a; y,b) - OT(x,a; x,a)/2 - OT(y,b; y,b)/2,
 * each OT the cost <a,f> + <b,g> of a fixed-budget solve of `iters`
 * iterations: the cross term with `mode`, the two self terms with
 * SK_SYMMETRIC (which keeps their f = g).
 *   flags      SK_NO_CENTER, SK_CHECK_FINITE (screens x, y, a, b once, as
 *              for the solve); warm starts do not apply.
 *   div        out: one double, S.
 *   grad_a     out (n, or NULL): f_ab - f_aa, the gradient of S in a along
 *              mass-preserving directions (off the simplex it holds up to an
 *              additive constant).
 *   grad_b     out (m, or NULL): g_ab - g_bb, likewise in b.
 *   grad_x     out (n x d, or NULL): gradient of S in x, the barycentric
 *              gradient of the cross term minus that of the self term
 *              (x enters the self term on both sides: twice the one-sided
 *              gradient, times 1/2).
 *   grad_y     out (m x d, or NULL): likewise in y.
 * The gradients are exact for the potentials the solves return (envelope
 * argument); they are the gradients of S at converged potentials.
 * Workspace: sk_workspace_bytes(SK_OP_DIVERGENCE, dtype, n, m, d, 0).
 * Requirements as for the solve; x and y may be the same array.
 */
int sk_sinkhorn_divergence(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                           const float* a, const float* b, double eps, int32_t iters, int mode,
                           uint32_t flags, double* div, float* grad_a, float* grad_b, float* grad_x,
                           float* grad_y, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free solve, for callers that cannot allocate device memory or
 * hand over a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Arguments, results and errors as for
 * sk_sinkhorn_solve without ws and ws_bytes. Its scratch is a device array of
 * sk_noalloc_scratch_bytes() bytes (64 MiB) inside the library, one per GPU,
 * held from the library's load until the process ends; the call allocates
 * nothing. A size whose solve workspace (sk_workspace_bytes(SK_OP_SOLVE, ...))
 * exceeds it returns SK_ERR_UNSUPPORTED before anything is enqueued.
 *   flags      SK_WARM_START, SK_NO_CENTER (SK_CHECK_FINITE, which waits for
 *              the stream, is refused with SK_ERR_INVALID_ARG).
 * Every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents (the solve initializes all it reads): calls that overlap on one
 * GPU (on other streams or threads) race, and the caller must order them.
 */
int sk_sinkhorn_solve_noalloc(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                              const float* a, const float* b, double eps, int32_t iters, int mode,
                              uint32_t flags, float* f, float* g, double* cost, void* stream);

/* Bytes of the scratch array sk_sinkhorn_solve_noalloc uses on each GPU. */
size_t sk_noalloc_scratch_bytes(void);

/* Workspace bytes needed by `op` for these sizes (0 on invalid sizes). */
size_t sk_workspace_bytes(int op, int dtype, int64_t n, int64_t m, int64_t d, int64_t k);

/* Message of the calling thread's last failed call ("" if none). Never NULL. */
const char* sk_last_error(void);

/* SK_VERSION of the loaded library. */
int sk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHSK_H */
