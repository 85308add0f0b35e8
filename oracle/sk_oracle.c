/*
 * sk_oracle.c -- CPU float64 reference ("oracle") for streaming log-domain Sinkhorn.
 *
 * TEST INFRASTRUCTURE ONLY. It is built and called by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg. The GPU library neither links
 * nor calls it, and the two share no source, header, table or helper.
 *
 * Problem (entropic optimal transport between weighted point clouds, squared
 * Euclidean cost; FlashSinkhorn abstract, and the replication review's Summary):
 *   points  x_i (i < n), y_j (j < m) in R^d, weights a_i >= 0, b_j >= 0
 *   cost    C_ij = sum_k (x_ik - y_jk)^2      (computed by direct differences,
 *                                              never by the |x|^2+|y|^2-2x.y expansion)
 *   plan    P_ij = a_i b_j exp((f_i + g_j - C_ij) / eps)
 *   maps    F(g)_i = -eps * LSE_j( log b_j + (g_j - C_ij)/eps )
 *           G(f)_j = -eps * LSE_i( log a_i + (f_i - C_ij)/eps )
 * The stabilized log-domain Sinkhorn update is exactly "f <- F(g)", a row-wise
 * log-sum-exp, and "g <- G(f)", a column-wise one (replication review, Summary).
 * LSE is evaluated in two passes: the maximum first, then max + log sum exp(z - max).
 *
 * Schedules (the review's Strengths paragraph names a symmetric and an
 * alternating variant; the averaged form is this code's reading of "symmetric"):
 *   alternating: f <- F(g); then g <- G(f) with the new f
 *   symmetric:   (f, g) <- ( (f + F(g))/2, (g + G(f))/2 ), both maps at the old pair
 * The reported cost is <a, f> + <b, g> at the final pair.
 *
 * Transport applications (review, Summary item ii): (P V)_i = sum_j P_ij V_j and
 * (P^T U)_j = sum_i P_ij U_i with the plan formed from the given (f, g), never stored.
 * Gradient (review, Summary item i: the EOT gradient as a barycentric projection):
 *   grad_i = 2 a_i (x_i - sum_j pi_ij y_j),  pi_ij = softmax_j(log b_j + (g_j - C_ij)/eps),
 * the exact derivative of x -> <a, F_x(g)> + <b, g> at fixed g.
 *
 * All arithmetic is IEEE float64 in plain loops; OpenMP splits the outer loop
 * over rows and nothing else.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SKO_ALTERNATING 0
#define SKO_SYMMETRIC 1

int sko_version(void) { return 1; }

void sko_set_threads(int t) {
#ifdef _OPENMP
  if (t > 0) omp_set_num_threads(t);
#else
  (void)t;
#endif
}

int sko_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Squared Euclidean distance by direct differences. */
static double sqdist(const double* u, const double* v, int64_t d) {
  double s = 0.0;
  for (int64_t k = 0; k < d; ++k) {
    double t = u[k] - v[k];
    s += t * t;
  }
  return s;
}

/* log-sum-exp of z[0..len), two passes; all terms -inf gives -inf. */
static double lse(const double* z, int64_t len) {
  double mx = -INFINITY;
  for (int64_t j = 0; j < len; ++j)
    if (z[j] > mx) mx = z[j];
  if (mx == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int64_t j = 0; j < len; ++j) s += exp(z[j] - mx);
  return mx + log(s);
}

/*
 * The one-sided log-domain map, written once for either side:
 *   out_r = -eps * LSE_c( log w_c + (pot_c - C(rows_r, cols_c)) / eps ).
 * F(g) is row_map(x, y, b, g); G(f) is row_map(y, x, a, f), since C is symmetric
 * in its two point arguments.
 */
static void row_map(const double* rows, const double* cols, int64_t nr, int64_t nc, int64_t d,
                    const double* w, const double* pot, double eps, double* out) {
#pragma omp parallel
  {
    double* z = (double*)malloc((size_t)(nc > 0 ? nc : 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < nr; ++r) {
      for (int64_t c = 0; c < nc; ++c) {
        double cost = sqdist(rows + r * d, cols + c * d, d);
        z[c] = log(w[c]) + (pot[c] - cost) / eps;
      }
      out[r] = -eps * lse(z, nc);
    }
    free(z);
  }
}

/* f_out = F(g) */
void sko_F(const double* x, const double* y, int64_t n, int64_t m, int64_t d, const double* b,
           const double* g, double eps, double* f_out) {
  row_map(x, y, n, m, d, b, g, eps, f_out);
}

/* g_out = G(f) */
void sko_G(const double* x, const double* y, int64_t n, int64_t m, int64_t d, const double* a,
           const double* f, double eps, double* g_out) {
  row_map(y, x, m, n, d, a, f, eps, g_out);
}

/*
 * Fixed-budget Sinkhorn. f (n) and g (m) hold the starting potentials on entry
 * (zeros for a cold start) and the final ones on exit. One iteration is two
 * half-steps in either schedule. *cost = <a, f> + <b, g> at the final pair.
 */
void sko_solve(const double* x, const double* y, int64_t n, int64_t m, int64_t d, const double* a,
               const double* b, double eps, int iters, int mode, double* f, double* g,
               double* cost) {
  double* tf = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  double* tg = (double*)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
  for (int t = 0; t < iters; ++t) {
    if (mode == SKO_SYMMETRIC) {
      sko_F(x, y, n, m, d, b, g, eps, tf); /* F at the old g */
      sko_G(x, y, n, m, d, a, f, eps, tg); /* G at the old f */
      for (int64_t i = 0; i < n; ++i) f[i] = 0.5 * (f[i] + tf[i]);
      for (int64_t j = 0; j < m; ++j) g[j] = 0.5 * (g[j] + tg[j]);
    } else {
      sko_F(x, y, n, m, d, b, g, eps, f);
      sko_G(x, y, n, m, d, a, f, eps, g); /* uses the new f */
    }
  }
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += a[i] * f[i];
  for (int64_t j = 0; j < m; ++j) s += b[j] * g[j];
  *cost = s;
  free(tf);
  free(tg);
}

/* Barycentric-projection gradient with respect to x, from the final g only. */
void sko_grad_x(const double* x, const double* y, int64_t n, int64_t m, int64_t d,
                const double* a, const double* b, const double* g, double eps, double* grad) {
#pragma omp parallel
  {
    double* z = (double*)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      for (int64_t j = 0; j < m; ++j)
        z[j] = log(b[j]) + (g[j] - sqdist(x + i * d, y + j * d, d)) / eps;
      double L = lse(z, m);
      for (int64_t k = 0; k < d; ++k) grad[i * d + k] = 0.0;
      for (int64_t j = 0; j < m; ++j) {
        double pi = exp(z[j] - L);
        for (int64_t k = 0; k < d; ++k) grad[i * d + k] += pi * y[j * d + k];
      }
      for (int64_t k = 0; k < d; ++k) grad[i * d + k] = 2.0 * a[i] * (x[i * d + k] - grad[i * d + k]);
    }
    free(z);
  }
}

/* The plan entry P_ij at the given potentials. */
static double plan_entry(const double* xi, const double* yj, int64_t d, double ai, double bj,
                         double fi, double gj, double eps) {
  if (ai == 0.0 || bj == 0.0) return 0.0;
  return ai * bj * exp((fi + gj - sqdist(xi, yj, d)) / eps);
}

/* Diagnostic gradient from the plan itself: 2 (r_i x_i - sum_j P_ij y_j), r = P 1. */
void sko_grad_x_plan(const double* x, const double* y, int64_t n, int64_t m, int64_t d,
                     const double* a, const double* b, const double* f, const double* g,
                     double eps, double* grad) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double r = 0.0;
    for (int64_t k = 0; k < d; ++k) grad[i * d + k] = 0.0;
    for (int64_t j = 0; j < m; ++j) {
      double p = plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps);
      r += p;
      for (int64_t k = 0; k < d; ++k) grad[i * d + k] += p * y[j * d + k];
    }
    for (int64_t k = 0; k < d; ++k) grad[i * d + k] = 2.0 * (r * x[i * d + k] - grad[i * d + k]);
  }
}

/*
 * transpose == 0: out (n x k) = P V with V (m x k).
 * transpose == 1: out (m x k) = P^T V with V (n x k).
 */
void sko_apply(const double* x, const double* y, int64_t n, int64_t m, int64_t d, const double* a,
               const double* b, const double* f, const double* g, double eps, int transpose,
               const double* V, int64_t k, double* out) {
  if (!transpose) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      for (int64_t c = 0; c < k; ++c) out[i * k + c] = 0.0;
      for (int64_t j = 0; j < m; ++j) {
        double p = plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps);
        for (int64_t c = 0; c < k; ++c) out[i * k + c] += p * V[j * k + c];
      }
    }
  } else {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < m; ++j) {
      for (int64_t c = 0; c < k; ++c) out[j * k + c] = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        double p = plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps);
        for (int64_t c = 0; c < k; ++c) out[j * k + c] += p * V[i * k + c];
      }
    }
  }
}

/*
 * Hadamard-weighted application (the replication review, Summary item ii,
 * names Hadamard-weighted transport applications; W is not defined on the
 * pages: here W = A B^T with A (n x r), B (m x r), the form that streams).
 * Written from the definition, entry by entry: W_ij = sum_s A_is B_js and
 *   transpose == 0: out (n x k) = (P o W) V,       V (m x k)
 *   transpose == 1: out (m x k) = (P o W)^T V,     V (n x k)
 */
void sko_apply_hadamard(const double* x, const double* y, int64_t n, int64_t m, int64_t d,
                        const double* a, const double* b, const double* f, const double* g, double eps,
                        int transpose, const double* A, const double* B, int64_t r, const double* V,
                        int64_t k, double* out) {
  if (!transpose) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      for (int64_t c = 0; c < k; ++c) out[i * k + c] = 0.0;
      for (int64_t j = 0; j < m; ++j) {
        double w = 0.0;
        for (int64_t s2 = 0; s2 < r; ++s2) w += A[i * r + s2] * B[j * r + s2];
        const double pw = plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps) * w;
        for (int64_t c = 0; c < k; ++c) out[i * k + c] += pw * V[j * k + c];
      }
    }
  } else {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < m; ++j) {
      for (int64_t c = 0; c < k; ++c) out[j * k + c] = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        double w = 0.0;
        for (int64_t s2 = 0; s2 < r; ++s2) w += A[i * r + s2] * B[j * r + s2];
        const double pw = plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps) * w;
        for (int64_t c = 0; c < k; ++c) out[j * k + c] += pw * V[i * k + c];
      }
    }
  }
}

/* Row and column sums of the plan: r = P 1 (n), c = P^T 1 (m). */
void sko_marginals(const double* x, const double* y, int64_t n, int64_t m, int64_t d,
                   const double* a, const double* b, const double* f, const double* g, double eps,
                   double* r, double* c) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < m; ++j) s += plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps);
    r[i] = s;
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < m; ++j) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += plan_entry(x + i * d, y + j * d, d, a[i], b[j], f[i], g[j], eps);
    c[j] = s;
  }
}

/*
 * Primal and dual objectives at (f, g):
 *   primal = <P, C> + eps * KL(P | a (x) b), generalized KL = sum P log(P/ab) - sum P + sum ab
 *            (the extra terms of the generalized divergence: "Fused & Furious", section II.A)
 *   dual   = <a, f> + <b, g> - eps * (sum P - sum ab)
 * log(P_ij / (a_i b_j)) is (f_i + g_j - C_ij) / eps by the plan's definition.
 */
void sko_objectives(const double* x, const double* y, int64_t n, int64_t m, int64_t d,
                    const double* a, const double* b, const double* f, const double* g, double eps,
                    double* primal, double* dual) {
  double pc = 0.0, plogp = 0.0, psum = 0.0, absum = 0.0, af = 0.0, bg = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : pc, plogp, psum, absum)
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t j = 0; j < m; ++j) {
      double cost = sqdist(x + i * d, y + j * d, d);
      double ab = a[i] * b[j];
      absum += ab;
      if (ab == 0.0) continue;
      double lr = (f[i] + g[j] - cost) / eps;
      double p = ab * exp(lr);
      pc += p * cost;
      plogp += p * lr;
      psum += p;
    }
  }
  for (int64_t i = 0; i < n; ++i) af += a[i] * f[i];
  for (int64_t j = 0; j < m; ++j) bg += b[j] * g[j];
  *primal = pc + eps * (plogp - psum + absum);
  *dual = af + bg - eps * (psum - absum);
}
