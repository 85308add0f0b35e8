// compose.hip -- operations composed from the core entry points: the debiased
// Sinkhorn divergence, the Hadamard-weighted transport application, the solve
// to a marginal tolerance and the Hessian-vector product (declared in
// include/flashsk.h). Each validates its arguments on the host, lays out the
// caller's workspace, and calls the core entry points plus a few elementwise
// and reduction kernels of its own.
#include <math.h>

#include "flashsk.h"
#include "sk_api.h"

namespace sk {
namespace {

using namespace api;

// ---------------------------------------------------------------- divergence
// Debiased Sinkhorn divergence S = OT(a,b) - OT(a,a)/2 - OT(b,b)/2 and its
// gradients, composed from the solve and gradient entry points below (the
// review names a "debiased-Sinkhorn" sweep among the OTDD drivers,
// Weaknesses, "Downstream drivers absent"; the textbook form is used).

__global__ void k_div_combine(const double* __restrict__ c, double* __restrict__ out) {
  if (threadIdx.x == 0 && blockIdx.x == 0) out[0] = c[0] - 0.5 * c[1] - 0.5 * c[2];
}

// out = p - q, elementwise (out may alias p)
__global__ void k_sub(const float* p, const float* __restrict__ q, float* out, int64_t cnt) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = p[i] - q[i];
}

hipError_t launch_sub(const float* p, const float* q, float* out, int64_t cnt, hipStream_t s) {
  const int64_t blocks = (cnt + 255) / 256;
  k_sub<<<(int)(blocks < 4096 ? blocks : 4096), 256, 0, s>>>(p, q, out, cnt);
  return hipGetLastError();
}

struct DivWs {
  float *f_ab, *g_ab, *f_aa, *g_aa, *f_bb, *g_bb, *tmp;
  double* costs;
  unsigned* word;
  void* inner;
  size_t inner_bytes, bytes;
};

size_t div_inner_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  size_t need = 0;
  auto take = [&](size_t v) { need = v > need ? v : need; };
  take(solve_bytes(dtype, n, m, d));
  take(solve_bytes(dtype, n, n, d));
  take(solve_bytes(dtype, m, m, d));
  if (aux_path(dtype, d) != Path::None) {
    take(grad_bytes(dtype, n, m, d));
    take(grad_bytes(dtype, n, n, d));
    take(grad_bytes(dtype, m, n, d));
    take(grad_bytes(dtype, m, m, d));
  }
  return need;
}

DivWs layout_div(void* ws, int dtype, int64_t n, int64_t m, int64_t d) {
  Carve c{static_cast<char*>(ws)};
  DivWs L{};
  L.f_ab = c.take<float>(n);
  L.g_ab = c.take<float>(m);
  L.f_aa = c.take<float>(n);
  L.g_aa = c.take<float>(n);
  L.f_bb = c.take<float>(m);
  L.g_bb = c.take<float>(m);
  L.tmp = c.take<float>((size_t)(n > m ? n : m) * d);
  L.costs = c.take<double>(3);
  L.word = c.take<unsigned>(1);
  L.inner_bytes = div_inner_bytes(dtype, n, m, d);
  L.inner = c.take<char>(L.inner_bytes);
  L.bytes = c.off;
  return L;
}

// ---------------------------------------------------------------- run to tolerance
// Marginal error of a pair (f0, g0) from the next iteration (review,
// Weaknesses: iterations to convergence grow sharply at small eps, so a
// solve stops on a streamed marginal check). F(g0) normalizes the
// rows exactly, so the row sums of P(f0, g0) are a_i exp((f0_i - F(g0)_i)/eps)
// and ||P 1 - a||_1 = sum_i a_i |expm1((f0_i - F(g0)_i)/eps)|. The next
// iteration computes F(g0): f1 itself (alternating) or 2 f1 - f0 (averaged,
// whose G(f0) = 2 g1 - g0 gives the column term the same way; after an
// alternating g-step the columns are exact).

// out (+)= sum_i w_i |expm1((p0_i - M_i) inv_eps)|, M = p1 or 2 p1 - p0; one block
__global__ __launch_bounds__(1024) void k_marginal_error(const float* __restrict__ w, const float* __restrict__ p0,
                                                         const float* __restrict__ p1, int64_t cnt, double inv_eps,
                                                         int averaged, int accumulate, double* __restrict__ out) {
  __shared__ double red[16];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < cnt; i += blockDim.x) {
    const float m = averaged ? 2.0f * p1[i] - p0[i] : p1[i];
    acc += (double)w[i] * fabs(expm1((double)(p0[i] - m) * inv_eps));
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int q = 0; q < (int)(blockDim.x >> 6); ++q) t += red[q];
    out[0] = accumulate ? out[0] + t : t;
  }
}

struct TolWs {
  float *f0, *g0;
  double* err;
  unsigned* word;
  void* inner;
  size_t inner_bytes, bytes;
};

TolWs layout_tol(void* ws, int dtype, int64_t n, int64_t m, int64_t d) {
  Carve c{static_cast<char*>(ws)};
  TolWs L{};
  L.f0 = c.take<float>(n);
  L.g0 = c.take<float>(m);
  L.err = c.take<double>(1);
  L.word = c.take<unsigned>(1);
  L.inner_bytes = solve_bytes(dtype, n, m, d);
  L.inner = c.take<char>(L.inner_bytes);
  L.bytes = c.off;
  return L;
}

// ---------------------------------------------------------------- Hessian-vector product
// HVP of OT_eps in x at a pair (f, g) (review, Summary and Strengths:
// Theorem 5 reduces it to a Schur solve over streaming plan products).
// Implicit differentiation of the marginal constraints, for a tangent V:
//   dC_ij = 2 (x_i - y_j).v_i,  s_i = x_i.v_i,  r = P 1,  c = P^T 1
//   u = (P o dC) 1 = 2 (s o r - rowdot(P Y, V)),  w = (P o dC)^T 1 = 2 (P^T s - rowdot(Y, P^T V))
//   [diag(r) P; P^T diag(c)] [df; dg] = [u; w]:  S dg = w - P^T (u / r),
//   S = diag(c) - P^T diag(1/r) P  (conjugate gradients preconditioned by
//   diag(c), which maps the spectrum of S into [0, 1]; S 1 = 0 and the right
//   side is orthogonal to 1, so its mean is removed), df = (u - P dg) / r
//   (H V)_i = 2 r_i v_i - (2/eps) [(df_i - 2 s_i) (P Y)_i + (P (dg o Y))_i + 2 ((P o V Y^T) Y)_i]
// Every plan product is a matrix-free application; the last term is the
// Hadamard-weighted application with W = V Y^T (rank d).

__global__ void k_to_f32(const void* __restrict__ src, int bf16, int64_t cnt, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = bf16 ? __uint_as_float((unsigned)static_cast<const unsigned short*>(src)[i] << 16)
                  : static_cast<const float*>(src)[i];
}

__global__ void k_fill(float* __restrict__ p, float v, int64_t cnt) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// out_i = A_i . B_i (rows of length d)
__global__ void k_rowdot(const float* __restrict__ A, const float* __restrict__ B, int64_t rows, int64_t d,
                         float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += (int64_t)gridDim.x * blockDim.x) {
    float t = 0.0f;
    for (int64_t k = 0; k < d; ++k) t = fmaf(A[i * d + k], B[i * d + k], t);
    out[i] = t;
  }
}

// out = 2 (p * q - t), elementwise (u and w of the derivation)
__global__ void k_two_pq_minus_t(const float* __restrict__ p, const float* __restrict__ q, const float* __restrict__ t,
                                 int64_t cnt, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = 2.0f * ((q ? p[i] * q[i] : p[i]) - t[i]);
}

// out = p / q, elementwise
__global__ void k_div(const float* __restrict__ p, const float* __restrict__ q, int64_t cnt, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = p[i] / q[i];
}

// out = c * p - t, elementwise (the Schur product)
__global__ void k_cp_minus_t(const float* __restrict__ c, const float* __restrict__ p, const float* __restrict__ t,
                             int64_t cnt, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = c[i] * p[i] - t[i];
}

// out[slot] = sum_i p_i q_i in float64; one block
__global__ __launch_bounds__(1024) void k_dot(const float* __restrict__ p, const float* __restrict__ q, int64_t cnt,
                                              double* __restrict__ out) {
  __shared__ double red[16];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < cnt; i += blockDim.x) acc += (double)p[i] * (double)(q ? q[i] : 1.0f);
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) t += red[k];
    out[0] = t;
  }
}

// out[0] = p1 . q1, out[1] = p2 . q2 in float64; one block
__global__ __launch_bounds__(1024) void k_dot2(const float* __restrict__ p1, const float* __restrict__ q1,
                                               const float* __restrict__ p2, const float* __restrict__ q2,
                                               int64_t cnt, double* __restrict__ out) {
  __shared__ double red[2][16];
  double a1 = 0.0, a2 = 0.0;
  for (int64_t i = threadIdx.x; i < cnt; i += blockDim.x) {
    a1 += (double)p1[i] * (double)q1[i];
    a2 += (double)p2[i] * (double)q2[i];
  }
  for (int o = 32; o > 0; o >>= 1) {
    a1 += __shfl_xor(a1, o);
    a2 += __shfl_xor(a2, o);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = a1;
    red[1][threadIdx.x >> 6] = a2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t1 = 0.0, t2 = 0.0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) {
      t1 += red[0][k];
      t2 += red[1][k];
    }
    out[0] = t1;
    out[1] = t2;
  }
}

// p -= mean(p), the mean from a device sum
__global__ void k_sub_mean(float* __restrict__ p, const double* __restrict__ sum, int64_t cnt) {
  const float mean = (float)(sum[0] / (double)cnt);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    p[i] -= mean;
}

// y += alpha x; with xpby: y = x + alpha y
__global__ void k_axpy(float alpha, const float* __restrict__ x, float* __restrict__ y, int64_t cnt, int xpby) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = xpby ? fmaf(alpha, y[i], x[i]) : fmaf(alpha, x[i], y[i]);
}

// out_jk = s_j * Y_jk
__global__ void k_scale_rows(const float* __restrict__ sv, const float* __restrict__ Y, int64_t rows, int64_t d,
                             float* __restrict__ out) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < rows * d; t += (int64_t)gridDim.x * blockDim.x)
    out[t] = sv[t / d] * Y[t];
}

__global__ void k_hvp_out(const float* __restrict__ r, const float* __restrict__ V, const float* __restrict__ df,
                          const float* __restrict__ sv, const float* __restrict__ PY, const float* __restrict__ PDY,
                          const float* __restrict__ HY, int64_t n, int64_t d, float two_over_eps,
                          float* __restrict__ out) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n * d; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / d;
    const float inner = (df[i] - 2.0f * sv[i]) * PY[t] + PDY[t] + 2.0f * HY[t];
    out[t] = 2.0f * r[i] * V[t] - two_over_eps * inner;
  }
}

// Conjugate-gradient state on the device (float64): the scalars of the
// iteration never visit the host, which reads them once per batch.
// (rr, rz) and (rn, rzn) are adjacent: k_dot2 writes each pair at once.
enum CgSlot { kRr = 0, kRz, kZn, kPsp, kRn, kRzn, kIt, kDone, kCgSlots };

__global__ void k_cg_init(double* st, double tol) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    st[kZn] = sqrt(st[kRr]);
    st[kIt] = 0.0;
    st[kDone] = (sqrt(st[kRr]) > tol * st[kZn]) ? 0.0 : 1.0;
  }
}

// q += alpha p, res -= alpha Sp, z = res / c (alpha = rz / pSp), unless done
// or without curvature along p.
__global__ void k_cg_step1(const double* __restrict__ st, float* __restrict__ q, float* __restrict__ res,
                           const float* __restrict__ pp, const float* __restrict__ Sp, const float* __restrict__ c,
                           float* __restrict__ z, int64_t cnt) {
  if (st[kDone] != 0.0 || !(st[kPsp] > 0.0)) return;
  const float alpha = (float)(st[kRz] / st[kPsp]);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x) {
    q[i] = fmaf(alpha, pp[i], q[i]);
    const float r = fmaf(-alpha, Sp[i], res[i]);
    res[i] = r;
    z[i] = r / c[i];
  }
}

// p = z + beta p (beta = rzn / rz), unless done or without curvature.
__global__ void k_cg_step2(const double* __restrict__ st, const float* __restrict__ z, float* __restrict__ pp,
                           int64_t cnt) {
  if (st[kDone] != 0.0 || !(st[kPsp] > 0.0)) return;
  const float beta = (float)(st[kRzn] / st[kRz]);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    pp[i] = fmaf(beta, pp[i], z[i]);
}

// End of an iteration: count it and test the relative residual; no curvature
// along p ends the iteration without counting.
__global__ void k_cg_finish(double* st, double tol) {
  if (threadIdx.x != 0 || blockIdx.x != 0 || st[kDone] != 0.0) return;
  if (!(st[kPsp] > 0.0)) {
    st[kDone] = 1.0;
    return;
  }
  st[kRz] = st[kRzn];
  st[kRr] = st[kRn];
  st[kIt] += 1.0;
  if (!(sqrt(st[kRr]) > tol * st[kZn])) st[kDone] = 1.0;
}

// ---------------------------------------------------------------- Hadamard-weighted application
// (P o W) V with W = A B^T (review, Summary item ii names Hadamard-weighted
// transport applications; W is not defined on the pages, and the low-rank
// form is the one that streams):
//   ((P o W) V)_i = sum_s A_is sum_j P_ij (B_js V_j) = sum_s A_is (P U_s)_i,
// U_s = diag(B_s) V. Ranks go in groups whose values fit one application
// (group size x k <= 64 columns).

// U[row, q k + c] = Wv[row, s0 + q] * V[row, c] for q < gs
__global__ void k_hadamard_values(const float* __restrict__ V, const float* __restrict__ Wv, int64_t rows,
                                  int64_t r, int64_t k, int64_t s0, int64_t gs, float* __restrict__ U) {
  const int64_t total = rows * gs * k;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / (gs * k), rem = t % (gs * k), q = rem / k, c = rem % k;
    U[t] = Wv[row * r + s0 + q] * V[row * k + c];
  }
}

// out[row, c] (+)= sum_q Wo[row, s0 + q] * Z[row, q k + c]
__global__ void k_hadamard_combine(const float* __restrict__ Z, const float* __restrict__ Wo, int64_t rows,
                                   int64_t r, int64_t k, int64_t s0, int64_t gs, int accumulate,
                                   float* __restrict__ out) {
  const int64_t total = rows * k;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = t / k, c = t % k;
    float acc = accumulate ? out[t] : 0.0f;
    for (int64_t q = 0; q < gs; ++q) acc = fmaf(Wo[row * r + s0 + q], Z[row * gs * k + q * k + c], acc);
    out[t] = acc;
  }
}

int grid_for(int64_t total) {
  const int64_t blocks = (total + 255) / 256;
  return (int)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

struct HadWs {
  float *U, *Z;
  void* inner;
  size_t inner_bytes, bytes;
};

HadWs layout_hadamard(void* ws, int dtype, int64_t n, int64_t m, int64_t d) {
  Carve c{static_cast<char*>(ws)};
  HadWs L{};
  const int64_t big = n > m ? n : m;
  L.U = c.take<float>((size_t)big * kHadamardCols);
  L.Z = c.take<float>((size_t)big * kHadamardCols);
  size_t need = 0;
  for (int64_t kk = 1; kk <= kHadamardCols; ++kk) {  // any group width may occur
    const size_t a0 = apply_bytes(dtype, n, m, d, kk, 0), a1 = apply_bytes(dtype, n, m, d, kk, 1);
    need = a0 > need ? a0 : need;
    need = a1 > need ? a1 : need;
  }
  L.inner_bytes = need;
  L.inner = c.take<char>(need);
  L.bytes = c.off;
  return L;
}

struct HvpWs {
  float *xf, *yf, *ones, *r, *c, *PY, *PtV, *sv, *Pts, *u, *w, *tn, *tm, *tm2, *q, *res, *pp, *Sp, *zv, *df, *DY,
      *PDY, *HY;
  double* dots;
  void* inner;
  size_t inner_bytes, bytes;
};

HvpWs layout_hvp(void* ws, int dtype, int64_t n, int64_t m, int64_t d) {
  Carve cv{static_cast<char*>(ws)};
  HvpWs L{};
  const int64_t big = n > m ? n : m;
  L.xf = cv.take<float>(n * d);
  L.yf = cv.take<float>(m * d);
  L.ones = cv.take<float>(big);
  L.r = cv.take<float>(n);
  L.c = cv.take<float>(m);
  L.PY = cv.take<float>(n * d);
  L.PtV = cv.take<float>(m * d);
  L.sv = cv.take<float>(n);
  L.Pts = cv.take<float>(m);
  L.u = cv.take<float>(n);
  L.w = cv.take<float>(m);
  L.tn = cv.take<float>(n);
  L.tm = cv.take<float>(m);
  L.tm2 = cv.take<float>(m);
  L.q = cv.take<float>(m);
  L.res = cv.take<float>(m);
  L.pp = cv.take<float>(m);
  L.Sp = cv.take<float>(m);
  L.zv = cv.take<float>(m);
  L.df = cv.take<float>(n);
  L.DY = cv.take<float>(m * d);
  L.PDY = cv.take<float>(n * d);
  L.HY = cv.take<float>(n * d);
  L.dots = cv.take<double>(kCgSlots);
  size_t need = apply_weighted_bytes(dtype, n, m, d);
  for (int64_t kk : {(int64_t)1, d}) {
    const size_t a0 = apply_bytes(dtype, n, m, d, kk, 0, true), a1 = apply_bytes(dtype, n, m, d, kk, 1, true);
    need = a0 > need ? a0 : need;
    need = a1 > need ? a1 : need;
  }
  L.inner_bytes = need;
  L.inner = cv.take<char>(L.inner_bytes);
  L.bytes = cv.off;
  return L;
}

// ---------------------------------------------------------------- Newton-CG
// Line-search Newton-CG on x -> OT_eps(mu_x, nu) (the replication review's
// Summary and Strengths: the streaming HVP makes Newton-CG on OT_eps possible
// in O((n + m) d) memory; the pages print no algorithm, so the textbook one is
// used): at each iterate the potentials are solved to a marginal tolerance,
// the gradient is the barycentric gradient, the inner CG on H p = -grad stops
// at the forcing term min(1/2, sqrt|g|) |g| or at the first direction of
// non-positive curvature (which falls back to -grad on the first inner
// iteration), and an Armijo backtracking (c1 = 1e-4, up to 30 halvings)
// chooses the step; each trial solve starts from the current potentials.

// out = x + t p, elementwise
__global__ void k_step(const float* __restrict__ x, const float* __restrict__ p, float t, int64_t cnt,
                       float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = fmaf(t, p[i], x[i]);
}

// dv = -r + beta dv, elementwise (the next conjugate direction)
__global__ void k_cg_dir(const float* __restrict__ r, float beta, int64_t cnt, float* __restrict__ dv) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    dv[i] = fmaf(beta, dv[i], -r[i]);
}

// out = -p, elementwise
__global__ void k_neg(const float* __restrict__ p, int64_t cnt, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = -p[i];
}

struct NewtonWs {
  float *f, *g, *ft, *gt, *grad, *z, *r, *dv, *Hd, *p, *xt;
  double *cost, *dots;
  void* inner;
  size_t inner_bytes, bytes;
};

NewtonWs layout_newton(void* ws, int64_t n, int64_t m, int64_t d) {
  Carve c{static_cast<char*>(ws)};
  NewtonWs L{};
  L.f = c.take<float>(n);
  L.g = c.take<float>(m);
  L.ft = c.take<float>(n);
  L.gt = c.take<float>(m);
  L.grad = c.take<float>(n * d);
  L.z = c.take<float>(n * d);
  L.r = c.take<float>(n * d);
  L.dv = c.take<float>(n * d);
  L.Hd = c.take<float>(n * d);
  L.p = c.take<float>(n * d);
  L.xt = c.take<float>(n * d);
  L.cost = c.take<double>(2);
  L.dots = c.take<double>(2);
  size_t need = solve_tol_ws_bytes(SK_F32, n, m, d);
  const size_t gb = grad_bytes(SK_F32, n, m, d), hb = hvp_ws_bytes(SK_F32, n, m, d);
  need = gb > need ? gb : need;
  need = hb > need ? hb : need;
  L.inner_bytes = need;
  L.inner = c.take<char>(need);
  L.bytes = c.off;
  return L;
}

}  // namespace

namespace api {
hipError_t launch_marginal_error(const float* w, const float* p0, const float* p1, int64_t cnt, double inv_eps,
                                 bool averaged, bool accumulate, double* out, hipStream_t s) {
  k_marginal_error<<<1, 1024, 0, s>>>(w, p0, p1, cnt, inv_eps, averaged ? 1 : 0, accumulate ? 1 : 0, out);
  return hipGetLastError();
}
size_t divergence_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  return layout_div(nullptr, dtype, n, m, d).bytes;
}
size_t hadamard_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  return layout_hadamard(nullptr, dtype, n, m, d).bytes;
}
size_t solve_tol_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  return layout_tol(nullptr, dtype, n, m, d).bytes;
}
size_t hvp_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d) { return layout_hvp(nullptr, dtype, n, m, d).bytes; }
size_t newton_ws_bytes(int64_t n, int64_t m, int64_t d) { return layout_newton(nullptr, n, m, d).bytes; }
}  // namespace api
}  // namespace sk

using namespace sk;
using namespace sk::api;

extern "C" {

int sk_sinkhorn_solve_tol(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                          const float* a, const float* b, double eps, double eps_start, int32_t max_iters,
                          int mode, uint32_t flags, double tol, int32_t check_every, float* f, float* g,
                          double* cost, int32_t* iters_done, double* err, void* ws, size_t ws_bytes,
                          void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, solve_path(dtype, d));
  if (rc) return rc;
  if (!f || !g || !cost || !iters_done || !err) return fail(SK_ERR_INVALID_ARG, "null output pointer");
  if (max_iters < 1) return fail(SK_ERR_INVALID_ARG, "max_iters must be >= 1");
  if (check_every < 1) return fail(SK_ERR_INVALID_ARG, "check_every must be >= 1");
  if (!(tol >= 0.0) || !isfinite(tol)) return fail(SK_ERR_INVALID_ARG, "tol must be finite and >= 0");
  if (!(eps_start >= 0.0) || !isfinite(eps_start)) return fail(SK_ERR_INVALID_ARG, "eps_start must be finite and >= 0");
  if (mode != SK_ALTERNATING && mode != SK_SYMMETRIC) return fail(SK_ERR_INVALID_ARG, "mode %d is not SK_ALTERNATING or SK_SYMMETRIC", mode);
  if (flags & ~(SK_WARM_START | SK_NO_CENTER | SK_CHECK_FINITE))
    return fail(SK_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  const TolWs L = layout_tol(ws, dtype, n, m, d);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((flags & SK_CHECK_FINITE) &&
      (rc = screen_inputs(x, y, dtype, n, m, d, a, b, (flags & SK_WARM_START) ? f : nullptr,
                          (flags & SK_WARM_START) ? g : nullptr, L.word, s)))
    return rc;
  const uint32_t keep = flags & SK_NO_CENTER;
  uint32_t fl = flags & (SK_WARM_START | SK_NO_CENTER);
  int32_t done = 0;
  // eps-scaling: one iteration at each of eps_start, eps_start / 2, ... above eps
  for (double ek = eps_start; ek > eps && done < max_iters; ek *= 0.5) {
    if ((rc = sk_sinkhorn_solve(x, y, dtype, n, m, d, a, b, ek, 1, mode, fl, f, g, cost, L.inner, L.inner_bytes,
                                stream)))
      return rc;
    ++done;
    fl = keep | SK_WARM_START;
  }
  int32_t at_eps = 0;
  double e_host = INFINITY;
  if (done < max_iters) {
    // the tolerance phase: one prep, the shifted sweep kept across checks
    if ((rc = solve_to_tolerance(x, y, dtype, n, m, d, a, b, eps, mode, fl, max_iters - done, check_every, tol, f, g,
                                 cost, TolScratch{L.f0, L.g0, L.err}, &at_eps, &e_host, L.inner, L.inner_bytes, s)))
      return rc;
  }
  *iters_done = done + at_eps;
  *err = e_host;
  return SK_OK;
}

int sk_transport_apply_hadamard(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                                const float* a, const float* b, const float* f, const float* g, double eps,
                                int transpose, const float* A, const float* B, int64_t r, const float* V,
                                int64_t k, float* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, aux_path(dtype, d));
  if (rc) return rc;
  if (!f || !g || !A || !B || !V || !out) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  if (transpose != 0 && transpose != 1) return fail(SK_ERR_INVALID_ARG, "transpose must be 0 or 1");
  if (k < 1 || r < 1) return fail(SK_ERR_INVALID_ARG, "k and r must be >= 1");
  if (k > kHadamardCols) return fail(SK_ERR_UNSUPPORTED, "k=%lld > 64 is not supported", (long long)k);
  if (!aligned(V, 16)) return fail(SK_ERR_INVALID_ARG, "V must be 16-byte aligned");
  const HadWs L = layout_hadamard(ws, dtype, n, m, d);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // value side: the points V is indexed by; output side: the other one
  const int64_t vrows = transpose ? n : m, orows = transpose ? m : n;
  const float* Wv = transpose ? A : B;
  const float* Wo = transpose ? B : A;
  const int64_t gmax = kHadamardCols / k;
  for (int64_t s0 = 0; s0 < r; s0 += gmax) {
    const int64_t gs = (r - s0) < gmax ? (r - s0) : gmax;
    k_hadamard_values<<<grid_for(vrows * gs * k), 256, 0, s>>>(V, Wv, vrows, r, k, s0, gs, L.U);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "hadamard values");
    if ((rc = sk_transport_apply(x, y, dtype, n, m, d, a, b, f, g, eps, transpose, L.U, gs * k, L.Z, L.inner,
                                 L.inner_bytes, stream)))
      return rc;
    k_hadamard_combine<<<grid_for(orows * k), 256, 0, s>>>(L.Z, Wo, orows, r, k, s0, gs, s0 > 0 ? 1 : 0, out);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hadamard combine");
  }
  return SK_OK;
}

int sk_ot_hvp_x(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                const float* b, const float* f, const float* g, double eps, const float* V, float* out,
                double cg_tol, int32_t cg_max_iters, int32_t* cg_iters, double* cg_resid, void* ws,
                size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, aux_path(dtype, d));
  if (rc) return rc;
  if (!f || !g || !V || !out || !cg_iters || !cg_resid) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  if (d > kHvpMaxD) return fail(SK_ERR_UNSUPPORTED, "the HVP supports d <= %d (d=%lld)", kHvpMaxD, (long long)d);
  if (!(cg_tol > 0.0) || !isfinite(cg_tol)) return fail(SK_ERR_INVALID_ARG, "cg_tol must be finite and > 0");
  if (cg_max_iters < 1) return fail(SK_ERR_INVALID_ARG, "cg_max_iters must be >= 1");
  if (!aligned(V, 16)) return fail(SK_ERR_INVALID_ARG, "V must be 16-byte aligned");
  const HvpWs L = layout_hvp(ws, dtype, n, m, d);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  // the CG's applications keep two bf16 parts per plan entry for bf16 points
  // (the Schur system amplifies the rounding of a single float16 part);
  // float32 points' applications are the plain ones
  auto apply = [&](const float* vals, int64_t k, int transpose, float* o) {
    return transport_apply(x, y, dtype, n, m, d, a, b, f, g, eps, transpose, vals, k, o, L.inner, L.inner_bytes,
                           stream, true);
  };
  const int64_t big = n > m ? n : m;
  k_to_f32<<<grid_for(n * d), 256, 0, s>>>(x, dtype == SK_BF16, n * d, L.xf);
  k_to_f32<<<grid_for(m * d), 256, 0, s>>>(y, dtype == SK_BF16, m * d, L.yf);
  k_fill<<<grid_for(big), 256, 0, s>>>(L.ones, 1.0f, big);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp prep");
  // marginals of the pair and the plan products the derivation needs
  if ((rc = apply(L.ones, 1, 0, L.r)) || (rc = apply(L.ones, 1, 1, L.c)) || (rc = apply(L.yf, d, 0, L.PY)) ||
      (rc = apply(V, d, 1, L.PtV)))
    return rc;
  k_rowdot<<<grid_for(n), 256, 0, s>>>(L.xf, V, n, d, L.sv);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
  if ((rc = apply(L.sv, 1, 1, L.Pts))) return rc;
  k_rowdot<<<grid_for(n), 256, 0, s>>>(L.PY, V, n, d, L.tn);
  k_two_pq_minus_t<<<grid_for(n), 256, 0, s>>>(L.sv, L.r, L.tn, n, L.u);
  k_rowdot<<<grid_for(m), 256, 0, s>>>(L.yf, L.PtV, m, d, L.tm);
  k_two_pq_minus_t<<<grid_for(m), 256, 0, s>>>(L.Pts, nullptr, L.tm, m, L.w);
  k_div<<<grid_for(n), 256, 0, s>>>(L.u, L.r, n, L.tn);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
  // right side of the Schur system, w - P^T (u / r), with its mean removed
  if ((rc = apply(L.tn, 1, 1, L.tm))) return rc;
  if ((e = launch_sub(L.w, L.tm, L.res, m, s)) != hipSuccess) return hip_fail(e, "hvp");
  k_dot<<<1, 1024, 0, s>>>(L.res, nullptr, m, L.dots + kPsp);
  k_sub_mean<<<grid_for(m), 256, 0, s>>>(L.res, L.dots + kPsp, m);
  k_fill<<<grid_for(m), 256, 0, s>>>(L.q, 0.0f, m);
  k_div<<<grid_for(m), 256, 0, s>>>(L.res, L.c, m, L.zv);
  if ((e = hipGetLastError()) != hipSuccess ||
      (e = hipMemcpyAsync(L.pp, L.zv, m * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return hip_fail(e, "hvp");
  // preconditioned conjugate gradients on S = diag(c) - P^T diag(1/r) P, the
  // scalars on the device; the host looks once per batch of iterations
  k_dot2<<<1, 1024, 0, s>>>(L.res, L.res, L.res, L.zv, m, L.dots + kRr);  // rr, then rz
  k_cg_init<<<1, 64, 0, s>>>(L.dots, cg_tol);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
  double host[kCgSlots];
  int32_t launched = 0;
  constexpr int32_t kBatch = 8;
  bool done = false;
  while (!done && launched < cg_max_iters) {
    const int32_t batch = (cg_max_iters - launched) < kBatch ? cg_max_iters - launched : kBatch;
    for (int32_t t = 0; t < batch; ++t) {
      if ((rc = apply(L.pp, 1, 0, L.tn))) return rc;
      k_div<<<grid_for(n), 256, 0, s>>>(L.tn, L.r, n, L.tn);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
      if ((rc = apply(L.tn, 1, 1, L.tm))) return rc;
      k_cp_minus_t<<<grid_for(m), 256, 0, s>>>(L.c, L.pp, L.tm, m, L.Sp);
      k_dot<<<1, 1024, 0, s>>>(L.pp, L.Sp, m, L.dots + kPsp);
      k_cg_step1<<<grid_for(m), 256, 0, s>>>(L.dots, L.q, L.res, L.pp, L.Sp, L.c, L.zv, m);
      k_dot2<<<1, 1024, 0, s>>>(L.res, L.res, L.res, L.zv, m, L.dots + kRn);  // rn, rzn
      k_cg_step2<<<grid_for(m), 256, 0, s>>>(L.dots, L.zv, L.pp, m);
      k_cg_finish<<<1, 64, 0, s>>>(L.dots, cg_tol);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
    }
    launched += batch;
    if ((e = hipMemcpyAsync(host, L.dots, sizeof(host), hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
      return hip_fail(e, "hvp");
    done = host[kDone] != 0.0;
  }
  if (launched == 0 &&
      ((e = hipMemcpyAsync(host, L.dots, sizeof(host), hipMemcpyDeviceToHost, s)) != hipSuccess ||
       (e = hipStreamSynchronize(s)) != hipSuccess))
    return hip_fail(e, "hvp");
  *cg_iters = (int32_t)host[kIt];
  *cg_resid = host[kZn] > 0.0 ? sqrt(host[kRr]) / host[kZn] : 0.0;
  // df = (u - P dg) / r
  if ((rc = apply(L.q, 1, 0, L.tn))) return rc;
  if ((e = launch_sub(L.u, L.tn, L.tn, n, s)) != hipSuccess) return hip_fail(e, "hvp");
  k_div<<<grid_for(n), 256, 0, s>>>(L.tn, L.r, n, L.df);
  k_scale_rows<<<grid_for(m * d), 256, 0, s>>>(L.q, L.yf, m, d, L.DY);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
  if ((rc = apply(L.DY, d, 0, L.PDY))) return rc;
  // (P o V Y^T) Y: the plan entries weighted by v_i . y_j, applied to Y
  if ((rc = apply_weighted(x, y, dtype, n, m, d, a, b, f, g, eps, V, L.HY, L.inner, L.inner_bytes, s))) return rc;
  k_hvp_out<<<grid_for(n * d), 256, 0, s>>>(L.r, V, L.df, L.sv, L.PY, L.PDY, L.HY, n, d, (float)(2.0 / eps), out);
  if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "hvp");
  return SK_OK;
}

int sk_ot_newton_x(const float* x0, const float* y, int64_t n, int64_t m, int64_t d, const float* a,
                   const float* b, double eps, double sk_tol, int32_t sk_max_iters, int32_t newton_iters,
                   double grad_tol, int32_t cg_max_iters, float* x, double* costs, double* grad_norms,
                   int32_t* steps_done, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(x0, y, SK_F32, n, m, d, a, b, eps, aux_path(SK_F32, d));
  if (rc) return rc;
  if (!x || !steps_done) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(x, 16)) return fail(SK_ERR_INVALID_ARG, "x must be 16-byte aligned");
  if (d > kHvpMaxD) return fail(SK_ERR_UNSUPPORTED, "Newton-CG supports d <= %d (d=%lld)", kHvpMaxD, (long long)d);
  if (!(sk_tol > 0.0) || !isfinite(sk_tol)) return fail(SK_ERR_INVALID_ARG, "sk_tol must be finite and > 0");
  if (sk_max_iters < 1 || cg_max_iters < 1 || newton_iters < 0)
    return fail(SK_ERR_INVALID_ARG, "sk_max_iters and cg_max_iters must be >= 1, newton_iters >= 0");
  if (!(grad_tol >= 0.0) || !isfinite(grad_tol)) return fail(SK_ERR_INVALID_ARG, "grad_tol must be finite and >= 0");
  const NewtonWs L = layout_newton(ws, n, m, d);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int64_t nd = n * d;
  double host[2];
  int32_t its = 0;
  double err = 0.0;
  auto dot = [&](const float* p, const float* q, double& out) -> int {
    k_dot<<<1, 1024, 0, s>>>(p, q, nd, L.dots);
    if ((e = hipGetLastError()) != hipSuccess ||
        (e = hipMemcpyAsync(host, L.dots, sizeof(double), hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
      return hip_fail(e, "newton reduction");
    out = host[0];
    return SK_OK;
  };
  // potentials at xx to the marginal tolerance, warm from (fw, gw) if warm; cost to host
  auto solve_at = [&](const float* xx, float* fw, float* gw, bool warm, double& cost) -> int {
    int r2 = sk_sinkhorn_solve_tol(xx, y, SK_F32, n, m, d, a, b, eps, 0.0, sk_max_iters, SK_ALTERNATING,
                                   warm ? SK_WARM_START : 0u, sk_tol, 10, fw, gw, L.cost, &its, &err, L.inner,
                                   L.inner_bytes, stream);
    if (r2) return r2;
    if ((e = hipMemcpyAsync(host, L.cost, sizeof(double), hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
      return hip_fail(e, "newton cost");
    cost = host[0];
    return SK_OK;
  };
  if (x != x0 && (e = hipMemcpyAsync(x, x0, nd * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return hip_fail(e, "newton copy");
  double cost = 0.0;
  if ((rc = solve_at(x, L.f, L.g, false, cost))) return rc;
  if (costs) costs[0] = cost;
  int32_t steps = 0;
  for (int32_t k = 0; k <= newton_iters; ++k) {
    if ((rc = sk_eot_grad_x(x, y, SK_F32, n, m, d, a, b, L.g, eps, L.grad, L.inner, L.inner_bytes, stream)))
      return rc;
    double gg = 0.0;
    if ((rc = dot(L.grad, L.grad, gg))) return rc;
    const double gn = sqrt(gg);
    if (grad_norms) grad_norms[k] = gn;
    if (k == newton_iters || gn <= grad_tol) break;
    // truncated CG on H p = -grad
    const double tolk = (sqrt(gn) < 0.5 ? sqrt(gn) : 0.5) * gn;
    k_fill<<<grid_for(nd), 256, 0, s>>>(L.z, 0.0f, nd);
    k_neg<<<grid_for(nd), 256, 0, s>>>(L.grad, nd, L.dv);
    if ((e = hipGetLastError()) != hipSuccess ||
        (e = hipMemcpyAsync(L.r, L.grad, nd * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "newton");
    double rr = gg;
    const float* p = L.z;
    for (int32_t j = 0; j < cg_max_iters; ++j) {
      int32_t hits = 0;
      double hres = 0.0;
      if ((rc = sk_ot_hvp_x(x, y, SK_F32, n, m, d, a, b, L.f, L.g, eps, L.dv, L.Hd, 1e-6, 500, &hits, &hres, L.inner,
                            L.inner_bytes, stream)))
        return rc;
      double curv = 0.0;
      if ((rc = dot(L.dv, L.Hd, curv))) return rc;
      if (!(curv > 0.0)) {
        if (j == 0) {
          k_neg<<<grid_for(nd), 256, 0, s>>>(L.grad, nd, L.p);
          if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "newton");
          p = L.p;
        }
        break;
      }
      const double alpha = rr / curv;
      k_axpy<<<grid_for(nd), 256, 0, s>>>((float)alpha, L.dv, L.z, nd, 0);
      k_axpy<<<grid_for(nd), 256, 0, s>>>((float)alpha, L.Hd, L.r, nd, 0);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "newton");
      double rr_new = 0.0;
      if ((rc = dot(L.r, L.r, rr_new))) return rc;
      if (sqrt(rr_new) < tolk) break;
      k_cg_dir<<<grid_for(nd), 256, 0, s>>>(L.r, (float)(rr_new / rr), nd, L.dv);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "newton");
      rr = rr_new;
    }
    // Armijo backtracking along p
    double slope = 0.0;
    if ((rc = dot(L.grad, p, slope))) return rc;
    double t = 1.0, ct = 0.0;
    bool accepted = false;
    for (int h = 0; h <= 30; ++h) {
      k_step<<<grid_for(nd), 256, 0, s>>>(x, p, (float)t, nd, L.xt);
      if ((e = hipGetLastError()) != hipSuccess ||
          (e = hipMemcpyAsync(L.ft, L.f, n * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess ||
          (e = hipMemcpyAsync(L.gt, L.g, m * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail(e, "newton");
      if ((rc = solve_at(L.xt, L.ft, L.gt, true, ct))) return rc;
      if (ct <= cost + 1e-4 * t * slope) {
        accepted = true;
        break;
      }
      t *= 0.5;
    }
    if (!accepted) break;
    if ((e = hipMemcpyAsync(x, L.xt, nd * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(L.f, L.ft, n * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(L.g, L.gt, m * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "newton");
    cost = ct;
    ++steps;
    if (costs) costs[steps] = cost;
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "newton");
  *steps_done = steps;
  return SK_OK;
}

int sk_sinkhorn_divergence(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                           const float* a, const float* b, double eps, int32_t iters, int mode,
                           uint32_t flags, double* div, float* grad_a, float* grad_b, float* grad_x,
                           float* grad_y, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, solve_path(dtype, d));
  if (rc) return rc;
  if (!div) return fail(SK_ERR_INVALID_ARG, "null output pointer");
  if (iters < 0) return fail(SK_ERR_INVALID_ARG, "iters must be >= 0");
  if (mode != SK_ALTERNATING && mode != SK_SYMMETRIC) return fail(SK_ERR_INVALID_ARG, "mode %d is not SK_ALTERNATING or SK_SYMMETRIC", mode);
  if (flags & ~(SK_NO_CENTER | SK_CHECK_FINITE))
    return fail(SK_ERR_INVALID_ARG, "flags 0x%x: only SK_NO_CENTER and SK_CHECK_FINITE apply", flags);
  if ((grad_x || grad_y) && aux_path(dtype, d) == Path::None)
    return fail(SK_ERR_UNSUPPORTED, "gradients at d=%lld are not supported by this library", (long long)d);
  const DivWs L = layout_div(ws, dtype, n, m, d);
  if ((rc = check_ws(ws, ws_bytes, L.bytes))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((flags & SK_CHECK_FINITE) && (rc = screen_inputs(x, y, dtype, n, m, d, a, b, nullptr, nullptr, L.word, s)))
    return rc;
  flags &= SK_NO_CENTER;
  // every sub-call below passes the same validation, so none fails before
  // enqueuing anything unless the HIP runtime does
  if ((rc = sk_sinkhorn_solve(x, y, dtype, n, m, d, a, b, eps, iters, mode, flags, L.f_ab, L.g_ab,
                              L.costs, L.inner, L.inner_bytes, stream)))
    return rc;
  if ((rc = sk_sinkhorn_solve(x, x, dtype, n, n, d, a, a, eps, iters, SK_SYMMETRIC, flags, L.f_aa, L.g_aa,
                              L.costs + 1, L.inner, L.inner_bytes, stream)))
    return rc;
  if ((rc = sk_sinkhorn_solve(y, y, dtype, m, m, d, b, b, eps, iters, SK_SYMMETRIC, flags, L.f_bb, L.g_bb,
                              L.costs + 2, L.inner, L.inner_bytes, stream)))
    return rc;
  k_div_combine<<<1, 64, 0, s>>>(L.costs, div);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "divergence");
  if (grad_a && (e = launch_sub(L.f_ab, L.f_aa, grad_a, n, s)) != hipSuccess) return hip_fail(e, "grad_a");
  if (grad_b && (e = launch_sub(L.g_ab, L.g_bb, grad_b, m, s)) != hipSuccess) return hip_fail(e, "grad_b");
  if (grad_x) {
    if ((rc = sk_eot_grad_x(x, y, dtype, n, m, d, a, b, L.g_ab, eps, grad_x, L.inner, L.inner_bytes, stream)))
      return rc;
    if ((rc = sk_eot_grad_x(x, x, dtype, n, n, d, a, a, L.g_aa, eps, L.tmp, L.inner, L.inner_bytes, stream)))
      return rc;
    if ((e = launch_sub(grad_x, L.tmp, grad_x, n * d, s)) != hipSuccess) return hip_fail(e, "grad_x");
  }
  if (grad_y) {
    if ((rc = sk_eot_grad_x(y, x, dtype, m, n, d, b, a, L.f_ab, eps, grad_y, L.inner, L.inner_bytes, stream)))
      return rc;
    if ((rc = sk_eot_grad_x(y, y, dtype, m, m, d, b, b, L.g_bb, eps, L.tmp, L.inner, L.inner_bytes, stream)))
      return rc;
    if ((e = launch_sub(grad_y, L.tmp, grad_y, m * d, s)) != hipSuccess) return hip_fail(e, "grad_y");
  }
  return SK_OK;
}

}  // extern "C"
