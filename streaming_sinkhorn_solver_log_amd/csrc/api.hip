// api.hip -- the extern "C" entry points declared in include/flashsk.h:
// host-side validation, workspace layout and the launch sequence of each call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "flashsk.h"
#include "sk_internal.h"

namespace sk {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SK_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxRows = (int64_t)1 << 30;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Bump allocator over the caller's workspace; with base == nullptr it only sizes.
struct Carve {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += round_up(count * sizeof(T) > 0 ? count * sizeof(T) : 1, kAlign);
    return p;
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Which kernel family serves (dtype, d).
enum class Path { Valu, None };
Path choose_path(int dtype, int64_t d) {
  (void)dtype;
  if (d >= 1 && d <= 16) return Path::Valu;
  return Path::None;
}

int check_common(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                 const float* a, const float* b, double eps) {
  if (!x || !y || !a || !b) return fail(SK_ERR_INVALID_ARG, "null input pointer");
  if (dtype != SK_F32 && dtype != SK_BF16) return fail(SK_ERR_INVALID_ARG, "dtype %d is not SK_F32 or SK_BF16", dtype);
  if (n < 1 || m < 1 || d < 1) return fail(SK_ERR_INVALID_ARG, "sizes must be >= 1 (n=%lld m=%lld d=%lld)", (long long)n, (long long)m, (long long)d);
  if (!(eps > 0.0) || !isfinite(eps)) return fail(SK_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(SK_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (n > kMaxRows || m > kMaxRows || n * d > ((int64_t)1 << 31) - 1 || m * d > ((int64_t)1 << 31) - 1)
    return fail(SK_ERR_UNSUPPORTED, "n*d and m*d must be below 2^31");
  if (choose_path(dtype, d) == Path::None) return fail(SK_ERR_UNSUPPORTED, "dimension d=%lld is not supported by this build", (long long)d);
  return SK_OK;
}

// Workspace of one side (points + per-point vectors).
struct Side {
  float* pts;
  float* alpha;
  float* lw;
  float* h[2];
  float* L;
};

struct SolveLayout {
  Side x, y;
  float2* part;
  unsigned* counters;
  double* centroid;
  float* shift;
  size_t bytes;
};

struct Plans {
  PassPlan f, g;
};

Plans make_plans(int64_t n, int64_t m, int64_t d) {
  Plans p;
  p.f = plan_valu_pass(n, m, (int)d);
  p.g = plan_valu_pass(m, n, (int)d);
  return p;
}

Side carve_side(Carve& c, int64_t cnt, int dp) {
  Side s;
  s.pts = c.take<float>((size_t)cnt * dp);
  s.alpha = c.take<float>(cnt);
  s.lw = c.take<float>(cnt);
  s.h[0] = c.take<float>(cnt);
  s.h[1] = c.take<float>(cnt);
  s.L = c.take<float>(cnt);
  return s;
}

SolveLayout layout_solve(void* ws, int64_t n, int64_t m, int64_t d, size_t part_elems_f2,
                         int n_counters) {
  Carve c{static_cast<char*>(ws)};
  SolveLayout L;
  const int dp = valu_dp((int)d);
  L.x = carve_side(c, n, dp);
  L.y = carve_side(c, m, dp);
  L.part = c.take<float2>(part_elems_f2);
  L.counters = c.take<unsigned>(n_counters);
  L.centroid = c.take<double>((size_t)kCentroidBlocks * 2 * d);
  L.shift = c.take<float>(d);
  L.bytes = c.off;
  return L;
}

size_t solve_part_elems(const Plans& p, int64_t n, int64_t m) {
  const size_t pf = p.f.splits > 1 ? (size_t)p.f.splits * n : 0;
  const size_t pg = p.g.splits > 1 ? (size_t)p.g.splits * m : 0;
  return pf > pg ? pf : pg;
}
int n_counters_for(const Plans& p) { return p.f.row_blocks > p.g.row_blocks ? p.f.row_blocks : p.g.row_blocks; }

size_t solve_bytes(int64_t n, int64_t m, int64_t d) {
  const Plans p = make_plans(n, m, d);
  return layout_solve(nullptr, n, m, d, solve_part_elems(p, n, m), n_counters_for(p)).bytes;
}

// Apply and gradient share the solve's side layout; their partial records are wider.
size_t wide_part_floats(const PassPlan& pl, int64_t nr, int64_t rec) {
  return pl.splits > 1 ? (size_t)pl.splits * nr * rec : 0;
}

size_t apply_bytes(int64_t n, int64_t m, int64_t d, int64_t k, int transpose) {
  const int64_t nr = transpose ? m : n, nc = transpose ? n : m;
  const PassPlan pl = plan_valu_pass(nr, nc, (int)d);
  const size_t f2 = (wide_part_floats(pl, nr, k) + 1) / 2;
  return layout_solve(nullptr, n, m, d, f2, pl.row_blocks).bytes;
}

size_t grad_bytes(int64_t n, int64_t m, int64_t d) {
  const PassPlan pl = plan_valu_pass(n, m, (int)d);
  const size_t f2 = (wide_part_floats(pl, n, 2 + d) + 1) / 2;
  return layout_solve(nullptr, n, m, d, f2, pl.row_blocks).bytes;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(SK_ERR_WORKSPACE, "workspace pointer is null (%zu bytes needed)", need);
  if (!aligned(ws, kAlign)) return fail(SK_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(SK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return SK_OK;
}

struct Scalars {
  float c2, neg_eps_ln2, log2e_over_eps;
};
Scalars scalars(double eps) {
  Scalars s;
  s.c2 = (float)(2.0 * 1.4426950408889634 / eps);
  s.neg_eps_ln2 = (float)(-eps * 0.6931471805599453);
  s.log2e_over_eps = (float)(1.4426950408889634 / eps);
  return s;
}

hipError_t prep_sides(const SolveLayout& L, const void* x, const void* y, int dtype, int64_t n,
                      int64_t m, int64_t d, const float* a, const float* b, const float* f_start,
                      const float* g_start, float* f_zero, float* g_zero, bool center,
                      int n_counters, const Scalars& sc, hipStream_t s) {
  PrepSide px{x, a, f_start, f_zero, L.x.pts, L.x.alpha, L.x.lw, L.x.h[0], n};
  PrepSide py{y, b, g_start, g_zero, L.y.pts, L.y.alpha, L.y.lw, L.y.h[0], m};
  return launch_prep(px, py, dtype, (int)d, valu_dp((int)d), center, L.centroid, L.shift,
                     L.counters, n_counters, sc.log2e_over_eps, s);
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sk_version(void) { return SK_VERSION; }

const char* sk_last_error(void) { return g_err; }

size_t sk_workspace_bytes(int op, int dtype, int64_t n, int64_t m, int64_t d, int64_t k) {
  if (n < 1 || m < 1 || d < 1 || n > kMaxRows || m > kMaxRows) return 0;
  if (choose_path(dtype, d) == Path::None) return 0;
  switch (op) {
    case SK_OP_SOLVE: return solve_bytes(n, m, d);
    case SK_OP_APPLY: {
      if (k < 1 || k > 64) return 0;
      const size_t a0 = apply_bytes(n, m, d, k, 0), a1 = apply_bytes(n, m, d, k, 1);
      return a0 > a1 ? a0 : a1;
    }
    case SK_OP_GRAD: return grad_bytes(n, m, d);
    default: return 0;
  }
}

int sk_sinkhorn_solve(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                      const float* a, const float* b, double eps, int32_t iters, int mode,
                      uint32_t flags, float* f, float* g, double* cost, void* ws, size_t ws_bytes,
                      void* stream) {
  g_err[0] = 0;
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps);
  if (rc) return rc;
  if (!f || !g || !cost) return fail(SK_ERR_INVALID_ARG, "null output pointer");
  if (iters < 0) return fail(SK_ERR_INVALID_ARG, "iters must be >= 0");
  if (mode != SK_ALTERNATING && mode != SK_SYMMETRIC) return fail(SK_ERR_INVALID_ARG, "mode %d is not SK_ALTERNATING or SK_SYMMETRIC", mode);
  if (flags & ~(SK_WARM_START | SK_NO_CENTER)) return fail(SK_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  const Plans pl = make_plans(n, m, d);
  const int ncnt = n_counters_for(pl);
  const size_t need = layout_solve(nullptr, n, m, d, solve_part_elems(pl, n, m), ncnt).bytes;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const SolveLayout L = layout_solve(ws, n, m, d, solve_part_elems(pl, n, m), ncnt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Scalars sc = scalars(eps);
  const bool warm = (flags & SK_WARM_START) != 0;
  const bool center = (flags & SK_NO_CENTER) == 0;

  hipError_t e = prep_sides(L, x, y, dtype, n, m, d, a, b, warm ? f : nullptr,
                            warm ? g : nullptr, warm ? nullptr : f, warm ? nullptr : g, center,
                            ncnt, sc, s);
  if (e != hipSuccess) return hip_fail(e, "prep");

  const bool sym = (mode == SK_SYMMETRIC);
  int cur = 0;
  for (int t = 0; t < iters; ++t) {
    const int nxt = sym ? 1 - cur : cur;
    PassArgs pf{};
    pf.rows = L.x.pts; pf.cols = L.y.pts; pf.hcol = L.y.h[cur];
    pf.alpha = L.x.alpha; pf.lw = L.x.lw; pf.pot = f; pf.hout = L.x.h[nxt]; pf.Lout = L.x.L;
    pf.part = L.part; pf.counters = L.counters; pf.nr = (int)n; pf.nc = (int)m;
    pf.splits = pl.f.splits; pf.cols_per_split = pl.f.cols_per_split;
    pf.c2 = sc.c2; pf.neg_eps_ln2 = sc.neg_eps_ln2; pf.log2e_over_eps = sc.log2e_over_eps;
    pf.symmetric = sym;
    if ((e = launch_lse_valu(pf, (int)d, pl.f, s)) != hipSuccess) return hip_fail(e, "f half-pass");
    PassArgs pg = pf;
    pg.rows = L.y.pts; pg.cols = L.x.pts; pg.hcol = L.x.h[cur];  // alternating: the new f's bias
    pg.alpha = L.y.alpha; pg.lw = L.y.lw; pg.pot = g; pg.hout = L.y.h[nxt]; pg.Lout = L.y.L;
    pg.nr = (int)m; pg.nc = (int)n; pg.splits = pl.g.splits; pg.cols_per_split = pl.g.cols_per_split;
    if ((e = launch_lse_valu(pg, (int)d, pl.g, s)) != hipSuccess) return hip_fail(e, "g half-pass");
    cur = nxt;
  }
  if ((e = launch_cost(a, f, n, b, g, m, cost, s)) != hipSuccess) return hip_fail(e, "cost");
  return SK_OK;
}

int sk_transport_apply(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                       const float* a, const float* b, const float* f, const float* g, double eps,
                       int transpose, const float* V, int64_t k, float* out, void* ws,
                       size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps);
  if (rc) return rc;
  if (!f || !g || !V || !out) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  if (transpose != 0 && transpose != 1) return fail(SK_ERR_INVALID_ARG, "transpose must be 0 or 1");
  if (k < 1) return fail(SK_ERR_INVALID_ARG, "k must be >= 1");
  if (k > 64) return fail(SK_ERR_UNSUPPORTED, "k=%lld > 64 is not supported", (long long)k);
  const int64_t nr = transpose ? m : n, nc = transpose ? n : m;
  const PassPlan pl = plan_valu_pass(nr, nc, (int)d);
  const size_t f2 = (wide_part_floats(pl, nr, k) + 1) / 2;
  const size_t need = layout_solve(nullptr, n, m, d, f2, pl.row_blocks).bytes;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const SolveLayout L = layout_solve(ws, n, m, d, f2, pl.row_blocks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Scalars sc = scalars(eps);
  hipError_t e = prep_sides(L, x, y, dtype, n, m, d, a, b, f, g, nullptr, nullptr, true,
                            pl.row_blocks, sc, s);
  if (e != hipSuccess) return hip_fail(e, "prep");
  const Side& R = transpose ? L.y : L.x;
  const Side& Cs = transpose ? L.x : L.y;
  ApplyArgs aa{};
  aa.rows = R.pts; aa.cols = Cs.pts; aa.hrow = R.h[0]; aa.hcol = Cs.h[0]; aa.V = V; aa.out = out;
  aa.part = reinterpret_cast<float*>(L.part); aa.counters = L.counters;
  aa.nr = (int)nr; aa.nc = (int)nc; aa.k = (int)k; aa.splits = pl.splits;
  aa.cols_per_split = pl.cols_per_split; aa.c2 = sc.c2;
  if ((e = launch_apply_valu(aa, (int)d, pl, s)) != hipSuccess) return hip_fail(e, "apply");
  return SK_OK;
}

int sk_eot_grad_x(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                  const float* a, const float* b, const float* g, double eps, float* grad_x,
                  void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps);
  if (rc) return rc;
  if (!g || !grad_x) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  const PassPlan pl = plan_valu_pass(n, m, (int)d);
  const size_t f2 = (wide_part_floats(pl, n, 2 + d) + 1) / 2;
  const size_t need = layout_solve(nullptr, n, m, d, f2, pl.row_blocks).bytes;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  const SolveLayout L = layout_solve(ws, n, m, d, f2, pl.row_blocks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Scalars sc = scalars(eps);
  hipError_t e = prep_sides(L, x, y, dtype, n, m, d, a, b, nullptr, g, nullptr, nullptr, true,
                            pl.row_blocks, sc, s);
  if (e != hipSuccess) return hip_fail(e, "prep");
  GradArgs ga{};
  ga.rows = L.x.pts; ga.cols = L.y.pts; ga.hcol = L.y.h[0]; ga.wrow = a; ga.out = grad_x;
  ga.part = reinterpret_cast<float*>(L.part); ga.counters = L.counters;
  ga.nr = (int)n; ga.nc = (int)m; ga.d = (int)d; ga.splits = pl.splits;
  ga.cols_per_split = pl.cols_per_split; ga.c2 = sc.c2;
  if ((e = launch_grad_valu(ga, pl, s)) != hipSuccess) return hip_fail(e, "grad");
  return SK_OK;
}

}  // extern "C"
