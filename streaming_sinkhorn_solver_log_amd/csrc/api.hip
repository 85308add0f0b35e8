// api.hip -- the extern "C" entry points of the core path declared in
// include/flashsk.h (solve, transport application, gradient, sizing, errors):
// host-side validation, workspace layout and the launch sequence of each call.
// The operations composed from them live in compose.hip.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "flashsk.h"
#include "sk_internal.h"
#include "sk_check.h"
#include "sk_mfma.h"
#include "sk_gemm.h"
#include "sk_api.h"
#include <stdlib.h>

namespace sk {
namespace api {

namespace {
thread_local char g_err[512] = "";
}  // namespace

void clear_error() { g_err[0] = 0; }
const char* last_error() { return g_err; }

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

// Kernel family of a call: the matrix-core kernels with register-resident row
// records when they fit (bf16: d <= 128, float32: d <= 21), else the GEMM-tiled
// matrix-core kernels (d <= 4096).
Path solve_path(int dtype, int64_t d) {
  if (d < 1) return Path::None;
  if (d <= 4096 && mfma_nkb(dtype, (int)d) > 0) return Path::Mfma;
  if (d <= 4096) return Path::Gemm;
  return Path::None;
}

Path aux_path(int dtype, int64_t d) { return solve_path(dtype, d); }

int check_common(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                 const float* a, const float* b, double eps, Path path) {
  if (!x || !y || !a || !b) return fail(SK_ERR_INVALID_ARG, "null input pointer");
  if (dtype != SK_F32 && dtype != SK_BF16) return fail(SK_ERR_INVALID_ARG, "dtype %d is not SK_F32 or SK_BF16", dtype);
  if (n < 1 || m < 1 || d < 1) return fail(SK_ERR_INVALID_ARG, "sizes must be >= 1 (n=%lld m=%lld d=%lld)", (long long)n, (long long)m, (long long)d);
  if (!(eps > 0.0) || !isfinite(eps)) return fail(SK_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(SK_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (n > kMaxRows || m > kMaxRows || n * d > ((int64_t)1 << 31) - 1 || m * d > ((int64_t)1 << 31) - 1)
    return fail(SK_ERR_UNSUPPORTED, "n*d and m*d must be below 2^31");
  if (path == Path::None) return fail(SK_ERR_UNSUPPORTED, "dimension d=%lld is not supported by this library", (long long)d);
  return SK_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(SK_ERR_WORKSPACE, "workspace pointer is null (%zu bytes needed)", need);
  if (!aligned(ws, kAlign)) return fail(SK_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(SK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return SK_OK;
}

// SK_CHECK_FINITE: screens the inputs on the device and waits for the
// verdict, so that a bad input fails before the solve enqueues anything that
// writes f, g or cost. `word` is a workspace word the caller re-initializes
// (f, g: warm-start potentials, or null).
int screen_inputs(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                  const float* b, const float* f, const float* g, unsigned* word, hipStream_t s) {
  hipError_t e = launch_check_inputs(x, y, dtype, n, m, d, a, b, f, g, word, s);
  unsigned bits = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&bits, word, sizeof(bits), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "input check");
  if (bits & kBadPoints) return fail(SK_ERR_INVALID_ARG, "x or y holds a NaN or an infinity");
  if (bits & kBadWeights) return fail(SK_ERR_INVALID_ARG, "a or b holds a negative, NaN or infinite weight");
  if (!(bits & kPositiveA) || !(bits & kPositiveB)) return fail(SK_ERR_INVALID_ARG, "a or b has no positive weight");
  if (bits & kBadPotentials) return fail(SK_ERR_INVALID_ARG, "the starting f or g holds a NaN or an infinity");
  return SK_OK;
}

}  // namespace api

namespace {

using namespace api;

// FLASHSK_DEBUG=1: after each matrix-core solve, synchronize the stream and
// report how many workgroups fell back to the exact sweep.
bool debug_enabled() {
  static const bool v = [] {
    const char* e = getenv("FLASHSK_DEBUG");
    return e && e[0] == '1';
  }();
  return v;
}

// FLASHSK_FORCE_EXACT=1 (read on every solve): every shifted half-pass
// recomputes its row blocks exactly, so tests can check that path.
// The one-launch solve of small problems is on unless FLASHSK_SMALL_SOLVE=0
// (read at each plan: tests and timings compare it with the streaming passes).
bool small_enabled() {
  const char* e = getenv("FLASHSK_SMALL_SOLVE");
  return !(e && e[0] == '0');
}

bool force_exact_enabled() {
  const char* e = getenv("FLASHSK_FORCE_EXACT");
  return e && e[0] == '1';
}

// ---------------------------------------------------------------- workspace layouts
// Matrix-core layout of one side: row-form and column-form records, bias records.
struct SideM {
  bf16x8* row_rec;
  bf16x8* col_rec;
  float* alpha;
  float* lw;
  bf16x8* bias[2];
  float* hacc[2];  // the same biases as float32 in accumulator units (padded)
  float* hval[2];
  float* dmax[2];
  float* L;
};

struct Common {
  float2* part;
  unsigned* counters;
  unsigned* exact_count;
  double* centroid;
  float* shift;
};

SideM carve_side_m(Carve& c, int64_t cnt, int nkb, int row_blocks) {
  SideM s;
  const int64_t padded = mfma_padded_count(cnt);
  s.row_rec = c.take<bf16x8>((size_t)cnt * nkb * 2);
  s.col_rec = c.take<bf16x8>((size_t)padded * nkb * 2);
  s.alpha = c.take<float>(cnt);
  s.lw = c.take<float>(cnt);
  s.bias[0] = c.take<bf16x8>((size_t)padded * 2);
  s.bias[1] = c.take<bf16x8>((size_t)padded * 2);
  s.hacc[0] = c.take<float>(padded);
  s.hacc[1] = c.take<float>(padded);
  s.hval[0] = c.take<float>(cnt);
  s.hval[1] = c.take<float>(cnt);
  s.dmax[0] = c.take<float>(row_blocks);
  s.dmax[1] = c.take<float>(row_blocks);
  s.L = c.take<float>(cnt);
  return s;
}

Common carve_common(Carve& c, size_t part_f2, int n_counters, int64_t d) {
  Common k;
  k.part = c.take<float2>(part_f2);
  k.counters = c.take<unsigned>((n_counters > 0 ? n_counters : 1) + 1);
  // (a sizing pass carves from a null base: no pointer arithmetic on it)
  k.exact_count = k.counters ? k.counters + (n_counters > 0 ? n_counters : 1) : nullptr;
  k.centroid = c.take<double>((size_t)kCentroidBlocks * 2 * d);
  k.shift = c.take<float>(d);
  return k;
}

size_t part_f2_of(const PassPlan& pl, int64_t nr) { return pl.splits > 1 ? (size_t)pl.splits * nr : 0; }

// Split partials of the two half-passes: shared when they run one after the
// other, side by side when they share a launch (fused).
size_t part_f2(const PassPlan& f, int64_t n, const PassPlan& g, int64_t m, bool fused = false) {
  const size_t pf = part_f2_of(f, n), pg = part_f2_of(g, m);
  if (fused) return pf + pg;
  return pf > pg ? pf : pg;
}

struct SolvePlan {
  Path path;
  int nkb;      // matrix-core records: K blocks per record
  bool merged;  // register-resident pass with the bias chunk inside the column records
  bool fused;   // averaged schedule, register-resident pass: F and G in one launch
  PassPlan f, g;
};

// The merged layout keeps one bias copy per side inside its column records, so
// it serves the alternating schedule only (the averaged one reads the old
// biases of both sides while writing the new ones).
SolvePlan plan_solve(int dtype, int64_t n, int64_t m, int64_t d, bool alternating, bool allow_small = true) {
  SolvePlan sp;
  sp.path = solve_path(dtype, d);
  sp.nkb = 0;
  sp.merged = false;
  sp.fused = false;
  if (allow_small && sp.path != Path::None && small_fits(n, m, d, alternating) && small_enabled()) {
    sp.path = Path::Small;
    sp.f = PassPlan{};
    sp.g = PassPlan{};
    return sp;
  }
  if (sp.path == Path::Mfma) {
    sp.nkb = mfma_nkb(dtype, (int)d);
    sp.merged = alternating && mfma_merged(dtype, (int)d, sp.nkb);
    // the averaged schedule's two half-passes read only the previous pair:
    // one launch runs both, each on half of the resident workgroups
    sp.fused = !alternating;
    const int share = sp.fused ? 2 : 1;
    sp.f = plan_mfma_pass(n, m, sp.nkb, sp.merged, dtype == SK_BF16, share);
    sp.g = plan_mfma_pass(m, n, sp.nkb, sp.merged, dtype == SK_BF16, share);
  } else if (sp.path == Path::Gemm) {
    sp.nkb = gemm_nkb(dtype, (int)d);
    sp.f = plan_gemm_pass(n, m);
    sp.g = plan_gemm_pass(m, n);
  }
  return sp;
}

struct SolveWs {
  SideM xm, ym;
  Common c;
  void* tags;  // one-launch solve of small problems: its tagged potentials
  size_t bytes;
};

// Row-block arrival counters: one set shared by passes that run one after the
// other, one per pass when they share a launch.
int solve_counters(const SolvePlan& sp) {
  if (sp.fused) return sp.f.row_blocks + sp.g.row_blocks;
  return sp.f.row_blocks > sp.g.row_blocks ? sp.f.row_blocks : sp.g.row_blocks;
}

SolveWs layout_solve(void* ws, const SolvePlan& sp, int64_t n, int64_t m, int64_t d) {
  Carve c{static_cast<char*>(ws)};
  SolveWs L{};
  if (sp.path == Path::Small) {  // the tagged potentials and the input screen's flag only
    L.c = carve_common(c, 1, 1, d);
    L.tags = c.take<char>(small_ws_bytes(n, m));
    L.bytes = c.off;
    return L;
  }
  L.xm = carve_side_m(c, n, sp.nkb, sp.f.row_blocks);
  L.ym = carve_side_m(c, m, sp.nkb, sp.g.row_blocks);
  L.c = carve_common(c, part_f2(sp.f, n, sp.g, m, sp.fused), solve_counters(sp), d);
  L.bytes = c.off;
  return L;
}

struct Scalars {
  float c2, inv_c2, neg_eps_ln2, log2e_over_eps;
};
Scalars scalars(double eps) {
  Scalars s;
  s.c2 = (float)(2.0 * 1.4426950408889634 / eps);
  s.inv_c2 = (float)(eps / (2.0 * 1.4426950408889634));
  s.neg_eps_ln2 = (float)(-eps * 0.6931471805599453);
  s.log2e_over_eps = (float)(1.4426950408889634 / eps);
  return s;
}

// Matrix-core gradient / transport application: records of both sides, value
// fragments of the column side, split partials of (mu, S, values).
struct AuxPlan {
  Path path;
  int nkb;
  int kv, nobt, nob, nchunks, pp, vp;
  bool half;  // float16 parts of entries and values (else bf16 parts)
  int wq;  // weighted application: tangent record arrays (0: unweighted)
  int64_t nr, nc;
  PassPlan pl;
};

// weighted: the application of the plan entries times t_i.y_j to the values
// y (rows x, columns y), which runs on the GEMM-tiled wide kernel at any d.
AuxPlan plan_aux(int dtype, int64_t n, int64_t m, int64_t d, int64_t kv, bool grad, int transpose,
                 bool weighted = false, bool precise = false) {
  AuxPlan ap{};
  ap.path = weighted ? (d <= 4096 ? Path::Gemm : Path::None) : aux_path(dtype, d);
  ap.wq = weighted ? (dtype == SK_BF16 ? 2 : 1) : 0;
  ap.nr = transpose ? m : n;
  ap.nc = transpose ? n : m;
  ap.kv = (int)kv;
  if (ap.path == Path::Mfma || ap.path == Path::Gemm) {
    const bool gemm = ap.path == Path::Gemm;
    ap.nkb = gemm ? gemm_nkb(dtype, (int)d) : mfma_nkb(dtype, (int)d);
    const int blocks = (int)((kv + 31) / 32);
    // the float16 form runs on the register-resident kernel and, on the
    // GEMM path, on the wide kernel (value widths above 64) and, for float32
    // points, the 8-wave kernel (one value block); not in the weighted
    // application
    const bool half_kernel = !gemm || (!weighted && (blocks > 2 || (blocks == 1 && dtype == SK_F32)));
    pv_parts(dtype, grad || weighted, half_kernel, precise, ap.pp, ap.vp, ap.half);
    ap.nob = weighted ? pv_wide_nob(blocks, ap.vp, true) : pv_nob(gemm, blocks, ap.vp);
    ap.nchunks = (blocks + ap.nob - 1) / ap.nob;
    ap.nobt = ap.nchunks * ap.nob;
    ap.pl = plan_pv(gemm, ap.nr, ap.nc, ap.nkb, ap.nob, ap.vp, ap.nchunks, ap.half);
  }
  return ap;
}

struct AuxWsM {
  SideM x, y;
  bf16x8* vfrag;
  unsigned* vmax;  // half-precision form: column maxima of the values
  int64_t vtiles;
  bf16x8* wrec;  // weighted application: tangent records of the rows
  float* qoff;
  Common c;
  size_t bytes;
};

AuxWsM layout_aux_m(void* ws, const AuxPlan& ap, int64_t n, int64_t m, int64_t d) {
  Carve c{static_cast<char*>(ws)};
  AuxWsM L{};
  L.x = carve_side_m(c, n, ap.nkb, 1);
  L.y = carve_side_m(c, m, ap.nkb, 1);
  L.vtiles = mfma_padded_count(ap.nc) / 32;
  L.vfrag = c.take<bf16x8>((size_t)L.vtiles * ap.nobt * ap.vp * 2 * 64);
  if (ap.half) L.vmax = c.take<unsigned>((size_t)ap.kv);
  // (mu, S) pairs, padded to 16 bytes, then the value partials
  const size_t slots_rows = (size_t)ap.nchunks * ap.pl.splits * ap.nr;
  const size_t part_floats = ap.pl.splits > 1
      ? round_up(2 * slots_rows, 4) + slots_rows * 32 * ap.nob : 0;
  L.c = carve_common(c, (part_floats + 1) / 2, ap.nchunks * ap.pl.row_blocks, d);
  if (ap.wq > 0) {
    L.wrec = c.take<bf16x8>((size_t)ap.wq * ap.nr * ap.nkb * 2);
    L.qoff = c.take<float>(ap.nr);
  }
  L.bytes = c.off;
  return L;
}

// Workspace of a transport application or gradient.
size_t aux_bytes(const AuxPlan& ap, int64_t n, int64_t m, int64_t d) {
  return layout_aux_m(nullptr, ap, n, m, d).bytes;
}

// Prep of both sides (records, norms, log-weights, biases of the given
// potentials, centering shift), value fragments of the column side, then the
// P V / gradient launch.
int run_aux_m(const AuxPlan& ap, const AuxWsM& L, const void* x, const void* y, int dtype, int64_t n,
              int64_t m, int64_t d, const float* a, const float* b, const float* f, const float* g,
              bool grad, int transpose, const void* vsrc, bool vsrc_bf16, float* out,
              const Scalars& sc, hipStream_t s, const float* tangent = nullptr) {
  const int ncnt = ap.nchunks * ap.pl.row_blocks;
  MfmaPrepSide px{x, a, f, nullptr, L.x.row_rec, L.x.col_rec, L.x.alpha, L.x.lw,
                  L.x.bias[0], L.x.bias[1], L.x.hval[0], n};
  MfmaPrepSide py{y, b, g, nullptr, L.y.row_rec, L.y.col_rec, L.y.alpha, L.y.lw,
                  L.y.bias[0], L.y.bias[1], L.y.hval[0], m};
  hipError_t e = launch_prep_mfma(px, py, dtype, (int)d, ap.nkb, false, true, L.c.centroid, L.c.shift,
                                  L.c.counters, ncnt + 1, sc.log2e_over_eps, sc.c2, ap.path == Path::Gemm, s);
  if (e != hipSuccess) return hip_fail(e, "prep");
  const float* shift = L.c.shift;  // centering shift of both clouds (exact for bf16 points)
  e = launch_pack_values(vsrc, vsrc_bf16, ap.nc, ap.kv, grad ? shift : nullptr, ap.vp, ap.nobt,
                         L.vtiles, ap.half ? L.vmax : nullptr, L.vfrag, s);
  if (e != hipSuccess) return hip_fail(e, "value packing");
  const SideM& R = transpose ? L.y : L.x;
  const SideM& C = transpose ? L.x : L.y;
  PvArgs pa{};
  pa.rows = R.row_rec; pa.cols = C.col_rec; pa.bias_col = C.bias[0]; pa.vfrag = L.vfrag;
  pa.vmax = ap.half ? L.vmax : nullptr;
  pa.nobt = ap.nobt; pa.kv = ap.kv; pa.out = out;
  pa.hrow = R.hval[0]; pa.wrow = a; pa.xrow = x; pa.xbf16 = dtype == SK_BF16; pa.shift = shift;
  pa.grad = grad ? 1 : 0;
  pa.part = reinterpret_cast<float*>(L.c.part);
  pa.nr = (int)ap.nr; pa.nc = (int)ap.nc; pa.row_blocks = ap.pl.row_blocks; pa.nchunks = ap.nchunks;
  pa.splits = ap.pl.splits; pa.cols_per_split = ap.pl.cols_per_split;
  pa.escale = mfma_escale(dtype, sc.c2);
  if (ap.wq > 0) {
    const int64_t stride = (int64_t)ap.nr * ap.nkb * 2;
    e = launch_pack_tangent(tangent, dtype == SK_BF16, ap.nr, (int)d, ap.nkb, shift, L.wrec, stride, L.qoff, s);
    if (e != hipSuccess) return hip_fail(e, "tangent records");
    pa.wrec = L.wrec;
    pa.wrec_stride = stride;
    pa.qoff = L.qoff;
  }
  e = launch_pv(pa, ap.path == Path::Gemm, ap.nkb, ap.nob, ap.pp, ap.vp, ap.half, ap.pl, s);
  if (e != hipSuccess) return hip_fail(e, grad ? "grad" : "apply");
  return SK_OK;
}

hipError_t launch_pass(const SolvePlan& sp, const MfmaPassArgs& a, bool shifted, bool scaled,
                       const PassPlan& pl, hipStream_t s) {
  if (sp.path == Path::Gemm) return launch_lse_gemm(a, sp.nkb, shifted, scaled, pl, s);
  return launch_lse_mfma(a, sp.nkb, shifted, scaled, sp.merged, pl, s);
}

// Iterations t0 .. t0 + iters - 1 of a solve whose prep has run (t counts the
// iterations since the prep: each side's first pass, t = 0, is the exact
// sweep, every later one the shifted sweep). `cur` selects the bias buffers the
// next iteration reads (the averaged schedule alternates them).
int solve_mfma(const SolveWs& L, const SolvePlan& sp, int dtype, int64_t n, int64_t m, int t0, int iters,
               int& cur, bool sym, float* f, float* g, const Scalars& sc, hipStream_t s) {
  hipError_t e;
  const bool scaled = dtype == SK_BF16;
  const int force_exact = force_exact_enabled() ? 1 : 0;
  for (int t = t0; t < t0 + iters; ++t) {
    const int nxt = sym ? 1 - cur : cur;
    // Each side's first pass has no previous log-sum-exp to shift by: exact sweep.
    const bool shifted = t > 0;
    MfmaPassArgs pf{};
    pf.rows = L.xm.row_rec; pf.cols = L.ym.col_rec; pf.bias_col = L.ym.bias[cur];
    pf.alpha = L.xm.alpha; pf.lw = L.xm.lw; pf.pot = f; pf.bias_out = L.xm.bias[nxt]; pf.bias_stride = 2;
    if (sp.merged) {  // the bias chunk is the last chunk of each column record
      pf.bias_col = nullptr;
      pf.bias_out = L.xm.col_rec + (2 * sp.nkb - 1);
      pf.bias_stride = 2 * sp.nkb;
    }
    pf.Lout = L.xm.L; pf.Lin = L.xm.L; pf.hval_in = L.xm.hval[cur]; pf.hval_out = L.xm.hval[nxt];
    pf.hcol = L.ym.hacc[cur]; pf.hout = L.xm.hacc[nxt];
    pf.dmax_in = L.ym.dmax[cur]; pf.n_dmax_in = sp.g.row_blocks; pf.dmax_out = L.xm.dmax[nxt];
    pf.exact_count = L.c.exact_count;
    pf.part = L.c.part; pf.counters = L.c.counters;
    pf.nr = (int)n; pf.nc = (int)m; pf.splits = sp.f.splits; pf.cols_per_split = sp.f.cols_per_split;
    pf.row_blocks = sp.f.row_blocks; pf.stages = sp.f.stages; pf.chunks = sp.f.chunks;
    pf.escale = mfma_escale(dtype, sc.c2); pf.bias_scale = mfma_bias_scale(dtype, sc.c2);
    pf.neg_eps_ln2 = sc.neg_eps_ln2; pf.log2e_over_eps = sc.log2e_over_eps; pf.symmetric = sym;
    pf.force_exact = force_exact;
    if (!sp.fused && (e = launch_pass(sp, pf, shifted, scaled, sp.f, s)) != hipSuccess)
      return hip_fail(e, "f half-pass");
    MfmaPassArgs pg = pf;
    pg.rows = L.ym.row_rec; pg.cols = L.xm.col_rec; pg.bias_col = L.xm.bias[cur];
    pg.alpha = L.ym.alpha; pg.lw = L.ym.lw; pg.pot = g; pg.bias_out = L.ym.bias[nxt]; pg.bias_stride = 2;
    if (sp.merged) {
      pg.bias_col = nullptr;
      pg.bias_out = L.ym.col_rec + (2 * sp.nkb - 1);
      pg.bias_stride = 2 * sp.nkb;
    }
    pg.Lout = L.ym.L; pg.Lin = L.ym.L; pg.hval_in = L.ym.hval[cur]; pg.hval_out = L.ym.hval[nxt];
    pg.hcol = L.xm.hacc[cur]; pg.hout = L.ym.hacc[nxt];
    pg.dmax_in = L.xm.dmax[cur]; pg.n_dmax_in = sp.f.row_blocks; pg.dmax_out = L.ym.dmax[nxt];
    pg.nr = (int)m; pg.nc = (int)n; pg.splits = sp.g.splits; pg.cols_per_split = sp.g.cols_per_split;
    pg.row_blocks = sp.g.row_blocks; pg.stages = sp.g.stages; pg.chunks = sp.g.chunks;
    if (sp.fused) {
      // both passes in one launch, each with its own partials and counters
      pg.part = L.c.part + part_f2_of(sp.f, n);
      pg.counters = L.c.counters + sp.f.row_blocks;
      if ((e = launch_lse_mfma_pair(pf, sp.f, pg, &sp.g, sp.nkb, shifted, scaled, sp.merged, s)) != hipSuccess)
        return hip_fail(e, "f and g half-passes");
    } else if ((e = launch_pass(sp, pg, shifted, scaled, sp.g, s)) != hipSuccess) {
      return hip_fail(e, "g half-pass");
    }
    cur = nxt;
  }
  return SK_OK;
}

// The state of one solve between its launches: plan, workspace layout and the
// position in the schedule. solve_begin validates the workspace, screens the
// inputs when asked, and runs the prep; solve_iterate then adds iterations, so
// a caller can stop between them (to measure an error) and continue with the
// same records, biases and shifted-sweep state.
struct SolveState {
  SolvePlan sp;
  SolveWs L;
  Scalars sc;
  int dtype;
  int64_t n, m, d;
  bool sym;
  int t;    // iterations since the prep
  int cur;  // bias buffers the next iteration reads
  bool cold;  // started from zero potentials (not SK_WARM_START)
  // the one-launch path recomputes everything from the inputs and (f, g)
  const void* x;
  const void* y;
  const float* a;
  const float* b;
  double eps;
};

int solve_begin(SolveState& st, const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                const float* a, const float* b, double eps, int mode, uint32_t flags, float* f, float* g,
                void* ws, size_t ws_bytes, hipStream_t s) {
  st.sp = plan_solve(dtype, n, m, d, mode == SK_ALTERNATING);
  int rc = check_ws(ws, ws_bytes, layout_solve(nullptr, st.sp, n, m, d).bytes);
  if (rc) return rc;
  st.L = layout_solve(ws, st.sp, n, m, d);
  st.sc = scalars(eps);
  st.dtype = dtype;
  st.n = n;
  st.m = m;
  st.d = d;
  st.sym = mode == SK_SYMMETRIC;
  st.t = 0;
  st.cur = 0;
  st.x = x;
  st.y = y;
  st.a = a;
  st.b = b;
  st.eps = eps;
  const bool warm = (flags & SK_WARM_START) != 0;
  st.cold = !warm;
  if ((flags & SK_CHECK_FINITE) &&
      (rc = screen_inputs(x, y, dtype, n, m, d, a, b, warm ? f : nullptr, warm ? g : nullptr, st.L.c.counters, s)))
    return rc;
  if (st.sp.path == Path::Small) return SK_OK;  // a cold start is zeroed by the first launch
  const SolveWs& L = st.L;
  MfmaPrepSide px{x, a, warm ? f : nullptr, warm ? nullptr : f, L.xm.row_rec, L.xm.col_rec, L.xm.alpha, L.xm.lw,
                  L.xm.bias[0], L.xm.bias[1], L.xm.hval[0], n};
  MfmaPrepSide py{y, b, warm ? g : nullptr, warm ? nullptr : g, L.ym.row_rec, L.ym.col_rec, L.ym.alpha, L.ym.lw,
                  L.ym.bias[0], L.ym.bias[1], L.ym.hval[0], m};
  px.hacc = L.xm.hacc[0]; px.hacc_alt = L.xm.hacc[1];
  py.hacc = L.ym.hacc[0]; py.hacc_alt = L.ym.hacc[1];
  // counters and the exact-fallback count are zeroed together (adjacent)
  hipError_t e = launch_prep_mfma(px, py, dtype, (int)d, st.sp.nkb, st.sp.merged, (flags & SK_NO_CENTER) == 0,
                                  L.c.centroid, L.c.shift, L.c.counters, solve_counters(st.sp) + 1,
                                  st.sc.log2e_over_eps, st.sc.c2, st.sp.path == Path::Gemm, s);
  if (e != hipSuccess) return hip_fail(e, "prep");
  return SK_OK;
}

int solve_iterate(SolveState& st, int iters, float* f, float* g, hipStream_t s) {
  if (st.sp.path == Path::Small) {
    const hipError_t e = launch_small_solve(st.x, st.y, st.dtype, st.n, st.m, st.d, st.a, st.b, st.eps, iters,
                                            st.sym, f, g, st.cold && st.t == 0, st.L.tags, s);
    if (e != hipSuccess) return hip_fail(e, "small-problem solve");
    st.t += iters;
    return SK_OK;
  }
  const int rc = solve_mfma(st.L, st.sp, st.dtype, st.n, st.m, st.t, iters, st.cur, st.sym, f, g, st.sc, s);
  st.t += iters;
  return rc;
}

}  // namespace

namespace api {

size_t solve_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  // the schedule is not known here: the larger of the two plans, sized for
  // the streaming passes also where the one-launch solve would run (so that
  // the workspace serves either choice)
  const size_t a = layout_solve(nullptr, plan_solve(dtype, n, m, d, true, false), n, m, d).bytes;
  const size_t b = layout_solve(nullptr, plan_solve(dtype, n, m, d, false, false), n, m, d).bytes;
  return a > b ? a : b;
}

size_t apply_bytes(int dtype, int64_t n, int64_t m, int64_t d, int64_t k, int transpose, bool precise) {
  return aux_bytes(plan_aux(dtype, n, m, d, k, false, transpose, false, precise), n, m, d);
}

size_t grad_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  return aux_bytes(plan_aux(dtype, n, m, d, d, true, 0), n, m, d);
}

size_t apply_weighted_bytes(int dtype, int64_t n, int64_t m, int64_t d) {
  return aux_bytes(plan_aux(dtype, n, m, d, d, false, 0, true), n, m, d);
}

int apply_weighted(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                   const float* b, const float* f, const float* g, double eps, const float* T, float* out, void* ws,
                   size_t ws_bytes, hipStream_t s) {
  const AuxPlan ap = plan_aux(dtype, n, m, d, d, false, 0, true);
  if (ap.path == Path::None) return fail(SK_ERR_UNSUPPORTED, "d=%lld is beyond the weighted application", (long long)d);
  int rc = check_ws(ws, ws_bytes, aux_bytes(ap, n, m, d));
  if (rc) return rc;
  const AuxWsM L = layout_aux_m(ws, ap, n, m, d);
  // values: the column points as given (the centering only enters the records)
  return run_aux_m(ap, L, x, y, dtype, n, m, d, a, b, f, g, false, 0, y, dtype == SK_BF16, out, scalars(eps), s, T);
}

int solve_to_tolerance(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                       const float* b, double eps, int mode, uint32_t flags, int32_t max_iters, int32_t check_every,
                       double tol, float* f, float* g, double* cost, TolScratch scratch, int32_t* iters_done,
                       double* err, void* ws, size_t ws_bytes, hipStream_t s) {
  SolveState st;
  int rc = solve_begin(st, x, y, dtype, n, m, d, a, b, eps, mode, flags & ~SK_CHECK_FINITE, f, g, ws, ws_bytes, s);
  if (rc) return rc;
  const double inv_eps = 1.0 / eps;
  const bool avg = mode == SK_SYMMETRIC;
  int32_t done = 0;
  double e_host = INFINITY;
  hipError_t e;
  while (done < max_iters) {
    // iterations up to the next check, then the checking iteration itself
    const int32_t left = max_iters - done;
    const int32_t run = (check_every - 1 < left - 1) ? check_every - 1 : left - 1;
    if (run > 0) {
      if ((rc = solve_iterate(st, run, f, g, s))) return rc;
      done += run;
    }
    // alternating: the columns of the checked pair are exact only once this
    // loop's own g-step produced it, so a check of the starting pair is skipped
    const bool measurable = avg || done > 0;
    if (measurable && ((e = hipMemcpyAsync(scratch.f0, f, n * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess ||
                       (e = hipMemcpyAsync(scratch.g0, g, m * sizeof(float), hipMemcpyDeviceToDevice, s)) != hipSuccess))
      return hip_fail(e, "copy");
    if ((rc = solve_iterate(st, 1, f, g, s))) return rc;
    done += 1;
    if (!measurable) continue;
    if ((e = launch_marginal_error(a, scratch.f0, f, n, inv_eps, avg, false, scratch.err, s)) != hipSuccess ||
        (avg && (e = launch_marginal_error(b, scratch.g0, g, m, inv_eps, true, true, scratch.err, s)) != hipSuccess))
      return hip_fail(e, "marginal error");
    if ((e = hipMemcpyAsync(&e_host, scratch.err, sizeof(double), hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess)
      return hip_fail(e, "marginal error");
    if (e_host <= tol) break;
  }
  if ((e = launch_cost(a, f, n, b, g, m, cost, s)) != hipSuccess) return hip_fail(e, "cost");
  *iters_done = done;
  *err = e_host;
  return SK_OK;
}

int transport_apply(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                    const float* b, const float* f, const float* g, double eps, int transpose, const float* V,
                    int64_t k, float* out, void* ws, size_t ws_bytes, void* stream, bool precise) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, aux_path(dtype, d));
  if (rc) return rc;
  if (!f || !g || !V || !out) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  if (transpose != 0 && transpose != 1) return fail(SK_ERR_INVALID_ARG, "transpose must be 0 or 1");
  if (k < 1) return fail(SK_ERR_INVALID_ARG, "k must be >= 1");
  if (k > kMaxValueCols)
    return fail(SK_ERR_UNSUPPORTED, "k=%lld > %lld is not supported", (long long)k, (long long)kMaxValueCols);
  const AuxPlan ap = plan_aux(dtype, n, m, d, k, false, transpose, false, precise);
  if ((rc = check_ws(ws, ws_bytes, aux_bytes(ap, n, m, d)))) return rc;
  if (small_aux_fits(n, m, d, k) && small_enabled()) {
    const hipError_t e = launch_small_aux(x, y, dtype, n, m, d, a, b, f, g, eps, transpose, false, V, k, out,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SK_OK : hip_fail(e, "small-problem transport application");
  }
  const AuxWsM L = layout_aux_m(ws, ap, n, m, d);
  return run_aux_m(ap, L, x, y, dtype, n, m, d, a, b, f, g, false, transpose, V, false, out, scalars(eps),
                   static_cast<hipStream_t>(stream));
}

}  // namespace api
}  // namespace sk

using namespace sk;
using namespace sk::api;

extern "C" {

int sk_version(void) { return SK_VERSION; }

const char* sk_last_error(void) { return last_error(); }

size_t sk_workspace_bytes(int op, int dtype, int64_t n, int64_t m, int64_t d, int64_t k) {
  if (n < 1 || m < 1 || d < 1 || n > kMaxRows || m > kMaxRows) return 0;
  if (dtype != SK_F32 && dtype != SK_BF16) return 0;
  switch (op) {
    case SK_OP_SOLVE:
      if (solve_path(dtype, d) == Path::None) return 0;
      return solve_bytes(dtype, n, m, d);
    case SK_OP_APPLY: {
      if (aux_path(dtype, d) == Path::None || k < 1 || k > kMaxValueCols) return 0;
      const size_t a0 = apply_bytes(dtype, n, m, d, k, 0), a1 = apply_bytes(dtype, n, m, d, k, 1);
      return a0 > a1 ? a0 : a1;
    }
    case SK_OP_GRAD:
      if (aux_path(dtype, d) == Path::None) return 0;
      return grad_bytes(dtype, n, m, d);
    case SK_OP_SOLVE_TOL:
      if (solve_path(dtype, d) == Path::None) return 0;
      return solve_tol_ws_bytes(dtype, n, m, d);
    case SK_OP_HVP:
      if (aux_path(dtype, d) == Path::None || d > kHvpMaxD) return 0;
      return hvp_ws_bytes(dtype, n, m, d);
    case SK_OP_APPLY_HADAMARD:
      if (aux_path(dtype, d) == Path::None || k < 1 || k > kHadamardCols) return 0;
      return hadamard_ws_bytes(dtype, n, m, d);
    case SK_OP_NEWTON:
      if (dtype != SK_F32 || aux_path(dtype, d) == Path::None || d > kHvpMaxD) return 0;
      return newton_ws_bytes(n, m, d);
    case SK_OP_DIVERGENCE:
      if (solve_path(dtype, d) == Path::None) return 0;
      return divergence_ws_bytes(dtype, n, m, d);
    default: return 0;
  }
}

int sk_sinkhorn_solve(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                      const float* a, const float* b, double eps, int32_t iters, int mode,
                      uint32_t flags, float* f, float* g, double* cost, void* ws, size_t ws_bytes,
                      void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, solve_path(dtype, d));
  if (rc) return rc;
  if (!f || !g || !cost) return fail(SK_ERR_INVALID_ARG, "null output pointer");
  if (iters < 0) return fail(SK_ERR_INVALID_ARG, "iters must be >= 0");
  if (mode != SK_ALTERNATING && mode != SK_SYMMETRIC) return fail(SK_ERR_INVALID_ARG, "mode %d is not SK_ALTERNATING or SK_SYMMETRIC", mode);
  if (flags & ~(SK_WARM_START | SK_NO_CENTER | SK_CHECK_FINITE))
    return fail(SK_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SolveState st;
  if ((rc = solve_begin(st, x, y, dtype, n, m, d, a, b, eps, mode, flags, f, g, ws, ws_bytes, s))) return rc;
  if ((rc = solve_iterate(st, iters, f, g, s))) return rc;
  if (debug_enabled() && st.sp.path != Path::Small) {
    unsigned cnt = 0;
    if (hipMemcpyAsync(&cnt, st.L.c.exact_count, sizeof(cnt), hipMemcpyDeviceToHost, s) == hipSuccess &&
        hipStreamSynchronize(s) == hipSuccess)
      fprintf(stderr, "[flashsk] solve n=%lld m=%lld d=%lld iters=%d: %u workgroup(s) used the exact fallback\n",
              (long long)n, (long long)m, (long long)d, iters, cnt);
  }
  hipError_t e = launch_cost(a, f, n, b, g, m, cost, s);
  if (e != hipSuccess) return hip_fail(e, "cost");
  return SK_OK;
}

int sk_transport_apply(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                       const float* a, const float* b, const float* f, const float* g, double eps,
                       int transpose, const float* V, int64_t k, float* out, void* ws,
                       size_t ws_bytes, void* stream) {
  return sk::api::transport_apply(x, y, dtype, n, m, d, a, b, f, g, eps, transpose, V, k, out, ws, ws_bytes,
                                  stream, false);
}

int sk_eot_grad_x(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                  const float* a, const float* b, const float* g, double eps, float* grad_x,
                  void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, aux_path(dtype, d));
  if (rc) return rc;
  if (!g || !grad_x) return fail(SK_ERR_INVALID_ARG, "null pointer argument");
  const AuxPlan ap = plan_aux(dtype, n, m, d, d, true, 0);
  if ((rc = check_ws(ws, ws_bytes, aux_bytes(ap, n, m, d)))) return rc;
  if (small_aux_fits(n, m, d, d) && small_enabled()) {
    const hipError_t e = launch_small_aux(x, y, dtype, n, m, d, a, b, nullptr, g, eps, 0, true, nullptr, 0, grad_x,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SK_OK : hip_fail(e, "small-problem gradient");
  }
  const AuxWsM L = layout_aux_m(ws, ap, n, m, d);
  return run_aux_m(ap, L, x, y, dtype, n, m, d, a, b, nullptr, g, true, 0, y, dtype == SK_BF16, grad_x,
                   scalars(eps), static_cast<hipStream_t>(stream));
}

}  // extern "C"
