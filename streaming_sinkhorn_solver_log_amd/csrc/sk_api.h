// sk_api.h -- helpers shared by the C-ABI entry points (api.hip) and the
// operations composed from them (compose.hip). Library-internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "flashsk.h"

namespace sk {
namespace api {

constexpr size_t kAlign = 256;                  // workspace alignment
constexpr int64_t kMaxRows = (int64_t)1 << 30;  // largest n or m
constexpr int64_t kHadamardCols = 64;           // value columns per application
constexpr int kHvpMaxD = 4096;                  // largest d of the Hessian-vector product
constexpr int64_t kMaxValueCols = 4096;         // largest value width of a transport application

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

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

// Small: the whole fixed-budget solve of a small problem in one cooperative
// launch (solve only; see small.hip).
enum class Path { Mfma, Gemm, Small, None };

// Thread-local error message (sk_last_error): fail() formats it and returns code.
void clear_error();
const char* last_error();
int fail(int code, const char* fmt, ...);
int hip_fail(hipError_t e, const char* where);

Path solve_path(int dtype, int64_t d);
Path aux_path(int dtype, int64_t d);
// Host validation common to every entry point (pointers, dtype, sizes, eps, path).
int check_common(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                 const float* a, const float* b, double eps, Path path);
int check_ws(void* ws, size_t ws_bytes, size_t need);
// SK_CHECK_FINITE screening: launches the input check, waits for its verdict
// (one synchronization of s) and returns SK_ERR_INVALID_ARG on a NaN or an
// infinity in x, y (or f, g when non-null), a negative or non-finite weight,
// or a marginal with no positive weight. `word` is a workspace word.
int screen_inputs(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                  const float* b, const float* f, const float* g, unsigned* word, hipStream_t s);

// Device scratch of the tolerance loop: the pair before the checking
// iteration and the error it measures.
struct TolScratch {
  float* f0;
  float* g0;
  double* err;
};
// The tolerance phase of sk_sinkhorn_solve_tol at a fixed eps (arguments
// validated by the caller; SK_CHECK_FINITE is the caller's to apply): one
// prep, then iterations in one workspace lifetime (every pass after each
// side's first runs the shifted sweep), the marginal error of the pair before
// every check_every-th iteration measured from that iteration, until it is
// <= tol or max_iters iterations have run. ws: solve_bytes(dtype, n, m, d).
int solve_to_tolerance(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                       const float* b, double eps, int mode, uint32_t flags, int32_t max_iters, int32_t check_every,
                       double tol, float* f, float* g, double* cost, TolScratch scratch, int32_t* iters_done,
                       double* err, void* ws, size_t ws_bytes, hipStream_t s);
// out (+)= sum_i w_i |expm1((p0_i - M_i) inv_eps)| in float64 with M = p1
// (or 2 p1 - p0 when averaged): the L1 marginal error of the pair (p0, .)
// from the map value the following iteration computed (compose.hip).
hipError_t launch_marginal_error(const float* w, const float* p0, const float* p1, int64_t cnt, double inv_eps,
                                 bool averaged, bool accumulate, double* out, hipStream_t s);

// Workspace bytes of the core entry points (api.hip).
size_t solve_bytes(int dtype, int64_t n, int64_t m, int64_t d);
size_t apply_bytes(int dtype, int64_t n, int64_t m, int64_t d, int64_t k, int transpose, bool precise = false);
// sk_transport_apply with precise = true: bf16 points keep two bf16 parts per
// plan entry (relative error 2^-16) instead of one float16 part; for the
// applications inside the Hessian-vector product's CG, whose Schur system
// amplifies entry rounding (float32 points are the same either way).
// ws: apply_bytes(..., precise).
int transport_apply(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                    const float* b, const float* f, const float* g, double eps, int transpose, const float* V,
                    int64_t k, float* out, void* ws, size_t ws_bytes, void* stream, bool precise);
size_t grad_bytes(int dtype, int64_t n, int64_t m, int64_t d);
// Weighted application (rows x, columns y, any d <= 4096, arguments validated
// by the caller): out_i = sum_j P_ij (t_i . y_j) y_j, out and T n x d float32;
// the (P o T Y^T) Y term of the Hessian-vector product.
size_t apply_weighted_bytes(int dtype, int64_t n, int64_t m, int64_t d);
int apply_weighted(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d, const float* a,
                   const float* b, const float* f, const float* g, double eps, const float* T, float* out, void* ws,
                   size_t ws_bytes, hipStream_t s);
// Workspace bytes of the composed operations (compose.hip).
size_t divergence_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d);
size_t hadamard_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d);
size_t solve_tol_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d);
size_t hvp_ws_bytes(int dtype, int64_t n, int64_t m, int64_t d);
size_t newton_ws_bytes(int64_t n, int64_t m, int64_t d);

}  // namespace api
}  // namespace sk
