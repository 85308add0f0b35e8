// sk_internal.h -- declarations shared by the translation units of libflashsk.
// Not installed; the public interface is include/flashsk.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sk {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;  // threads per workgroup of every pass kernel

// Launch plan of one side's pass: rows per workgroup, column splits.
struct PassPlan {
  int rows_per_block;
  int row_blocks;
  int splits;          // column splits (partial slots per row for the balanced plan)
  int cols_per_split;
  int grid;            // balanced plan: workgroups (one resident wave of them)
  int stages;          // balanced plan: 128-column stages per row block
  int chunks;          // balanced plan: column chunks, each swept by the workgroups of 8 / chunks XCDs
  int tile;            // GEMM-tiled half-pass: workgroup tile (0: 256 x 256, 1: 128 x 128, 2: 128 x 256)
};

hipError_t launch_centroid(const void* x, int64_t n, const void* y, int64_t m, int dtype, int d,
                           double* centroid_part, float* shift, hipStream_t s);
// Exact per-coordinate shift of two bf16 clouds (see prep.hip): part holds
// kCentroidBlocks x 2 x d doubles of scratch.
hipError_t launch_bf16_shift(const void* x, int64_t n, const void* y, int64_t m, int d, double* part, float* shift,
                             hipStream_t s);
hipError_t launch_zero_u32(unsigned* p, int64_t count, hipStream_t s);
// Small problems (small.hip): whether the one-launch solve serves n, m, d, its
// grid, its scratch (tags: small_ws_bytes, 8-byte aligned) and a batch of
// iterations on it (cold: from zero potentials, which it writes when iters = 0).
bool small_fits(int64_t n, int64_t m, int64_t d, bool alternating);
int small_grid(int64_t n, int64_t m);
size_t small_ws_bytes(int64_t n, int64_t m);
hipError_t launch_small_solve(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                              const float* a, const float* b, double eps, int iters, bool averaged, float* f,
                              float* g, bool cold, void* tags, hipStream_t s);
// Small problems' transport applications (V: m x k, or n x k transposed) and
// barycentric gradient (grad: V, k, f unused) in one launch, no workspace.
bool small_aux_fits(int64_t n, int64_t m, int64_t d, int64_t k);
hipError_t launch_small_aux(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                            const float* a, const float* b, const float* f, const float* g, double eps,
                            int transpose, bool grad, const float* V, int64_t k, float* out, hipStream_t s);
hipError_t launch_cost(const float* a, const float* f, int64_t n, const float* b, const float* g,
                       int64_t m, double* cost, hipStream_t s);

constexpr int kCentroidBlocks = 256;

}  // namespace sk
