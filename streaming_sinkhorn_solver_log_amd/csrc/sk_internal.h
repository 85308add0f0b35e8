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

// One half-pass of the log-domain update, seen from the side whose potential is
// being recomputed ("rows"); the other side is "cols". With
//   s_ij = h_j + c2 * (p_i . q_j)              (log2 units, c2 = 2 log2(e) / eps)
//   L_i  = log2 sum_j 2^{s_ij}
//   new_i = -eps ln2 L_i + alpha_i             (alpha_i = |p_i|^2)
// the row potential becomes new_i (alternating) or (pot_i + new_i)/2 (averaged),
// and the pass writes this side's column bias for the next pass of the other
// side: hout_i = log2(e) (lw_i + (pot_i - alpha_i)/eps), lw_i = ln(weight_i).
struct PassArgs {
  const void* rows;     // row points, kernel-specific packed layout
  const void* cols;     // column points, same layout
  const float* hcol;    // nc column biases (log2 units)
  const float* alpha;   // nr squared norms of the row points
  const float* lw;      // nr natural-log weights of the rows
  float* pot;           // nr potentials, updated in place
  float* hout;          // nr biases this side contributes as columns next time
  float* Lout;          // nr log2-sum-exp values (may be null)
  float2* part;         // split partials (M, S): [split][nr]
  unsigned* counters;   // one per row block, zero on entry, zero on exit
  int nr, nc;
  int splits, cols_per_split;
  float c2;             // 2 log2(e) / eps
  float neg_eps_ln2;    // -eps ln 2
  float log2e_over_eps; // log2(e) / eps
  int symmetric;        // averaged update
};

// Barycentric gradient pass: out_i = 2 a_i (p_i - sum_j pi_ij q_j / sum_j pi_ij),
// pi_ij = 2^{s_ij}. Partials per split: (M, S, O[0..d)).
struct GradArgs {
  const void* rows;
  const void* cols;
  const float* hcol;
  const float* wrow;    // nr row weights a_i (linear, as stored)
  float* out;           // nr x d, row-major
  float* part;          // [split][nr][2 + d]
  unsigned* counters;
  int nr, nc, d;
  int splits, cols_per_split;
  float c2;
};

// Transport application: out_i = sum_j 2^{r_i + h_j + c2 p_i.q_j} V_j, V is nc x k.
// Partials per split: k floats.
struct ApplyArgs {
  const void* rows;
  const void* cols;
  const float* hrow;    // nr row biases r_i (log2 units)
  const float* hcol;    // nc column biases
  const float* V;       // nc x k
  float* out;           // nr x k
  float* part;          // [split][nr][k]
  unsigned* counters;
  int nr, nc, k;
  int splits, cols_per_split;
  float c2;
};

// Point layout produced by the prep kernels and consumed by a pass kernel.
enum class Layout : int {
  F32Padded = 0,  // float32, centered, row stride DP = round_up(d, 4), zero padded
};

// Launch plan of one side's pass: rows per workgroup, column splits.
struct PassPlan {
  int rows_per_block;
  int row_blocks;
  int splits;          // column splits (partial slots per row for the balanced plan)
  int cols_per_split;
  int grid;            // balanced plan: workgroups (one resident wave of them)
  int stages;          // balanced plan: 128-column stages per row block
  int chunks;          // balanced plan: column chunks, each swept by the workgroups of 8 / chunks XCDs
};

PassPlan plan_valu_pass(int64_t nr, int64_t nc, int d);
int valu_dclass(int d);  // template dimension of the VALU kernels serving d (d <= 64)
int valu_dp(int d);      // row stride of their packed float32 points

// Launchers (return hipGetLastError() after the launch).
hipError_t launch_lse_valu(const PassArgs& a, int d, const PassPlan& pl, hipStream_t s);
hipError_t launch_grad_valu(const GradArgs& a, const PassPlan& pl, hipStream_t s);
hipError_t launch_apply_valu(const ApplyArgs& a, int d, const PassPlan& pl, hipStream_t s);

// Prep: centroid of both clouds (shift t), packed centered points, squared
// norms, log-weights and biases from the starting potentials; zeroes counters.
struct PrepSide {
  const void* pts;       // n x d as stored
  const float* w;        // weights
  const float* pot;      // starting potential (null: zeros)
  float* pot_init;       // if non-null, written with zeros (cold start)
  float* packed;         // output points (layout)
  float* alpha;          // output |p|^2
  float* lw;             // output ln w
  float* h;              // output bias log2(e)(ln w + (pot - alpha)/eps)
  int64_t n;
};
hipError_t launch_prep(const PrepSide& xs, const PrepSide& ys, int dtype, int d, int dp,
                       bool center, double* centroid_part, float* shift, unsigned* counters,
                       int n_counters, float log2e_over_eps, hipStream_t s);
hipError_t launch_centroid(const void* x, int64_t n, const void* y, int64_t m, int dtype, int d,
                           double* centroid_part, float* shift, hipStream_t s);
hipError_t launch_zero_u32(unsigned* p, int64_t count, hipStream_t s);
hipError_t launch_cost(const float* a, const float* f, int64_t n, const float* b, const float* g,
                       int64_t m, double* cost, hipStream_t s);

constexpr int kCentroidBlocks = 64;

}  // namespace sk
