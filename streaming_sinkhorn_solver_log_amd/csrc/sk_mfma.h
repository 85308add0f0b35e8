// sk_mfma.h -- types and arguments of the matrix-core passes (library-internal).
#pragma once

#include "sk_internal.h"

namespace sk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One half-pass on the matrix cores. Records are NKB * 32 bytes per point; a
// bias record is two bf16x8 (half 0: the three bf16 parts of h~ = h / c2).
struct MfmaPassArgs {
  const void* rows;        // nr row-form records
  const void* cols;        // nc column-form records
  const bf16x8* bias_col;  // nc bias records of the columns
  const float* alpha;      // nr squared norms of the rows
  const float* lw;         // nr natural-log row weights
  float* pot;              // nr potentials, updated in place
  bf16x8* bias_out;        // bias chunk of row 0 for the next pass of the other side
  int bias_stride;         // bf16x8 units between consecutive rows' bias chunks
  float* Lout;             // nr log2-sum-exp values of this pass
  const float* Lin;        // nr log2-sum-exp values of this side's previous pass (shifted sweep)
  const float* hval_in;    // nr biases (log2 units) this side had before this pass
  float* hval_out;         // nr biases (log2 units) after this pass
  const float* dmax_in;    // per-block maxima of the columns' bias change since this side's previous pass
  int n_dmax_in;
  float* dmax_out;         // one entry per row block: max bias change of its rows
  unsigned* exact_count;   // workgroups that fell back to the exact sweep (may be null)
  float2* part;            // split partials (M, S) in log2 units: [split][nr]
  unsigned* counters;      // one per row block, zero on entry and exit
  int nr, nc;
  int splits, cols_per_split;  // GEMM-tiled pass: column splits
  int row_blocks, stages;      // register-resident pass: balanced split of row blocks x stages
  int chunks;                  // register-resident pass: column chunks (PassPlan::chunks)
  // Exponent of a pair in log2 units = escale * (acc - M). float32 points have
  // c2 folded into their row records (escale = 1, biases in log2 units); bf16
  // points keep exact records (escale = c2, biases stored divided by c2).
  float escale, bias_scale, neg_eps_ln2, log2e_over_eps;
  int symmetric;
  // Column biases as float32 in accumulator units (h~ = h * bias_scale,
  // masked like the bias records), padded like them; the bf16-point kernels
  // with a separate bias record add them as the first MFMA's accumulator
  // input instead of multiplying the bias record. hout: the rows' values for
  // the other side's next pass (may be null).
  const float* hcol;
  float* hout;
  // Nonzero: every shifted row block takes the exact recomputation, as if its
  // shifted sum had fallen below the floor (a test hook; normally 0).
  int force_exact;
};

// Weighted sums over the columns of the half-pass scores, on the matrix cores:
//   apply: out_i = sum_j 2^{hrow_i + e acc_ij} V_j                 (kv = k)
//   grad:  out_i = 2 a_i (x_i - sum_j 2^{e acc_ij} q_j / sum_j 2^{e acc_ij})  (kv = d)
// acc_ij = score + column bias, as in a half-pass with no row shift. Values
// come as fragments (pack_values); a launch covers value blocks
// [z * NOB, z * NOB + NOB) for z = blockIdx.z.
struct PvArgs {
  const void* rows;        // nr row-form records
  const void* cols;        // nc column-form records (padded)
  const bf16x8* bias_col;  // nc bias records of the columns (padded)
  const bf16x8* vfrag;     // value fragments of the columns (padded)
  const unsigned* vmax;    // half-precision form: kv column maxima (float bits), else null
  int nobt;                // value blocks (of 32) per tile in vfrag
  int kv;                  // value width; out is nr x kv, row-major
  float* out;
  const float* hrow;       // apply: nr row biases (log2 units)
  const float* wrow;       // grad: nr row weights
  const void* xrow;        // grad: nr x kv row points as stored
  int xbf16;               // grad: row points are bf16
  const float* shift;      // grad: centering shift of float32 points (or null)
  int grad;
  float* part;             // split partials: (mu, S) pairs then values, per (chunk, split)
  int pcw;                 // value partials per (slot, row) (set by launch_pv)
  int nr, nc, row_blocks, nchunks;
  int splits, cols_per_split;
  float escale;
  // Weighted application (wide kernel, apply mode): each plan entry is
  // multiplied by q_ij = acc'_ij + qoff_i, acc'_ij the product of row i's
  // tangent records (wq arrays of nr records, wrec_stride bf16x8 apart) with
  // column j's records. Null wrec: unweighted.
  const bf16x8* wrec;
  int64_t wrec_stride;
  const float* qoff;       // nr per-row offsets of q (or null)
};

struct MfmaPrepSide {
  const void* pts;   // n x d as stored
  const float* w;    // weights
  const float* pot;  // starting potential (null: zeros)
  float* pot_zero;   // written with zeros if non-null
  bf16x8* row_rec;   // n records (row form)
  bf16x8* col_rec;   // n records (column form)
  float* alpha;
  float* lw;
  bf16x8* bias;      // n bias records of the starting potential (separate layout)
  bf16x8* bias_alt;  // the second bias buffer (its padding is initialized too)
  float* hval;       // n biases (log2 units) of the starting potential
  int64_t n;
  float* hacc = nullptr;      // padded float biases in accumulator units (or null)
  float* hacc_alt = nullptr;  // the second float bias buffer (its padding is initialized too)
};

int mfma_nkb(int dtype, int d);  // K blocks per record, 0 if the resident kernel does not serve d
// Merged layout: the column bias chunk lives in the last (free) 16-byte chunk
// of each column record instead of a separate bias record, saving one MFMA
// and one LDS block per tile. Possible when the data leaves that chunk free.
bool mfma_merged(int dtype, int d, int nkb);
int mfma_rb(int nkb);
// Points per side including the masked padding columns (records, bias buffers).
int64_t mfma_padded_count(int64_t n);
// share > 1: the pass shares its launch with share - 1 others (launch_lse_mfma_pair).
PassPlan plan_mfma_pass(int64_t nr, int64_t nc, int nkb, bool merged, bool scaled, int share = 1);
hipError_t launch_lse_mfma(const MfmaPassArgs& a, int nkb, bool shifted, bool scaled, bool merged,
                           const PassPlan& pl, hipStream_t s);
// Two independent half-passes of the same kernel in one launch (pl1 null: one).
hipError_t launch_lse_mfma_pair(const MfmaPassArgs& a0, const PassPlan& pl0, const MfmaPassArgs& a1,
                                const PassPlan* pl1, int nkb, bool shifted, bool scaled, bool merged,
                                hipStream_t s);
// interleave: records for the GEMM-tiled kernels (K block by K block).
hipError_t launch_prep_mfma(const MfmaPrepSide& xs, const MfmaPrepSide& ys, int dtype, int d,
                            int nkb, bool merged, bool center, double* centroid_part, float* shift,
                            unsigned* counters, int n_counters, float log2e_over_eps,
                            float c2, bool interleave, hipStream_t s);
// escale and bias_scale of a storage type (see MfmaPassArgs).
inline float mfma_escale(int dtype, float c2) { return dtype == 1 ? c2 : 1.0f; }
inline float mfma_bias_scale(int dtype, float c2) { return dtype == 1 ? 1.0f / c2 : 1.0f; }

}  // namespace sk
