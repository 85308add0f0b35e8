// sk_gemm.h -- GEMM-tiled half-pass and transport application / gradient
// kernels (library-internal).
#pragma once

#include "sk_mfma.h"

namespace sk {

// Column splits for `units` independent row units (row blocks, or row blocks x
// value chunks) so that whole rounds of `resident` workgroups are filled;
// writes the columns per split (a multiple of unit_cols).
int64_t round_filling_splits(int64_t units, int64_t nc, int64_t unit_cols, int64_t max_splits,
                             int64_t resident, int64_t& cols_per_split);
// GEMM-tiled half-pass for wide records (any NKB that is a multiple of 4).
// The workgroup tile is 256 x 256 unless the environment variable
// FLASHSK_GEMM_TILE names 128x128 or 128x256 (read at each plan; the plan
// records it in PassPlan::tile, which the launch follows).
int gemm_nkb(int dtype, int d);
int gemm_tile_choice();
PassPlan plan_gemm_pass(int64_t nr, int64_t nc);
hipError_t launch_lse_gemm(const MfmaPassArgs& a, int nkb, bool shifted, bool scaled, const PassPlan& pl,
                           hipStream_t s);
// Transport application / gradient kernels. pv_parts: parts of the plan
// entries (pp) and of the values (vp) for a storage type and operation, and
// the form: half (a kernel that has it, unless precise with bf16 points) =
// float16 parts, the values scaled per column; else bf16 parts.
void pv_parts(int dtype, bool grad, bool half_kernel, bool precise, int& pp, int& vp, bool& half);
int pv_nob(bool gemm, int nobt, int vp);  // value blocks per launch chunk
PassPlan plan_pv(bool gemm, int64_t nr, int64_t nc, int nkb, int nob, int vp, int nchunks, bool half);
hipError_t launch_pv(const PvArgs& a, bool gemm, int nkb, int nob, int pp, int vp, bool half,
                     const PassPlan& pl, hipStream_t s);
// Tangent records of n rows (T n x d float32) for the weighted application:
// one record array (float32 points) or two (bf16 points, part_stride bf16x8
// apart), GEMM-tiled order; qoff (or null) = T . shift per row.
hipError_t launch_pack_tangent(const float* T, bool bf16pts, int64_t n, int d, int nkb, const float* shift,
                               bf16x8* out, int64_t part_stride, float* qoff, hipStream_t s);
// Value blocks per chunk of the wide kernel (the weighted application always
// runs on it): 4 NOBW, NOBW <= 4, and <= 2 in the weighted mode (its
// registers would spill at 4).
inline int pv_wide_nob(int nobt, int vp, bool weighted) {
  (void)vp;
  const int w = nobt <= 4 ? 1 : (nobt <= 8 || weighted ? 2 : 4);
  return 4 * w;
}
// Value fragments of nv points (src nv x kv, float32 or bf16 bits) for vp parts;
// with vmax (kv words, kv <= 4096) the half-precision form, whose column
// maxima it writes there first.
hipError_t launch_pack_values(const void* src, bool src_bf16, int64_t nv, int kv, const float* shift,
                              int vp, int nobt, int64_t ntiles, unsigned* vmax, bf16x8* out, hipStream_t s);

}  // namespace sk
