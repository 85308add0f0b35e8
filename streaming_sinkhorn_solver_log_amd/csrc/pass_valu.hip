// pass_valu.hip -- vector-ALU passes for small dimension (1 <= d <= 64; d > 16 is
// served by the padded classes 32 and 64).
//
// One half-pass of the stabilized log-domain Sinkhorn update, evaluated as a
// row-wise log-sum-exp of biased dot-product scores that are formed on the fly
// and never stored (FlashSinkhorn abstract; replication review, Summary: tiles
// are streamed, running row-wise LSE statistics stay on chip, only the updated
// potential is written back). Each lane owns one row and keeps c2 * p_i in
// registers; all lanes of a wave walk the same columns, so column points and
// biases are wave-uniform loads. The running maximum is refreshed once per
// chunk of columns (online max/sum-exp), in base 2.
//
// When a row's columns are split over several workgroups, each writes its
// partial (max, sum); the last workgroup of a row block to finish (counted
// with a device-scope atomic) combines the partials in split order, so the
// result does not depend on which workgroup finishes last.
#include "sk_internal.h"
#include "sk_sync.h"

#include <math.h>

namespace sk {
namespace {

// Columns per online-max refresh: the chunk's column points are wave-uniform
// (scalar) registers, so the chunk shrinks as d grows.
template <int D>
constexpr int chunk_for() { return D <= 4 ? 8 : (D <= 8 ? 4 : (D <= 16 ? 2 : 1)); }
constexpr int kChunkMax = 8;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }


__device__ __forceinline__ void finish_row(const PassArgs& p, int i, float M, float S) {
  const float L = M + fast_log2(S);
  const float al = p.alpha[i];
  float v = fmaf(p.neg_eps_ln2, L, al);
  if (p.symmetric) v = 0.5f * (p.pot[i] + v);
  p.pot[i] = v;
  p.hout[i] = fmaf(kLog2e, p.lw[i], (v - al) * p.log2e_over_eps);
  if (p.Lout) p.Lout[i] = L;
}

template <int D, int DP>
__device__ __forceinline__ void load_col(const float* __restrict__ cols, int j, float (&q)[D]) {
  const float4* c4 = reinterpret_cast<const float4*>(cols + (int64_t)j * DP);
#pragma unroll
  for (int v = 0; v < DP / 4; ++v) {
    const float4 t = c4[v];
    if (4 * v + 0 < D) q[4 * v + 0] = t.x;
    if (4 * v + 1 < D) q[4 * v + 1] = t.y;
    if (4 * v + 2 < D) q[4 * v + 2] = t.z;
    if (4 * v + 3 < D) q[4 * v + 3] = t.w;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_lse_valu(const PassArgs p) {
  constexpr int DP = (D + 3) & ~3;
  constexpr int kChunk = chunk_for<D>();
  const float* __restrict__ rows = static_cast<const float*>(p.rows);
  const float* __restrict__ cols = static_cast<const float*>(p.cols);
  const float* __restrict__ hcol = p.hcol;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const int sp = blockIdx.y;
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);

  float px[D];
#pragma unroll
  for (int k = 0; k < D; ++k) px[k] = (i < p.nr) ? p.c2 * rows[(int64_t)i * DP + k] : 0.0f;
  float M = -INFINITY, S = 0.0f;

  for (int j = j0; j < j1; j += kChunk) {
    // Loads of the whole chunk are issued together; past the end of the range the
    // last column is reloaded and its bias replaced by -inf (a zero term).
    float t[kChunk];
    float yv[kChunk][D];
    float hv[kChunk];
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int jj = __builtin_amdgcn_readfirstlane(min(j + q, j1 - 1));
      load_col<D, DP>(cols, jj, yv[q]);
      hv[q] = (j + q < j1) ? hcol[jj] : -INFINITY;
    }
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      float acc = hv[q];
#pragma unroll
      for (int k = 0; k < D; ++k) acc = fmaf(px[k], yv[q][k], acc);
      t[q] = acc;
    }
    float mx = t[0];
#pragma unroll
    for (int q = 1; q < kChunk; ++q) mx = fmaxf(mx, t[q]);
    const float Mn = fmaxf(M, mx);
    const float Ms = (Mn == -INFINITY) ? 0.0f : Mn;  // all terms so far are zero
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < kChunk; ++q) s += fast_exp2(t[q] - Ms);
    S = fmaf(S, fast_exp2(M - Ms), s);
    M = Mn;
  }

  if (p.splits == 1) {
    if (i < p.nr) finish_row(p, i, M, S);
    return;
  }
  if (i < p.nr) store_coherent(&p.part[(int64_t)sp * p.nr + i], make_float2(M, S));
  if (!arrive_last(p.counters + blockIdx.x, p.splits)) return;
  if (i < p.nr) {
    float Mt = -INFINITY;
    for (int s2 = 0; s2 < p.splits; ++s2) Mt = fmaxf(Mt, load_coherent(&p.part[(int64_t)s2 * p.nr + i].x));
    const float Ms = (Mt == -INFINITY) ? 0.0f : Mt;
    float St = 0.0f;
    for (int s2 = 0; s2 < p.splits; ++s2) {
      const float Mp = load_coherent(&p.part[(int64_t)s2 * p.nr + i].x);
      const float Sp = load_coherent(&p.part[(int64_t)s2 * p.nr + i].y);
      St = fmaf(Sp, fast_exp2(Mp - Ms), St);
    }
    finish_row(p, i, Mt, St);
  }
  if (threadIdx.x == 0) atomicExch(p.counters + blockIdx.x, 0u);
}

// Barycentric projection: online softmax over columns with a running weighted
// sum of the column points (the "attention output" with value = the points).
template <int D>
__global__ __launch_bounds__(kThreads) void k_grad_valu(const GradArgs p) {
  constexpr int DP = (D + 3) & ~3;
  constexpr int kChunk = chunk_for<D>();
  const float* __restrict__ rows = static_cast<const float*>(p.rows);
  const float* __restrict__ cols = static_cast<const float*>(p.cols);
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const int sp = blockIdx.y;
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);

  float px[D], O[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    px[k] = (i < p.nr) ? p.c2 * rows[(int64_t)i * DP + k] : 0.0f;
    O[k] = 0.0f;
  }
  float M = -INFINITY, S = 0.0f;
  for (int j = j0; j < j1; j += kChunk) {
    float t[kChunk];
    float yv[kChunk][D];
    float hv[kChunk];
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const int jj = __builtin_amdgcn_readfirstlane(min(j + q, j1 - 1));
      load_col<D, DP>(cols, jj, yv[q]);
      hv[q] = (j + q < j1) ? p.hcol[jj] : -INFINITY;
    }
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      float acc = hv[q];
#pragma unroll
      for (int k = 0; k < D; ++k) acc = fmaf(px[k], yv[q][k], acc);
      t[q] = acc;
    }
    float mx = t[0];
#pragma unroll
    for (int q = 1; q < kChunk; ++q) mx = fmaxf(mx, t[q]);
    const float Mn = fmaxf(M, mx);
    const float Ms = (Mn == -INFINITY) ? 0.0f : Mn;
    const float sc = fast_exp2(M - Ms);
    S *= sc;
#pragma unroll
    for (int k = 0; k < D; ++k) O[k] *= sc;
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const float e = fast_exp2(t[q] - Ms);
      S += e;
#pragma unroll
      for (int k = 0; k < D; ++k) O[k] = fmaf(e, yv[q][k], O[k]);
    }
    M = Mn;
  }

  auto finish = [&](float Sv, const float* Ov) {
    const float inv = 1.0f / Sv;
    const float tw = 2.0f * p.wrow[i];
#pragma unroll
    for (int k = 0; k < D; ++k)
      if (k < p.d) p.out[(int64_t)i * p.d + k] = tw * (rows[(int64_t)i * DP + k] - Ov[k] * inv);
  };
  if (p.splits == 1) {
    if (i < p.nr) finish(S, O);
    return;
  }
  constexpr int R = 2 + D;
  if (i < p.nr) {
    float* rec = p.part + ((int64_t)sp * p.nr + i) * R;
    store_coherent(rec, M);
    store_coherent(rec + 1, S);
#pragma unroll
    for (int k = 0; k < D; ++k) store_coherent(rec + 2 + k, O[k]);
  }
  if (!arrive_last(p.counters + blockIdx.x, p.splits)) return;
  if (i < p.nr) {
    float Mt = -INFINITY;
    for (int s2 = 0; s2 < p.splits; ++s2)
      Mt = fmaxf(Mt, load_coherent(p.part + ((int64_t)s2 * p.nr + i) * R));
    const float Ms = (Mt == -INFINITY) ? 0.0f : Mt;
    float St = 0.0f, Ot[D];
#pragma unroll
    for (int k = 0; k < D; ++k) Ot[k] = 0.0f;
    for (int s2 = 0; s2 < p.splits; ++s2) {
      const float* rec = p.part + ((int64_t)s2 * p.nr + i) * R;
      const float sc = fast_exp2(load_coherent(rec) - Ms);
      St = fmaf(load_coherent(rec + 1), sc, St);
#pragma unroll
      for (int k = 0; k < D; ++k) Ot[k] = fmaf(load_coherent(rec + 2 + k), sc, Ot[k]);
    }
    finish(St, Ot);
  }
  if (threadIdx.x == 0) atomicExch(p.counters + blockIdx.x, 0u);
}

// P V with P_ij = 2^{r_i + h_j + c2 p_i.q_j}; V rows are wave-uniform loads.
template <int D, int K>
__global__ __launch_bounds__(kThreads) void k_apply_valu(const ApplyArgs p) {
  constexpr int DP = (D + 3) & ~3;
  const float* __restrict__ rows = static_cast<const float*>(p.rows);
  const float* __restrict__ cols = static_cast<const float*>(p.cols);
  const float* __restrict__ V = p.V;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const int sp = blockIdx.y;
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);

  float px[D], acc[K];
#pragma unroll
  for (int k = 0; k < D; ++k) px[k] = (i < p.nr) ? p.c2 * rows[(int64_t)i * DP + k] : 0.0f;
#pragma unroll
  for (int c = 0; c < K; ++c) acc[c] = 0.0f;
  const float r = (i < p.nr) ? p.hrow[i] : -INFINITY;
  for (int j = j0; j < j1; ++j) {
    const int jj = __builtin_amdgcn_readfirstlane(j);
    float yv[D];
    load_col<D, DP>(cols, jj, yv);
    float e = p.hcol[jj] + r;
#pragma unroll
    for (int k = 0; k < D; ++k) e = fmaf(px[k], yv[k], e);
    const float w = fast_exp2(e);
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const float vv = (c < p.k) ? V[(int64_t)jj * p.k + c] : 0.0f;
      acc[c] = fmaf(w, vv, acc[c]);
    }
  }
  if (p.splits == 1) {
    if (i < p.nr) {
#pragma unroll
      for (int c = 0; c < K; ++c)
        if (c < p.k) p.out[(int64_t)i * p.k + c] = acc[c];
    }
    return;
  }
  if (i < p.nr) {
#pragma unroll
    for (int c = 0; c < K; ++c)
      if (c < p.k) store_coherent(p.part + ((int64_t)sp * p.nr + i) * p.k + c, acc[c]);
  }
  if (!arrive_last(p.counters + blockIdx.x, p.splits)) return;
  if (i < p.nr) {
    for (int c = 0; c < p.k; ++c) {
      float s = 0.0f;
      for (int s2 = 0; s2 < p.splits; ++s2) s += load_coherent(p.part + ((int64_t)s2 * p.nr + i) * p.k + c);
      p.out[(int64_t)i * p.k + c] = s;
    }
  }
  if (threadIdx.x == 0) atomicExch(p.counters + blockIdx.x, 0u);
}

template <template <int> class Fn, typename... A>
hipError_t dispatch_d(int d, A&&... args) {
  switch (d) {
#define SK_CASE(DD) case DD: return Fn<DD>::run(args...);
    SK_CASE(1) SK_CASE(2) SK_CASE(3) SK_CASE(4) SK_CASE(5) SK_CASE(6) SK_CASE(7) SK_CASE(8)
    SK_CASE(9) SK_CASE(10) SK_CASE(11) SK_CASE(12) SK_CASE(13) SK_CASE(14) SK_CASE(15) SK_CASE(16)
#undef SK_CASE
    default:
      if (d <= 32) return Fn<32>::run(args...);
      if (d <= 64) return Fn<64>::run(args...);
      return hipErrorInvalidValue;
  }
}

template <int D>
struct LseRun {
  static hipError_t run(const PassArgs& a, const PassPlan& pl, hipStream_t s) {
    k_lse_valu<D><<<dim3(pl.row_blocks, pl.splits), kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
};
template <int D>
struct GradRun {
  static hipError_t run(const GradArgs& a, const PassPlan& pl, hipStream_t s) {
    k_grad_valu<D><<<dim3(pl.row_blocks, pl.splits), kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
};
template <int D>
struct ApplyRun {
  static hipError_t run(const ApplyArgs& a, const PassPlan& pl, hipStream_t s) {
    dim3 grid(pl.row_blocks, pl.splits);
    if (a.k <= 4) k_apply_valu<D, 4><<<grid, kThreads, 0, s>>>(a);
    else if (a.k <= 16) k_apply_valu<D, 16><<<grid, kThreads, 0, s>>>(a);
    else if (a.k <= 32) k_apply_valu<D, 32><<<grid, kThreads, 0, s>>>(a);
    else k_apply_valu<D, 64><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
};

}  // namespace

int valu_dclass(int d) { return d <= 16 ? d : (d <= 32 ? 32 : 64); }
int valu_dp(int d) { return (valu_dclass(d) + 3) & ~3; }

PassPlan plan_valu_pass(int64_t nr, int64_t nc, int d) {
  (void)d;
  PassPlan pl{};
  pl.rows_per_block = kThreads;
  pl.row_blocks = (int)((nr + kThreads - 1) / kThreads);
  // Aim for about 2048 workgroups (8 waves per SIMD) and at least 512 columns per split.
  const int64_t target = 2048;
  int64_t splits = (target + pl.row_blocks - 1) / pl.row_blocks;
  const int64_t max_splits = nc / 512 > 1 ? nc / 512 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  pl.cols_per_split = (int)((nc + splits - 1) / splits);
  pl.cols_per_split = (pl.cols_per_split + kChunkMax - 1) / kChunkMax * kChunkMax;
  pl.splits = (int)((nc + pl.cols_per_split - 1) / pl.cols_per_split);
  return pl;
}

hipError_t launch_lse_valu(const PassArgs& a, int d, const PassPlan& pl, hipStream_t s) {
  return dispatch_d<LseRun>(d, a, pl, s);
}
hipError_t launch_grad_valu(const GradArgs& a, const PassPlan& pl, hipStream_t s) {
  return dispatch_d<GradRun>(a.d, a, pl, s);
}
hipError_t launch_apply_valu(const ApplyArgs& a, int d, const PassPlan& pl, hipStream_t s) {
  return dispatch_d<ApplyRun>(d, a, pl, s);
}

}  // namespace sk
