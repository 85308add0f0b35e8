// small.hip -- fixed-budget solve of small problems in one launch.
//
// For n, m of a few thousand points and small d, a half-pass has so little
// work (n m pairs, about a microsecond of the GPU) that the launch and the
// memory round trips around it (row records in, partials out, their merge)
// set its time. Here one cooperative launch runs a whole batch of
// iterations: each workgroup owns rows of both sides (one wave per row), and
// for each half-pass stages the other side's points and biases in LDS. The
// update itself is the log-domain one (Fused & Furious: Sinkhorn Triton
// Kernels, §II.C, the log-sum-exp form of the potentials' update):
//   f_i = -eps ln sum_j b_j exp((g_j - C_ij) / eps),   C_ij = |x_i - y_j|^2,
// in log2 units, t_ij = k (g_j + eps ln b_j) - k C_ij with k = log2(e) / eps,
// summed with an online maximum; C_ij is formed from direct differences (no
// centering needed). Alternating: f from g, then g from the new f; averaged:
// both from the previous pair, each new potential the mean of old and update.
//
// There is no grid barrier: every potential is published as one 64-bit word
// {value, generation} with an agent-coherent store, in one of two buffers per
// side (by generation parity), and a reader polls the words it stages until
// they carry the generation it needs. A workgroup can thus run at most one
// generation ahead of the slowest one, which the two buffers cover. A poll
// gives up after a bounded wait (setting a flag, so that every wave ends),
// and a launch that gave up poisons its potentials with NaN.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "flashsk.h"
#include "sk_internal.h"
#include "sk_sync.h"

namespace sk {
namespace {

constexpr int kSmallThreads = 256;
constexpr int kGroup = 64;                              // lanes that share one row: a wave
constexpr int kRowsPerPass = kSmallThreads / kGroup;    // rows a workgroup works on at a time
constexpr int kMaxChunks = 4;                           // row chunks of one side per workgroup
constexpr int kMaxSide = 256 * kRowsPerPass * kMaxChunks;  // points of a side (4096)
constexpr int kStageFloats = 16384;                     // LDS staging: 64 KB of floats
constexpr unsigned kSpinLimit = 1u << 22;               // polls before giving up
constexpr unsigned kStale = 0xFFFFFFFFu;                // generation of a word not written in this launch
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void put_tagged(unsigned long long* p, float v, unsigned gen) {
  const unsigned long long w = (unsigned long long)__float_as_uint(v) | ((unsigned long long)gen << 32);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long peek(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float point_coord(const void* p, int dtype, int64_t idx) {
  if (dtype == SK_BF16) return __uint_as_float((unsigned)static_cast<const unsigned short*>(p)[idx] << 16);
  return static_cast<const float*>(p)[idx];
}

// Waits until the potentials of generation gen of one side are published:
// a thread requests its words kBatch at a time (j = j0 + u * 256) and polls
// the stale ones again until they turn; then `put(j, pot_j)` for each.
constexpr int kBatch = 4;
template <typename Put>
__device__ __forceinline__ void poll_side(const unsigned long long* pot, unsigned gen, int64_t cnt,
                                          unsigned* timeout, Put put) {
  for (int64_t j0 = threadIdx.x; j0 < cnt; j0 += (int64_t)kBatch * kSmallThreads) {
    unsigned long long v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j = j0 + (int64_t)u * kSmallThreads;
      v[u] = j < cnt ? peek(pot + j) : ((unsigned long long)gen << 32);
    }
    unsigned polls = 0;
    bool ready = false;
    while (!ready) {
      ready = true;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) ready = ready && (unsigned)(v[u] >> 32) == gen;
      if (ready) break;
      if (++polls > kSpinLimit) {
        __hip_atomic_store(timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if ((unsigned)(v[u] >> 32) != gen) v[u] = peek(pot + j0 + (int64_t)u * kSmallThreads);  // live: j < cnt
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j = j0 + (int64_t)u * kSmallThreads;
      if (j < cnt) put(j, __uint_as_float((unsigned)v[u]));
    }
  }
}

// log2 w (k eps ln w = log2 w, since k = 1 / (eps ln 2)); a zero weight gives
// -inf, so that its point adds nothing.
__device__ __forceinline__ float log2_weight(float w) {
  return w > 0.0f ? __builtin_amdgcn_logf(w) : -INFINITY;
}

// Point j staged in slot `slot`: (d + 1) floats padded to DQ float4s, the
// coordinates (zero-padded) then, last, the log2-unit bias k pot_j + log2 w_j.
template <int DQ>
__device__ __forceinline__ void put_point(float4* st, int64_t slot, const void* pts, int dtype, int d, int64_t j,
                                          float bias) {
  float c[4 * DQ];
#pragma unroll
  for (int q = 0; q < 4 * DQ; ++q) c[q] = 0.0f;
#pragma unroll
  for (int q = 0; q < 4 * DQ - 1; ++q)
    if (q < d) c[q] = point_coord(pts, dtype, j * d + q);
  c[4 * DQ - 1] = bias;
#pragma unroll
  for (int q = 0; q < DQ; ++q) st[slot * DQ + q] = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
}

// log2 sum_j 2^{t_ij} for the staged side against one point p (this lane's
// share: columns lane, lane + 64, ...; combined over the wave).
template <int DQ>
__device__ __forceinline__ float score2(const float4* st, int64_t j, const float (&p)[4 * DQ - 1], float k) {
  float c = 0.0f, h = 0.0f;
#pragma unroll
  for (int q = 0; q < DQ; ++q) {
    const float4 v = st[j * DQ + q];
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (4 * q + u == 4 * DQ - 1) {
        h = vv[u];
      } else {
        const float df = p[4 * q + u] - vv[u];  // padded coordinates are zero on both sides
        c = fmaf(df, df, c);
      }
    }
  }
  return fmaf(-k, c, h);
}

// Online maximum with one exp2: the smaller of (t, max) is scaled down (a
// zero-weight point, t = -inf, adds nothing).
__device__ __forceinline__ void online_add(float t, float& mx, float& s) {
  const bool up = t > mx;
  const float e = t > -INFINITY ? __builtin_amdgcn_exp2f(up ? mx - t : t - mx) : 0.0f;
  s = up ? fmaf(s, e, 1.0f) : s + e;
  mx = up ? t : mx;
}

// One value of lane l ^ x within each row of 16 lanes (x = 1, 2) or the lane
// mirrored within the row's halves / the row (DPP quad_perm, row_half_mirror,
// row_mirror: every source lane lies in the row, so no lane reads an
// undefined value).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i within each 8 lanes: joins the two quads
constexpr int kDppMirror = 0x140;      // lane 15 - i within each 16 lanes: joins the two halves

// Wave-wide maximum and sum: combined within each row of 16 lanes by DPP
// (after the four steps every lane of a row holds the row's value), then
// over the four rows from lanes 0, 16, 32 and 48 (uniform results).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// log2 sum_j 2^{t_ij} for the staged side against one point p (this lane's
// share: columns lane, lane + 64, ..., in two interleaved running sums to
// halve the dependent chain). Over the wave: the maximum M of the lanes'
// running maxima, then the sum of their sums scaled to M.
template <int DQ>
__device__ float row_lse2(const float4* st, int64_t cnt, const float (&p)[4 * DQ - 1], float k, int lane) {
  float mx = -INFINITY, s = 0.0f, mx2 = -INFINITY, s2 = 0.0f;
  int64_t j = lane;
  // four columns a trip (their LDS reads go out together)
  for (; j + 3 * kGroup < cnt; j += 4 * kGroup) {
    const float t0 = score2<DQ>(st, j, p, k), t1 = score2<DQ>(st, j + kGroup, p, k);
    const float t2 = score2<DQ>(st, j + 2 * kGroup, p, k), t3 = score2<DQ>(st, j + 3 * kGroup, p, k);
    online_add(t0, mx, s);
    online_add(t1, mx2, s2);
    online_add(t2, mx, s);
    online_add(t3, mx2, s2);
  }
  for (; j < cnt; j += kGroup) online_add(score2<DQ>(st, j, p, k), mx, s);
  const float M = wave_max(fmaxf(mx, mx2));
  // a running sum whose maximum is -inf is zero (and M = -inf leaves every one so)
  const float sl = (mx > -INFINITY ? s * __builtin_amdgcn_exp2f(mx - M) : 0.0f) +
                   (mx2 > -INFINITY ? s2 * __builtin_amdgcn_exp2f(mx2 - M) : 0.0f);
  return M + __builtin_amdgcn_logf(wave_sum(sl));
}

// Update of row i (point p) of one side against the staged other side:
// -eps ln2 LSE2.
template <int DQ>
__device__ __forceinline__ float update_row(const float4* st, int64_t cnt_cols, const float (&p)[4 * DQ - 1],
                                            float eps, float k) {
  const int lane = threadIdx.x & (kGroup - 1);
  return -eps * kLn2 * row_lse2<DQ>(st, cnt_cols, p, k, lane);
}

// Coordinates of row i of a side (zeros past d, and for rows past cnt): from
// the staged points when the side is resident in LDS, else from memory.
template <int DQ>
__device__ __forceinline__ void row_point(float (&p)[4 * DQ - 1], const float4* rows, const void* pts, int dtype,
                                          int d, int64_t i, int64_t cnt) {
#pragma unroll
  for (int q = 0; q < 4 * DQ - 1; ++q) p[q] = 0.0f;
  if (i >= cnt) return;
  if (rows) {
#pragma unroll
    for (int qq = 0; qq < DQ; ++qq) {
      const float4 v = rows[i * DQ + qq];
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (4 * qq + u < 4 * DQ - 1) p[4 * qq + u] = vv[u];
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4 * DQ - 1; ++q)
      if (q < d) p[q] = point_coord(pts, dtype, i * d + q);
  }
}

// tags: four buffers of cap words (side x generation parity: F0, F1, G0, G1),
// all stale on entry, then the timeout flag (zero on entry).
// RES: both sides' points stay in LDS for the whole launch (float4s of X at
// [0, n DQ), of Y at [n DQ, (n + m) DQ), then the log2 weights of X and of
// Y), and a half-pass only writes the biases of the side it reads. Otherwise
// each half-pass stages the side it reads, coordinates included, at the start
// of the area, and rows take their coordinates from memory.
template <int DQ, bool RES>
__global__ __launch_bounds__(kSmallThreads) void k_small_solve(const void* x, const void* y, int dtype, int64_t n,
                                                               int64_t m, int d, const float* a, const float* b,
                                                               float eps, int iters, int averaged, int cold,
                                                               float* f, float* g, unsigned long long* tags,
                                                               int64_t cap) {
  __shared__ float4 st[kStageFloats / 4];
  const int wg = blockIdx.x, nwg = gridDim.x;
  const float k = 1.4426950408889634f / eps;
  unsigned long long* F[2] = {tags, tags + cap};
  unsigned long long* G[2] = {tags + 2 * cap, tags + 3 * cap};
  unsigned* timeout = reinterpret_cast<unsigned*>(tags + 4 * cap);
  const bool writer = (threadIdx.x & (kGroup - 1)) == 0;
  const int r_in = threadIdx.x / kGroup;
  auto row_of = [&](int c) { return ((int64_t)wg + (int64_t)c * nwg) * kRowsPerPass + r_in; };
  auto chunk_live = [&](int c, int64_t cnt) { return ((int64_t)wg + (int64_t)c * nwg) * kRowsPerPass < cnt; };
  float4* const stx = st;
  float4* const sty = RES ? st + n * DQ : st;
  float* const lwx = reinterpret_cast<float*>(st + (n + m) * DQ);  // RES only
  float* const lwy = lwx + n;
  if constexpr (RES) {
    for (int64_t j = threadIdx.x; j < n; j += kSmallThreads) {
      put_point<DQ>(stx, j, x, dtype, d, j, 0.0f);
      lwx[j] = log2_weight(a[j]);
    }
    for (int64_t j = threadIdx.x; j < m; j += kSmallThreads) {
      put_point<DQ>(sty, j, y, dtype, d, j, 0.0f);
      lwy[j] = log2_weight(b[j]);
    }
    __syncthreads();
  }
  // Biases of generation gen of one side into its staged points (RES), or the
  // side's points with their biases into the staging area.
  auto stage = [&](float4* sts, const float* lws, const void* pts, const float* w, const unsigned long long* pot,
                   unsigned gen, int64_t cnt) {
    if constexpr (RES) {
      float* sf = reinterpret_cast<float*>(sts);
      poll_side(pot, gen, cnt, timeout,
                [&](int64_t j, float v) { sf[(j * DQ + DQ - 1) * 4 + 3] = fmaf(k, v, lws[j]); });
    } else {
      poll_side(pot, gen, cnt, timeout, [&](int64_t j, float v) {
        put_point<DQ>(sts, j, pts, dtype, d, j, fmaf(k, v, log2_weight(w[j])));
      });
    }
  };
  // generation 0: the starting pair (zeros for a cold start), published by
  // the owners of the rows
  float fv[kMaxChunks], gv[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int64_t i = row_of(c);
    fv[c] = i < n && !cold ? f[i] : 0.0f;
    gv[c] = i < m && !cold ? g[i] : 0.0f;
    if (writer && i < n) put_tagged(F[0] + i, fv[c], 0u);
    if (writer && i < m) put_tagged(G[0] + i, gv[c], 0u);
  }
  for (int it = 0; it < iters; ++it) {
    const unsigned gen = (unsigned)it, nxt = gen + 1;
    float fn[kMaxChunks], gn[kMaxChunks];
    stage(sty, lwy, y, b, G[gen & 1], gen, m);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      fn[c] = 0.0f;
      if (chunk_live(c, n)) {
        float p[4 * DQ - 1];
        row_point<DQ>(p, RES ? stx : nullptr, x, dtype, d, row_of(c), n);
        fn[c] = update_row<DQ>(sty, m, p, eps, k);
      }
    }
    if (averaged) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) fn[c] = 0.5f * (fv[c] + fn[c]);
    } else {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (writer && row_of(c) < n) put_tagged(F[nxt & 1] + row_of(c), fn[c], nxt);
    }
    __syncthreads();  // the staging area is read before it is refilled
    // alternating: the new f (generation gen + 1); averaged: the previous one
    const unsigned gf = averaged ? gen : nxt;
    stage(stx, lwx, x, a, F[gf & 1], gf, n);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      gn[c] = 0.0f;
      if (chunk_live(c, m)) {
        float p[4 * DQ - 1];
        row_point<DQ>(p, RES ? sty : nullptr, y, dtype, d, row_of(c), m);
        gn[c] = update_row<DQ>(stx, n, p, eps, k);
      }
    }
    if (averaged) {
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        gn[c] = 0.5f * (gv[c] + gn[c]);
        if (writer && row_of(c) < n) put_tagged(F[nxt & 1] + row_of(c), fn[c], nxt);
      }
    }
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (writer && row_of(c) < m) put_tagged(G[nxt & 1] + row_of(c), gn[c], nxt);
      fv[c] = fn[c];
      gv[c] = gn[c];
    }
    __syncthreads();
  }
  const bool gave_up = __hip_atomic_load(timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int64_t i = row_of(c);
    if (writer && i < n) f[i] = gave_up ? NAN : fv[c];
    if (writer && i < m) g[i] = gave_up ? NAN : gv[c];
  }
}

__global__ __launch_bounds__(256) void k_small_reset(unsigned long long* tags, int64_t words) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < words; q += (int64_t)gridDim.x * 256)
    tags[q] = (unsigned long long)kStale << 32;
  if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<unsigned*>(tags + words) = 0u;
}

template <int DQ, bool RES>
hipError_t launch_dq(const void* x, const void* y, int dtype, int64_t n, int64_t m, int d, const float* a,
                     const float* b, float eps, int iters, int averaged, int cold, float* f, float* g,
                     unsigned long long* tags, int64_t cap, int nwg, hipStream_t s) {
  void* args[] = {(void*)&x,     (void*)&y,        (void*)&dtype, (void*)&n, (void*)&m,
                  (void*)&d,     (void*)&a,        (void*)&b,     (void*)&eps, (void*)&iters,
                  (void*)&averaged, (void*)&cold, (void*)&f,     (void*)&g, (void*)&tags, (void*)&cap};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_small_solve<DQ, RES>), dim3(nwg),
                                    dim3(kSmallThreads), args, 0, s);
}

// Transport applications and the barycentric gradient of small problems,
// in one launch with no traffic between workgroups: one wave per output row
// i, the column side streamed through LDS kAuxCols points at a time (with
// their values), in two sweeps: the row's maximum score M = max_j t_ij, then
// S = sum_j 2^{t_ij - M} and T = sum_j 2^{t_ij - M} v_j (t_ij as in the
// solve: k pot_j + log2 w_j - k C_ij). With the plan entries
// P_ij = a_i b_j exp((f_i + g_j - C_ij) / eps) (FlashSinkhorn replication
// review, Summary: applications of the plan without forming it, and the
// gradient as its barycentric projection):
//   apply (KQ > 0, v_j = V_j, kv <= 4 KQ values):
//     out_i = 2^{k pot_i + log2 w_i + M} T
//   gradient (KQ = 0, v_j = the column point y_j, pot_i unused):
//     out_i = 2 w_i (p_i - T / S)
// A single chunk is staged once for both sweeps.
constexpr int kAuxCols = 1024;  // LDS: up to 1024 x (2 + 4) float4 = 96 KB

template <int DQ, int KQ>
__global__ __launch_bounds__(kSmallThreads) void k_small_aux(const void* rows, const void* cols, int dtype,
                                                             int64_t nr, int64_t nc, int d, const float* wr,
                                                             const float* wc, const float* pr, const float* pc,
                                                             float eps, const float* V, int kv, float* out) {
  constexpr int NV = KQ > 0 ? 4 * KQ : 4 * DQ - 1;  // accumulated values per row
  __shared__ float4 pts[kAuxCols * DQ];
  __shared__ float4 vals[KQ > 0 ? kAuxCols * KQ : 1];
  const float k = 1.4426950408889634f / eps;
  const int lane = threadIdx.x & (kGroup - 1);
  const int64_t i = (int64_t)blockIdx.x * kRowsPerPass + threadIdx.x / kGroup;
  float p[4 * DQ - 1];
  row_point<DQ>(p, nullptr, rows, dtype, d, i, nr);  // zeros for a row past nr (it stores nothing)
  const int64_t nchunks = (nc + kAuxCols - 1) / kAuxCols;
  // Stages columns [c0, c0 + cnt): each thread's (up to kPer) columns are all
  // loaded into registers first, so that their loads are in flight together,
  // then written to LDS.
  constexpr int kPer = kAuxCols / kSmallThreads;
  auto stage = [&](int64_t c0, bool with_values) {
    const int64_t cnt = nc - c0 < kAuxCols ? nc - c0 : kAuxCols;
    float cb[kPer][4 * DQ], wb[kPer];
    float vb[kPer][KQ > 0 ? 4 * KQ : 1];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int64_t j = threadIdx.x + (int64_t)u * kSmallThreads;
#pragma unroll
      for (int q = 0; q < 4 * DQ; ++q) cb[u][q] = 0.0f;
      wb[u] = 0.0f;
      if constexpr (KQ > 0) {
#pragma unroll
        for (int c = 0; c < 4 * KQ; ++c) vb[u][c] = 0.0f;
      }
      if (j < cnt) {
#pragma unroll
        for (int q = 0; q < 4 * DQ - 1; ++q)
          if (q < d) cb[u][q] = point_coord(cols, dtype, (c0 + j) * d + q);
        cb[u][4 * DQ - 1] = pc[c0 + j];  // the potential; the bias once the loads are in
        wb[u] = wc[c0 + j];
        if constexpr (KQ > 0) {
          if (with_values) {
            const float* vj = V + (c0 + j) * kv;
#pragma unroll
            for (int c = 0; c < 4 * KQ; ++c)
              if (c < kv) vb[u][c] = vj[c];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int64_t j = threadIdx.x + (int64_t)u * kSmallThreads;
      if (j < cnt) {
        cb[u][4 * DQ - 1] = fmaf(k, cb[u][4 * DQ - 1], log2_weight(wb[u]));
#pragma unroll
        for (int q = 0; q < DQ; ++q)
          pts[j * DQ + q] = make_float4(cb[u][4 * q], cb[u][4 * q + 1], cb[u][4 * q + 2], cb[u][4 * q + 3]);
        if constexpr (KQ > 0) {
          if (with_values) {
#pragma unroll
            for (int q = 0; q < KQ; ++q)
              vals[j * KQ + q] = make_float4(vb[u][4 * q], vb[u][4 * q + 1], vb[u][4 * q + 2], vb[u][4 * q + 3]);
          }
        }
      }
    }
  };
  // sweep 1: the row's maximum score
  float mx = -INFINITY;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t c0 = ch * kAuxCols;
    const int64_t cnt = nc - c0 < kAuxCols ? nc - c0 : kAuxCols;
    if (ch > 0) __syncthreads();  // the previous chunk is read before it is replaced
    stage(c0, nchunks == 1);
    __syncthreads();
#pragma unroll 4
    for (int64_t j = lane; j < cnt; j += kGroup) mx = fmaxf(mx, score2<DQ>(pts, j, p, k));
  }
  const float M = wave_max(mx);
  // sweep 2: the shifted sums
  float S = 0.0f, T[NV];
#pragma unroll
  for (int c = 0; c < NV; ++c) T[c] = 0.0f;
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t c0 = ch * kAuxCols;
    const int64_t cnt = nc - c0 < kAuxCols ? nc - c0 : kAuxCols;
    if (nchunks > 1) {
      __syncthreads();
      stage(c0, true);
      __syncthreads();
    }
#pragma unroll 4
    for (int64_t j = lane; j < cnt; j += kGroup) {
      const float t = score2<DQ>(pts, j, p, k);
      const float e = t > -INFINITY ? __builtin_amdgcn_exp2f(t - M) : 0.0f;
      S += e;
      if constexpr (KQ > 0) {
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
          const float4 v = vals[j * KQ + q];
          T[4 * q] = fmaf(e, v.x, T[4 * q]);
          T[4 * q + 1] = fmaf(e, v.y, T[4 * q + 1]);
          T[4 * q + 2] = fmaf(e, v.z, T[4 * q + 2]);
          T[4 * q + 3] = fmaf(e, v.w, T[4 * q + 3]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < DQ; ++q) {
          const float4 v = pts[j * DQ + q];
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (4 * q + u < NV) T[4 * q + u] = fmaf(e, vv[u], T[4 * q + u]);
        }
      }
    }
  }
  float o = 0.0f;  // lane c: value c of the row
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const float tc = wave_sum(T[c]);
    if (lane == c) o = tc;
  }
  if (i >= nr) return;
  if constexpr (KQ > 0) {
    const float scale = __builtin_amdgcn_exp2f(fmaf(k, pr[i], log2_weight(wr[i])) + M);
    if (lane < kv) out[i * kv + lane] = o * scale;
  } else {
    const float St = wave_sum(S);
    float pl = 0.0f;  // lane c: coordinate c of the row's point
#pragma unroll
    for (int c = 0; c < NV; ++c)
      if (lane == c) pl = p[c];
    if (lane < d) out[i * d + lane] = 2.0f * wr[i] * (pl - o / St);
  }
}

template <int DQ, int KQ>
hipError_t launch_aux(const void* rows, const void* cols, int dtype, int64_t nr, int64_t nc, int d,
                      const float* wr, const float* wc, const float* pr, const float* pc, float eps, const float* V,
                      int kv, float* out, hipStream_t s) {
  const int64_t grid = (nr + kRowsPerPass - 1) / kRowsPerPass;
  k_small_aux<DQ, KQ><<<(unsigned)grid, kSmallThreads, 0, s>>>(rows, cols, dtype, nr, nc, d, wr, wc, pr, pc, eps,
                                                               V, kv, out);
  return hipGetLastError();
}

}  // namespace

bool small_fits(int64_t n, int64_t m, int64_t d, bool alternating) {
  if (d < 1 || d > 7) return false;  // up to two float4 a staged point (more would spill)
  const int64_t dq = (d + 1 + 3) / 4;
  const int64_t big = n > m ? n : m;
  // a side stages in LDS; a workgroup owns at most kMaxChunks rows of each side
  // per wave. Pair counts: where the launch is still faster than the streaming
  // passes (the averaged streaming schedule runs both half-passes in one launch,
  // so it wins from fewer pairs on).
  const int64_t max_pairs = alternating ? (int64_t(1) << 22) : (int64_t(1) << 21);
  return big * dq * 4 <= kStageFloats && big <= kMaxSide && n * m <= max_pairs;
}

size_t small_ws_bytes(int64_t n, int64_t m) {
  const int64_t cap = n > m ? n : m;
  return (size_t)(4 * cap) * sizeof(unsigned long long) + sizeof(unsigned long long);
}

int small_grid(int64_t n, int64_t m) {
  const int64_t big = n > m ? n : m;
  int64_t w = (big + kRowsPerPass - 1) / kRowsPerPass;
  if (w > 256) w = 256;
  return (int)(w < 1 ? 1 : w);
}

hipError_t launch_small_solve(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                              const float* a, const float* b, double eps, int iters, bool averaged, float* f,
                              float* g, bool cold, void* tags_ws, hipStream_t s) {
  if (iters <= 0) {
    if (!cold) return hipSuccess;
    hipError_t e = launch_zero_u32(reinterpret_cast<unsigned*>(f), n, s);
    return e != hipSuccess ? e : launch_zero_u32(reinterpret_cast<unsigned*>(g), m, s);
  }
  const int64_t cap = n > m ? n : m;
  unsigned long long* tags = static_cast<unsigned long long*>(tags_ws);
  const int64_t blocks = (4 * cap + 255) / 256;
  k_small_reset<<<(int)(blocks < 64 ? blocks : 64), 256, 0, s>>>(tags, 4 * cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nwg = small_grid(n, m);
  const int dq = (int)((d + 1 + 3) / 4);
  const float ef = (float)eps;
  const int di = (int)d, av = averaged ? 1 : 0, cd = cold ? 1 : 0;
  // both sides resident in LDS when their points and log2 weights fit
  const bool res = (n + m) * (4 * dq + 1) <= kStageFloats;
  switch (dq * 2 + (res ? 1 : 0)) {
    case 2: return launch_dq<1, false>(x, y, dtype, n, m, di, a, b, ef, iters, av, cd, f, g, tags, cap, nwg, s);
    case 3: return launch_dq<1, true>(x, y, dtype, n, m, di, a, b, ef, iters, av, cd, f, g, tags, cap, nwg, s);
    case 4: return launch_dq<2, false>(x, y, dtype, n, m, di, a, b, ef, iters, av, cd, f, g, tags, cap, nwg, s);
    case 5: return launch_dq<2, true>(x, y, dtype, n, m, di, a, b, ef, iters, av, cd, f, g, tags, cap, nwg, s);
    default: return hipErrorInvalidValue;
  }
}

bool small_aux_fits(int64_t n, int64_t m, int64_t d, int64_t k) {
  // one wave per output row; the row's k <= 16 sums stay in registers
  return d >= 1 && d <= 7 && k >= 1 && k <= 16 && n * m <= (int64_t(1) << 22);
}

hipError_t launch_small_aux(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                            const float* a, const float* b, const float* f, const float* g, double eps,
                            int transpose, bool grad, const float* V, int64_t k, float* out, hipStream_t s) {
  const int dq = (int)((d + 1 + 3) / 4);
  const int di = (int)d, kv = grad ? 0 : (int)k;
  const float ef = (float)eps;
  if (grad) {
    if (n == 0) return hipSuccess;
    if (dq == 1) return launch_aux<1, 0>(x, y, dtype, n, m, di, a, b, nullptr, g, ef, nullptr, 0, out, s);
    if (dq == 2) return launch_aux<2, 0>(x, y, dtype, n, m, di, a, b, nullptr, g, ef, nullptr, 0, out, s);
    return hipErrorInvalidValue;
  }
  // rows: x with (f, a), columns y with (g, b); transposed, the other way round
  const void* rows = transpose ? y : x;
  const void* cols = transpose ? x : y;
  const int64_t nr = transpose ? m : n, nc = transpose ? n : m;
  const float* wr = transpose ? b : a;
  const float* wc = transpose ? a : b;
  const float* pr = transpose ? g : f;
  const float* pc = transpose ? f : g;
  if (nr == 0) return hipSuccess;
  const int kq = (kv + 3) / 4;
  switch (dq * 8 + kq) {
    case 9: return launch_aux<1, 1>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 10: return launch_aux<1, 2>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 11: return launch_aux<1, 3>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 12: return launch_aux<1, 4>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 17: return launch_aux<2, 1>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 18: return launch_aux<2, 2>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 19: return launch_aux<2, 3>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    case 20: return launch_aux<2, 4>(rows, cols, dtype, nr, nc, di, wr, wc, pr, pc, ef, V, kv, out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sk
