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

// Stages the cnt points of one side with their log2-unit biases
// k (pot_j + eps ln w_j) into LDS, (d + 1) floats per point padded to DQ
// float4s (the bias last). The potentials are the words of generation gen
// in `pot`: a thread requests its words kBatch at a time and polls the stale
// ones again until they turn.
constexpr int kBatch = 4;
template <int DQ>
__device__ void stage_side(float4* st, const void* pts, int dtype, int d, const float* w,
                           const unsigned long long* pot, unsigned gen, int64_t cnt, float eps, float k,
                           unsigned* timeout) {
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
      if (j < cnt) {
        float c[4 * DQ];
#pragma unroll
        for (int q = 0; q < 4 * DQ; ++q) c[q] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4 * DQ - 1; ++q)
          if (q < d) c[q] = point_coord(pts, dtype, j * d + q);
        const float wj = w[j];
        // zero weight: the point adds nothing (its bias is -inf)
        c[4 * DQ - 1] =
            wj > 0.0f ? k * (__uint_as_float((unsigned)v[u]) + eps * kLn2 * __builtin_amdgcn_logf(wj)) : -INFINITY;
#pragma unroll
        for (int q = 0; q < DQ; ++q)
          st[j * DQ + q] = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
      }
    }
  }
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

__device__ __forceinline__ void online_merge(float mo, float so, float& mx, float& s) {
  const float mt = fmaxf(mx, mo);
  if (mt == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(mx - mt) + so * __builtin_amdgcn_exp2f(mo - mt);
  mx = mt;
}

// log2 sum_j 2^{t_ij} for the staged side against one point p (this lane's
// share: columns lane, lane + 64, ..., in two interleaved running sums to
// halve the dependent chain; combined over the wave).
template <int DQ>
__device__ float row_lse2(const float4* st, int64_t cnt, const float (&p)[4 * DQ - 1], float k, int lane) {
  float mx = -INFINITY, s = 0.0f, mx2 = -INFINITY, s2 = 0.0f;
  int64_t j = lane;
  for (; j + kGroup < cnt; j += 2 * kGroup) {
    online_add(score2<DQ>(st, j, p, k), mx, s);
    online_add(score2<DQ>(st, j + kGroup, p, k), mx2, s2);
  }
  if (j < cnt) online_add(score2<DQ>(st, j, p, k), mx, s);
  online_merge(mx2, s2, mx, s);
#pragma unroll
  for (int o = 1; o < kGroup; o <<= 1) {
    const float mo = __shfl_xor(mx, o, kGroup);
    const float so = __shfl_xor(s, o, kGroup);
    online_merge(mo, so, mx, s);
  }
  return mx + __builtin_amdgcn_logf(s);
}

// Update of row i of one side against the staged other side: -eps ln2 LSE2.
template <int DQ>
__device__ float update_row(const float4* st, int64_t cnt_cols, const void* pts, int dtype, int d, int64_t i,
                            int64_t cnt_rows, float eps, float k) {
  const int lane = threadIdx.x & (kGroup - 1);
  float p[4 * DQ - 1];
#pragma unroll
  for (int q = 0; q < 4 * DQ - 1; ++q) p[q] = (i < cnt_rows && q < d) ? point_coord(pts, dtype, i * d + q) : 0.0f;
  return -eps * kLn2 * row_lse2<DQ>(st, cnt_cols, p, k, lane);
}

// tags: four buffers of cap words (side x generation parity: F0, F1, G0, G1),
// all stale on entry, then the timeout flag (zero on entry).
template <int DQ>
__global__ __launch_bounds__(kSmallThreads) void k_small_solve(const void* x, const void* y, int dtype, int64_t n,
                                                               int64_t m, int d, const float* a, const float* b,
                                                               float eps, int iters, int averaged, float* f,
                                                               float* g, unsigned long long* tags, int64_t cap) {
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
  // generation 0: the starting pair, published by the owners of the rows
  float fv[kMaxChunks], gv[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int64_t i = row_of(c);
    fv[c] = i < n ? f[i] : 0.0f;
    gv[c] = i < m ? g[i] : 0.0f;
    if (writer && i < n) put_tagged(F[0] + i, fv[c], 0u);
    if (writer && i < m) put_tagged(G[0] + i, gv[c], 0u);
  }
  for (int it = 0; it < iters; ++it) {
    const unsigned gen = (unsigned)it, nxt = gen + 1;
    float fn[kMaxChunks], gn[kMaxChunks];
    stage_side<DQ>(st, y, dtype, d, b, G[gen & 1], gen, m, eps, k, timeout);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      fn[c] = chunk_live(c, n) ? update_row<DQ>(st, m, x, dtype, d, row_of(c), n, eps, k) : 0.0f;
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
    stage_side<DQ>(st, x, dtype, d, a, F[gf & 1], gf, n, eps, k, timeout);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      gn[c] = chunk_live(c, m) ? update_row<DQ>(st, n, y, dtype, d, row_of(c), m, eps, k) : 0.0f;
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

template <int DQ>
hipError_t launch_dq(const void* x, const void* y, int dtype, int64_t n, int64_t m, int d, const float* a,
                     const float* b, float eps, int iters, int averaged, float* f, float* g,
                     unsigned long long* tags, int64_t cap, int nwg, hipStream_t s) {
  void* args[] = {(void*)&x, (void*)&y, (void*)&dtype, (void*)&n, (void*)&m, (void*)&d, (void*)&a, (void*)&b,
                  (void*)&eps, (void*)&iters, (void*)&averaged, (void*)&f, (void*)&g, (void*)&tags, (void*)&cap};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_small_solve<DQ>), dim3(nwg),
                                    dim3(kSmallThreads), args, 0, s);
}

}  // namespace

bool small_fits(int64_t n, int64_t m, int64_t d) {
  if (d < 1 || d > 7) return false;  // up to two float4 a staged point (more would spill)
  const int64_t dq = (d + 1 + 3) / 4;
  const int64_t big = n > m ? n : m;
  // a side stages in LDS; a workgroup owns at most kMaxChunks rows of each side per wave
  return big * dq * 4 <= kStageFloats && big <= kMaxSide && n * m <= (int64_t(1) << 21);
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
                              float* g, void* tags_ws, hipStream_t s) {
  if (iters <= 0) return hipSuccess;
  const int64_t cap = n > m ? n : m;
  unsigned long long* tags = static_cast<unsigned long long*>(tags_ws);
  const int64_t blocks = (4 * cap + 255) / 256;
  k_small_reset<<<(int)(blocks < 64 ? blocks : 64), 256, 0, s>>>(tags, 4 * cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nwg = small_grid(n, m);
  const int dq = (int)((d + 1 + 3) / 4);
  const float ef = (float)eps;
  const int di = (int)d, av = averaged ? 1 : 0;
  switch (dq) {
    case 1: return launch_dq<1>(x, y, dtype, n, m, di, a, b, ef, iters, av, f, g, tags, cap, nwg, s);
    case 2: return launch_dq<2>(x, y, dtype, n, m, di, a, b, ef, iters, av, f, g, tags, cap, nwg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sk
