// prep.hip -- once-per-call preparation and the final cost reduction.
//
// The cost decomposes as C_ij = alpha_i + beta_j - 2 p_i.q_j with alpha, beta the
// squared norms (FlashSinkhorn replication review, Summary and Weaknesses: the
// fused update needs a cost of the form alpha_i + beta_j - Q_i.K_j). The prep
// kernels compute, for each side, the packed points, the norms, the natural-log
// weights and the column biases of the starting potentials. Float clouds are
// first translated by the midpoint of their two centroids: C is invariant
// under a common translation, and smaller norms make the expansion better
// conditioned in float32.
#include "sk_internal.h"
#include "sk_check.h"

#include <math.h>

namespace sk {
namespace {

__device__ inline float load_point(const void* pts, int dtype, int64_t idx) {
  if (dtype == 0) return static_cast<const float*>(pts)[idx];
  const unsigned short bits = static_cast<const unsigned short*>(pts)[idx];
  return __uint_as_float(static_cast<unsigned>(bits) << 16);
}

// Partial coordinate sums (float64) of both clouds: part[b][0..d) for x, part[b][d..2d) for y.
// Block b sums a contiguous range of rows. For d <= 256 the block reads the
// range as a flat, coalesced stream: thread t < T (T = the largest multiple of
// d not above 256) owns coordinate t % d and every (T / d)-th row; the T
// per-thread sums are then added per coordinate in a fixed order. Wider
// points: block (b, c) covers coordinates [256 c, 256 c + 256), a thread one
// coordinate of every row of the range (coalesced along the coordinates).
// Either way each thread keeps four running sums, so that its loads are in
// flight together.
__global__ __launch_bounds__(256) void k_centroid_partial(const void* x, int64_t n, const void* y,
                                                           int64_t m, int dtype, int d,
                                                           double* part) {
  __shared__ double acc[256];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  for (int side = 0; side < 2; ++side) {
    const void* pts = side ? y : x;
    const int64_t cnt = side ? m : n;
    const int64_t per = (cnt + gridDim.x - 1) / gridDim.x;
    const int64_t r0 = b * per, r1 = min(cnt, r0 + per);
    double* out = part + ((int64_t)b * 2 + side) * d;
    if (d <= 256) {
      const int T = (256 / d) * d;
      const int step = T / d;  // rows advanced per sweep of the block
      double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
      if (t < T) {
        const int k = t % d;
        int64_t r = r0 + t / d;
        for (; r + 3 * step < r1; r += 4 * step) {
          s0 += load_point(pts, dtype, r * d + k);
          s1 += load_point(pts, dtype, (r + step) * d + k);
          s2 += load_point(pts, dtype, (r + 2 * step) * d + k);
          s3 += load_point(pts, dtype, (r + 3 * step) * d + k);
        }
        for (; r < r1; r += step) s0 += load_point(pts, dtype, r * d + k);
      }
      acc[t] = (s0 + s1) + (s2 + s3);
      __syncthreads();
      if (t < d) {
        double tot = 0.0;
        for (int q = t; q < T; q += d) tot += acc[q];
        out[t] = tot;
      }
      __syncthreads();
    } else {
      const int k = blockIdx.y * 256 + t;
      if (k < d) {
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
        int64_t r = r0;
        for (; r + 3 < r1; r += 4) {
          s0 += load_point(pts, dtype, r * d + k);
          s1 += load_point(pts, dtype, (r + 1) * d + k);
          s2 += load_point(pts, dtype, (r + 2) * d + k);
          s3 += load_point(pts, dtype, (r + 3) * d + k);
        }
        for (; r < r1; ++r) s0 += load_point(pts, dtype, r * d + k);
        out[k] = (s0 + s1) + (s2 + s3);
      }
    }
  }
}

// shift_k = (mean_x + mean_y)_k / 2: a wave per coordinate, lane l summing the
// partials of blocks l, l + 64, ... in order, then the lanes in a fixed tree.
__global__ __launch_bounds__(256) void k_centroid_final(const double* part, int nb, int64_t n,
                                                        int64_t m, int d, float* shift) {
  const int k = (int)(((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64);
  const int lane = threadIdx.x & 63;
  if (k >= d) return;  // whole waves
  double sx = 0.0, sy = 0.0;
  for (int b = lane; b < nb; b += 64) {
    sx += part[((int64_t)b * 2 + 0) * d + k];
    sy += part[((int64_t)b * 2 + 1) * d + k];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sx += __shfl_xor(sx, o);
    sy += __shfl_xor(sy, o);
  }
  if (lane == 0) shift[k] = static_cast<float>(0.5 * (sx / (double)n + sy / (double)m));
}

__global__ __launch_bounds__(256) void k_zero_u32(unsigned* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

// Input screening for SK_CHECK_FINITE: ORs into *bad the bits of
// InputCheckBits that some element violates (one atomic per workgroup).
__device__ __forceinline__ bool finite_bits(unsigned u, unsigned expmask) { return (u & expmask) != expmask; }

__global__ __launch_bounds__(256) void k_check_inputs(const void* x, const void* y, int dtype, int64_t nx,
                                                      int64_t ny, const float* a, int64_t n, const float* b,
                                                      int64_t m, const float* f, const float* g,
                                                      unsigned* bad) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool pts = false, wts = false, apos = false, bpos = false, pot = false;
  for (int64_t i = t0; i < nx + ny; i += stride) {
    const void* src = i < nx ? x : y;
    const int64_t k = i < nx ? i : i - nx;
    if (dtype == 1) pts |= !finite_bits(static_cast<const unsigned short*>(src)[k], 0x7F80u);
    else pts |= !finite_bits(__float_as_uint(static_cast<const float*>(src)[k]), 0x7F800000u);
  }
  for (int64_t i = t0; i < n + m; i += stride) {
    const float w = i < n ? a[i] : b[i - n];
    // NaN fails both comparisons: !(w >= 0) catches it with the negatives
    wts |= !(w >= 0.0f) || !finite_bits(__float_as_uint(w), 0x7F800000u);
    if (i < n) apos |= w > 0.0f;
    else bpos |= w > 0.0f;
    if (f) {
      const float v = i < n ? f[i] : g[i - n];
      pot |= !finite_bits(__float_as_uint(v), 0x7F800000u);
    }
  }
  const unsigned bits = (__syncthreads_or(pts) ? kBadPoints : 0u) | (__syncthreads_or(wts) ? kBadWeights : 0u) |
                        (__syncthreads_or(apos) ? kPositiveA : 0u) | (__syncthreads_or(bpos) ? kPositiveB : 0u) |
                        (__syncthreads_or(pot) ? kBadPotentials : 0u);
  if (threadIdx.x == 0 && bits) atomicOr(bad, bits);
}

// cost = sum_i a_i f_i + sum_j b_j g_j in float64, one workgroup, fixed order.
__global__ __launch_bounds__(1024) void k_cost(const float* a, const float* f, int64_t n,
                                               const float* b, const float* g, int64_t m,
                                               double* cost) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += (double)a[i] * (double)f[i];
  for (int64_t j = threadIdx.x; j < m; j += blockDim.x) s += (double)b[j] * (double)g[j];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *cost = red[0];
}

// Exact shift of bf16 clouds. Translating bf16 points by their centroid would
// change their values (x - t is rarely a bf16 number), so the shift of
// coordinate k is taken where the difference stays exact: when every point of
// both clouds has the same sign in k, t_k is the largest multiple of U_k (the
// bf16 spacing at the largest |value|) not above the smallest |value|, with
// that sign. Then each x - t_k is a multiple of the spacing at x and smaller
// than |x|, so it has at most 8 significant bits: exactly a bf16 number. A
// coordinate whose values change sign keeps t_k = 0.

// Per-block minima and maxima of every coordinate over both clouds
// (mm[b][0..d) and mm[b][d..2d), floats), reduced by k_bf16_shift_final:
// each workgroup takes a contiguous range of rows, each thread a fixed
// coordinate of every rstep-th row (coalesced along the rows), combined
// through LDS.
__global__ __launch_bounds__(256) void k_bf16_shift_partial(const unsigned short* x, int64_t n,
                                                             const unsigned short* y, int64_t m, int d,
                                                             int rows_per_block, float* mm) {
  __shared__ float slo[256], shi[256];
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  float* out = mm + (int64_t)blockIdx.x * 2 * d;
  const int kt = d < 256 ? d : 256;  // coordinates per row sweep
  const int rstep = 256 / kt;        // rows per sweep
  const int k0 = threadIdx.x % kt, rr = threadIdx.x / kt;
  for (int kb = 0; kb < d; kb += kt) {
    const int k = kb + k0;
    float lo = INFINITY, hi = -INFINITY;
    if (rr < rstep && k < d) {
#pragma unroll 8
      for (int64_t r = r0 + rr; r < r0 + rows_per_block && r < n + m; r += rstep) {
        const unsigned short bits = r < n ? x[r * d + k] : y[(r - n) * d + k];
        const float v = __uint_as_float((unsigned)bits << 16);
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
    }
    slo[threadIdx.x] = lo;
    shi[threadIdx.x] = hi;
    __syncthreads();
    if (rr == 0 && k < d) {
      for (int q = 1; q < rstep; ++q) {
        lo = fminf(lo, slo[q * kt + k0]);
        hi = fmaxf(hi, shi[q * kt + k0]);
      }
      out[k] = lo;
      out[d + k] = hi;
    }
    __syncthreads();
  }
}

// The same for d a multiple of 8: each thread reads 8 coordinates of a row at
// once (16 bytes; rows of 8-coordinate groups are 16-byte aligned as the
// points are).
__global__ __launch_bounds__(256) void k_bf16_shift_partial8(const uint4* x, int64_t n, const uint4* y, int64_t m,
                                                              int d8, int rows_per_block, float* mm) {
  __shared__ float slo[8][256], shi[8][256];
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  float* out = mm + (int64_t)blockIdx.x * 16 * d8;
  const int gt = d8 < 256 ? d8 : 256;  // coordinate groups per row sweep
  const int rstep = 256 / gt;          // rows per sweep
  const int g0 = threadIdx.x % gt, rr = threadIdx.x / gt;
  for (int gb = 0; gb < d8; gb += gt) {
    const int g = gb + g0;
    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = INFINITY;
      hi[e] = -INFINITY;
    }
    if (rr < rstep && g < d8) {
#pragma unroll 4
      for (int64_t r = r0 + rr; r < r0 + rows_per_block && r < n + m; r += rstep) {
        const uint4 v = r < n ? x[r * d8 + g] : y[(r - n) * d8 + g];
        const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a0 = __uint_as_float(w[q] << 16), a1 = __uint_as_float(w[q] & 0xFFFF0000u);
          lo[2 * q] = fminf(lo[2 * q], a0);
          hi[2 * q] = fmaxf(hi[2 * q], a0);
          lo[2 * q + 1] = fminf(lo[2 * q + 1], a1);
          hi[2 * q + 1] = fmaxf(hi[2 * q + 1], a1);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      slo[e][threadIdx.x] = lo[e];
      shi[e][threadIdx.x] = hi[e];
    }
    __syncthreads();
    if (rr == 0 && g < d8) {
      for (int q = 1; q < rstep; ++q) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[e] = fminf(lo[e], slo[e][q * gt + g0]);
          hi[e] = fmaxf(hi[e], shi[e][q * gt + g0]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        out[8 * g + e] = lo[e];
        out[8 * d8 + 8 * g + e] = hi[e];
      }
    }
    __syncthreads();
  }
}

// The shift of each coordinate from the nb blocks' minima and maxima: a wave
// per coordinate (lanes over the blocks, then a shuffle tree).
__global__ __launch_bounds__(256) void k_bf16_shift_final(const float* mm, int nb, int d, float* shift) {
  const int k = (int)(((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64);
  const int lane = threadIdx.x & 63;
  if (k >= d) return;  // whole waves
  float lo = INFINITY, hi = -INFINITY;
  for (int b = lane; b < nb; b += 64) {
    lo = fminf(lo, mm[(int64_t)b * 2 * d + k]);
    hi = fmaxf(hi, mm[(int64_t)b * 2 * d + d + k]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if (lane != 0) return;
  float t = 0.0f;
  if (lo > 0.0f || hi < 0.0f) {
    const float small = lo > 0.0f ? lo : -hi, big = lo > 0.0f ? hi : -lo;
    int e = 0;
    frexpf(big, &e);                   // big = m 2^e, m in [0.5, 1)
    const float U = ldexpf(1.0f, e - 8);  // bf16 spacing in [2^(e-1), 2^e)
    t = floorf(small / U) * U;
    if (hi < 0.0f) t = -t;
  }
  shift[k] = t;
}

}  // namespace

hipError_t launch_bf16_shift(const void* x, int64_t n, const void* y, int64_t m, int d, double* part, float* shift,
                             hipStream_t s) {
  // per-block minima and maxima in the centroid scratch (kCentroidBlocks x 2 d
  // doubles hold kCentroidBlocks x 2 d floats)
  float* mm = reinterpret_cast<float*>(part);
  const int64_t total = n + m;
  const int rows = (int)((total + kCentroidBlocks - 1) / kCentroidBlocks);
  const int blocks = (int)((total + rows - 1) / rows);
  if (d % 8 == 0)
    k_bf16_shift_partial8<<<blocks, 256, 0, s>>>(static_cast<const uint4*>(x), n, static_cast<const uint4*>(y), m,
                                                 d / 8, rows, mm);
  else
    k_bf16_shift_partial<<<blocks, 256, 0, s>>>(static_cast<const unsigned short*>(x), n,
                                                static_cast<const unsigned short*>(y), m, d, rows, mm);
  k_bf16_shift_final<<<(d * 64 + 255) / 256, 256, 0, s>>>(mm, blocks, d, shift);
  return hipGetLastError();
}

hipError_t launch_centroid(const void* x, int64_t n, const void* y, int64_t m, int dtype, int d,
                           double* centroid_part, float* shift, hipStream_t s) {
  const dim3 grid(kCentroidBlocks, d > 256 ? (d + 255) / 256 : 1);
  k_centroid_partial<<<grid, 256, 0, s>>>(x, n, y, m, dtype, d, centroid_part);
  k_centroid_final<<<(d * 64 + 255) / 256, 256, 0, s>>>(centroid_part, kCentroidBlocks, n, m, d, shift);
  return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, int64_t count, hipStream_t s) {
  if (count > 0) k_zero_u32<<<(int)((count + 255) / 256), 256, 0, s>>>(p, count);
  return hipGetLastError();
}

hipError_t launch_cost(const float* a, const float* f, int64_t n, const float* b, const float* g,
                       int64_t m, double* cost, hipStream_t s) {
  k_cost<<<1, 1024, 0, s>>>(a, f, n, b, g, m, cost);
  return hipGetLastError();
}

hipError_t launch_check_inputs(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                               const float* a, const float* b, const float* f, const float* g,
                               unsigned* bad, hipStream_t s) {
  k_zero_u32<<<1, 256, 0, s>>>(bad, 1);
  k_check_inputs<<<1024, 256, 0, s>>>(x, y, dtype, n * d, m * d, a, n, b, m, f, g, bad);
  return hipGetLastError();
}

}  // namespace sk
