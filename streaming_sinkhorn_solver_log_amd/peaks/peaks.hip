// peaks.hip -- microbenchmarks of the gfx950 units the half-pass roofline is
// priced against: the transcendental rate (v_exp_f32), the non-packed fp32
// VALU rate (fma, add), the half-pass's own VALU mix (one exp2 and one add per
// score), whether exp2 and matrix-core work overlap, the bf16 and fp32 MFMA
// rates, and the read bandwidth of HBM, L2 and the MALL.
//
// Measurement tooling, not part of the library: built into libskpeaks.so and
// run by `bench.py --peaks`. Register-only kernels keep their operands opaque
// to the compiler with empty asm statements (no instruction is emitted), so
// the loops cannot be folded; every bandwidth kernel reads inside its buffer
// with grid-stride loops.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void opaque(T& v) {
  asm volatile("" : "+v"(v));
}

// 8 independent chains of v <- exp2(-v); v stays in [0.5, 1].
__global__ __launch_bounds__(kThreads) void k_exp(float* out, int iters) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.5f + 0.01f * (threadIdx.x % 7 + k);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_amdgcn_exp2f(-v[k]);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += v[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 8 independent chains of v <- v * a + b (a < 1: bounded).
__global__ __launch_bounds__(kThreads) void k_fma(float* out, int iters, float a, float b) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.1f * (threadIdx.x % 5 + k);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = fmaf(v[k], a, b);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += v[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 8 independent chains of v <- v + c.
__global__ __launch_bounds__(kThreads) void k_add(float* out, int iters, float c) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.1f * (threadIdx.x % 5 + k);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] += c;
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += v[k];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The half-pass VALU mix alone: per score one exp2 (after a multiply by e when
// SCALED) and one add into a running sum (16 scores per step, four sums).
template <bool SCALED>
__global__ __launch_bounds__(kThreads) void k_exp_add(float* out, int iters, float e) {
  float x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = -0.05f * (k + threadIdx.x % 3);
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  auto ex = [&](float v) { return __builtin_amdgcn_exp2f(SCALED ? v * e : v); };
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) opaque(x[k]);
#pragma unroll
    for (int k = 0; k < 16; k += 4) {
      s0 += ex(x[k]);
      s1 += ex(x[k + 1]);
      s2 += ex(x[k + 2]);
      s3 += ex(x[k + 3]);
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (s0 + s1) + (s2 + s3);
}

// bf16 MFMA: four independent 32x32x16 accumulators per wave.
__global__ __launch_bounds__(kThreads) void k_mfma_bf16(float* out, int iters) {
  bf16x8 A, B;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    A[e] = (__bf16)(1e-3f * (e + threadIdx.x % 5));
    B[e] = (__bf16)(1e-3f * (e + threadIdx.x % 3));
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
    opaque(A);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[q], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += acc[q][0] + acc[q][15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// fp32 MFMA: four independent 32x32x2 accumulators per wave.
__global__ __launch_bounds__(kThreads) void k_mfma_f32(float* out, int iters) {
  float A = 1e-3f * (threadIdx.x % 5), B = 1e-3f * (threadIdx.x % 3);
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
    opaque(A);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(A, B, acc[q], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += acc[q][0] + acc[q][15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The half-pass instruction mix with everything but the MFMAs and the VALU
// taken out: per step NMFMA chained bf16 MFMAs produce 1024 scores while the
// previous step's 1024 are folded as exp2(score) (times e first when SCALED)
// into four running sums -- the register-resident half-pass pattern. The
// occupancy hint keeps the accumulators in VGPRs, as in the half-pass kernel
// (accumulators in AGPRs would add one v_accvgpr_read per score).
template <int NMFMA, bool SCALED>
__global__ __launch_bounds__(kThreads, 2) void k_mfma_exp(float* out, int iters, float e) {
  bf16x8 A, B;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    A[k] = (__bf16)(-1e-3f * (k + 1));
    B[k] = (__bf16)(1e-3f * (k + threadIdx.x % 7));
  }
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  auto chain = [&]() {
    f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, f32x16{}, 0, 0, 0);
#pragma unroll
    for (int q = 1; q < NMFMA; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
    return acc;
  };
  auto fold = [&](const f32x16& acc) {
    auto ex = [&](float v) { return __builtin_amdgcn_exp2f(SCALED ? v * e : v); };
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      s0 += ex(acc[r]);
      s1 += ex(acc[r + 1]);
      s2 += ex(acc[r + 2]);
      s3 += ex(acc[r + 3]);
    }
  };
  f32x16 a0 = chain(), a1;
  for (int it = 0; it < iters; it += 2) {
    opaque(A);
    a1 = chain();
    fold(a0);
    opaque(A);
    a0 = chain();
    fold(a1);
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = (s0 + s1) + (s2 + s3);
}

// Streaming read bandwidth: the grid sums the float4s of the buffer once per
// pass (grid-stride, so each workgroup reads a 1/gridDim share of it).
__global__ __launch_bounds__(kThreads) void k_read(const f32x4* __restrict__ buf, int64_t count, int passes,
                                                  float* out) {
  f32x4 s = {};
  const int64_t G = (int64_t)gridDim.x * blockDim.x;
  for (int p = 0; p < passes; ++p) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * G < count; i += 4 * G) {  // four loads in flight per lane
      const f32x4 a = buf[i], b = buf[i + G], c = buf[i + 2 * G], d = buf[i + 3 * G];
      s += (a + b) + (c + d);
    }
    for (; i < count; i += G) s += buf[i];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// Cache-resident read bandwidth: every workgroup reads the whole buffer
// (count a power of two) `passes` times from its own rotated start, so each
// CU streams a working set larger than its L1 that every XCD's L2 holds.
__global__ __launch_bounds__(kThreads) void k_read_window(const f32x4* __restrict__ buf, int64_t count, int passes,
                                                         float* out) {
  f32x4 s = {};
  const int64_t mask = count - 1, start = ((int64_t)blockIdx.x * 4096) & mask;
  for (int p = 0; p < passes; ++p)
    for (int64_t i = threadIdx.x; i < count; i += 4 * blockDim.x) {  // indices masked: always in bounds
      const int64_t B = blockDim.x;
      const f32x4 a = buf[(start + i) & mask], b = buf[(start + i + B) & mask];
      const f32x4 c = buf[(start + i + 2 * B) & mask], d = buf[(start + i + 3 * B) & mask];
      s += (a + b) + (c + d);
    }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

int g_cus = 0;

hipError_t timed(hipEvent_t e0, hipEvent_t e1, float* ms, void (*launch)(void*), void* ctx) {
  launch(ctx);  // warm-up
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(e0)) != hipSuccess) return e;
  launch(ctx);
  if ((e = hipEventRecord(e1)) != hipSuccess) return e;
  if ((e = hipEventSynchronize(e1)) != hipSuccess) return e;
  return hipEventElapsedTime(ms, e0, e1);
}

struct Ctx {
  int which;
  int blocks;
  int iters;
  float* out;
  const f32x4* buf;
  int64_t count;
  int passes;
};

void launch_one(void* p) {
  const Ctx& c = *static_cast<const Ctx*>(p);
  switch (c.which) {
    case 0: k_exp<<<c.blocks, kThreads>>>(c.out, c.iters); break;
    case 1: k_fma<<<c.blocks, kThreads>>>(c.out, c.iters, 0.999f, 1e-4f); break;
    case 2: k_add<<<c.blocks, kThreads>>>(c.out, c.iters, 1e-7f); break;
    case 3: k_exp_add<false><<<c.blocks, kThreads>>>(c.out, c.iters, 1.0f); break;
    case 11: k_exp_add<true><<<c.blocks, kThreads>>>(c.out, c.iters, 1.0f); break;
    case 4: k_mfma_bf16<<<c.blocks, kThreads>>>(c.out, c.iters); break;
    case 5: k_mfma_f32<<<c.blocks, kThreads>>>(c.out, c.iters); break;
    case 6: k_mfma_exp<2, false><<<c.blocks, kThreads>>>(c.out, c.iters, 1.0f); break;
    case 10: k_mfma_exp<4, true><<<c.blocks, kThreads>>>(c.out, c.iters, 1.0f); break;
    case 8: k_read_window<<<c.blocks, kThreads>>>(c.buf, c.count, c.passes, c.out); break;
    default: k_read<<<c.blocks, kThreads>>>(c.buf, c.count, c.passes, c.out); break;
  }
}

}  // namespace

extern "C" {

// Benchmark `which`: 0 exp2, 1 fma, 2 add, 3 exp2 + add, 4 bf16 MFMA, 5 fp32 MFMA,
// 6 two chained bf16 MFMAs per 1024 scores overlapped with exp2 + add (the
// float32-record half-pass mix at d <= 5), 7 HBM read, 8 L2-resident read,
// 9 MALL-resident read, 10 four chained bf16 MFMAs per 1024 scores with
// multiply + exp2 + add (the bf16-point half-pass mix at d = 64: four data K
// blocks, the bias entering as accumulator input, the multiply an fma with
// the row shift), 11 multiply + exp2 + add.
// wgs_per_cu: workgroups of 256 threads per CU in the grid (0: 8, i.e. up to
// 8 waves per SIMD where registers allow). Writes the work done (operations,
// scores or bytes) and the kernel time in ms; returns 0, -1 for an invalid
// argument or a negative HIP error.
int skp_measure(int which, int wgs_per_cu, double* work, double* ms_out, int* cus) {
  if (which > 11 || which < 0 || wgs_per_cu < 0 || wgs_per_cu > 32) return -1;
  hipError_t e;
  if (g_cus == 0) {
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return -(int)e;
    if ((e = hipDeviceGetAttribute(&g_cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return -(int)e;
  }
  *cus = g_cus;
  Ctx c{};
  c.which = which;
  c.blocks = g_cus * (wgs_per_cu ? wgs_per_cu : 8);
  int64_t buf_bytes = 0;
  if (which <= 6 || which >= 10) {
    c.iters = (which == 4 || which == 5) ? 20000 : (which == 6 || which == 10 ? 8000 : 40000);
  } else {
    // HBM: 4 GiB read once (16x the MALL); L2: 1 MiB read by every workgroup
    // 16 times; MALL: 64 MiB (8 MiB per XCD share, twice an XCD's L2) 32 times.
    buf_bytes = which == 7 ? ((int64_t)4 << 30) : (which == 8 ? ((int64_t)1 << 20) : ((int64_t)64 << 20));
    c.count = buf_bytes / 16;
    c.passes = which == 7 ? 1 : (which == 8 ? 16 : 32);
  }
  const int64_t outs = (int64_t)c.blocks * kThreads;
  if ((e = hipMalloc(&c.out, outs * sizeof(float))) != hipSuccess) return -(int)e;
  f32x4* buf = nullptr;
  if (buf_bytes) {
    if ((e = hipMalloc(&buf, buf_bytes)) != hipSuccess) {
      (void)hipFree(c.out);
      return -(int)e;
    }
    if ((e = hipMemset(buf, 0, buf_bytes)) != hipSuccess) {
      (void)hipFree(buf);
      (void)hipFree(c.out);
      return -(int)e;
    }
    c.buf = buf;
  }
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  float ms = 0.0f;
  e = timed(e0, e1, &ms, launch_one, &c);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (buf) (void)hipFree(buf);
  (void)hipFree(c.out);
  if (e != hipSuccess) return -(int)e;
  const double threads = (double)outs, waves = threads / 64.0;
  switch (which) {
    case 0: case 1: case 2: *work = threads * c.iters * 8; break;   // lane operations
    case 3: case 11: *work = threads * c.iters * 16; break;          // scores
    case 4: *work = waves * c.iters * 4 * 32768.0; break;            // flops
    case 5: *work = waves * c.iters * 4 * 4096.0; break;             // flops
    case 6: case 10: *work = waves * c.iters * 1024.0; break;        // scores
    case 8: *work = (double)c.count * 16.0 * c.passes * c.blocks; break;  // bytes
    default: *work = (double)c.count * 16.0 * c.passes; break;       // bytes
  }
  *ms_out = ms;
  return 0;
}

}  // extern "C"
