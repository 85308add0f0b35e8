// sk_mfma_dev.h -- device helpers shared by the matrix-core half-pass kernels
// (library-internal; included by pass_mfma.hip, pass_gemm.hip and pass_pv.hip).
#pragma once

#include "sk_mfma.h"
#include "sk_sync.h"

#include <math.h>

namespace sk {
namespace dev {

constexpr float kMaskedBias = -1.0e30f;  // bias of a column that contributes nothing

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 64-bit coherent load of a split partial (M, S) (both words written with
// store_coherent before their writer counted itself in).
__device__ __forceinline__ float2 load_coherent2(const float2* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(float2, v);
}

// A row's split partials (M_s, S_s) at part[s * stride], s = 0 .. count - 1,
// combined in split order: M = max_s M_s and S = sum_s S_s 2^(M_s - M') with
// M' = M (0 when every M_s is -inf). The loads go out eight at a time, so the
// merge waits for about one memory round trip per eight partials instead of
// one per partial (up to eight partials are loaded once).
__device__ inline void merge_partials(const float2* part, int64_t stride, int count, float& M, float& S) {
  constexpr int kB = 8;
  float2 v[kB];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kB; ++u)
      v[u] = s0 + u < count ? load_coherent2(part + (int64_t)(s0 + u) * stride) : make_float2(-INFINITY, 0.0f);
  };
  float Mt = -INFINITY;
  for (int s0 = 0; s0 < count; s0 += kB) {
    load_batch(s0);
#pragma unroll
    for (int u = 0; u < kB; ++u) Mt = fmaxf(Mt, v[u].x);
  }
  const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
  float St = 0.0f;
  for (int s0 = 0; s0 < count; s0 += kB) {
    if (count > kB) load_batch(s0);  // else the batch is still in registers
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (s0 + u < count) St = fmaf(v[u].y, fast_exp2(v[u].x - Me), St);
  }
  M = Mt;
  S = St;
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Three-part bf16 split of v (v ~= hi + mid + lo to float32 precision).
__device__ __forceinline__ void split3(float v, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = (__bf16)v;
  const float r1 = v - (float)hi;
  mid = (__bf16)r1;
  lo = (__bf16)(r1 - (float)mid);
}

// A column bias with -inf (zero weight) replaced by the masked value; NaN kept.
__device__ __forceinline__ float masked_bias(float htilde) { return htilde < kMaskedBias ? kMaskedBias : htilde; }

// Bias chunk of one column: (hi, mid, lo, 1, 1, 1, 0, 0). The three ones meet
// the row side's (-M) parts in the shifted sweep.
__device__ __forceinline__ void write_bias_chunk(bf16x8* dst, float htilde) {
  const float v = masked_bias(htilde);
  bf16x8 h0 = {};
  __bf16 a, b, c;
  split3(v, a, b, c);
  h0[0] = a;
  h0[1] = b;
  h0[2] = c;
  h0[3] = (__bf16)1.0f;
  h0[4] = (__bf16)1.0f;
  h0[5] = (__bf16)1.0f;
  *dst = h0;
}

// Separate bias record of one column: half 0 = the bias chunk, half 1 = zeros.
__device__ __forceinline__ void write_bias_record(bf16x8* rec, float htilde) {
  write_bias_chunk(rec, htilde);
  rec[1] = bf16x8{};
}

// Row-side bias block: (1, 1, 1, -M parts) in half 0, zeros in half 1.
__device__ __forceinline__ bf16x8 row_aug(int half, float neg_m) {
  bf16x8 r = {};
  if (half == 0) {
    r[0] = (__bf16)1.0f;
    r[1] = (__bf16)1.0f;
    r[2] = (__bf16)1.0f;
    __bf16 a, b, c;
    split3(neg_m, a, b, c);
    r[3] = a;
    r[4] = b;
    r[5] = c;
  }
  return r;
}

// What the potential update of row i reads besides its log2-sum-exp; loaded
// ahead of the partial merge, so that the two latencies overlap.
struct RowIn {
  float alpha, lw, pot, hval;
};
__device__ __forceinline__ RowIn load_row_in(const MfmaPassArgs& p, int i) {
  return RowIn{p.alpha[i], p.lw[i], p.symmetric ? p.pot[i] : 0.0f, p.hval_in[i]};
}

// Potential update of row i from its log2-sum-exp L; returns the change of the
// row's bias (log2 units) since the previous pass of this side.
__device__ __forceinline__ float finish_row_mfma(const MfmaPassArgs& p, int i, float L, const RowIn& r) {
  float v = fmaf(p.neg_eps_ln2, L, r.alpha);
  if (p.symmetric) v = 0.5f * (r.pot + v);
  p.pot[i] = v;
  const float h = fmaf(kLog2e, r.lw, (v - r.alpha) * p.log2e_over_eps);
  write_bias_chunk(p.bias_out + (int64_t)i * p.bias_stride, h * p.bias_scale);
  if (p.hout) p.hout[i] = masked_bias(h * p.bias_scale);
  const float dh = h - r.hval;
  p.hval_out[i] = h;
  p.Lout[i] = L;
  return dh;
}
__device__ __forceinline__ float finish_row_mfma(const MfmaPassArgs& p, int i, float L) {
  return finish_row_mfma(p, i, L, load_row_in(p, i));
}

// max(a, b, c): one v_maximum3_f32 (IEEE maximum: a NaN operand gives NaN, so
// a NaN score still propagates to the sum). Plain builtins, so the compiler
// places the wait states an MFMA result needs before a vector-ALU read.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Online update of a lane's running (M, S) with one 32x32 tile (16 scores per lane).
// M is in accumulator units; the exponent of a score is e * (acc - M).
__device__ __forceinline__ void lse_update(const f32x16& acc, float e, float& M, float& S) {
  const float m1 = max3(acc[0], acc[1], acc[2]);
  const float m2 = max3(acc[3], acc[4], acc[5]);
  const float m3 = max3(acc[6], acc[7], acc[8]);
  const float m4 = max3(acc[9], acc[10], acc[11]);
  const float m5 = max3(acc[12], acc[13], acc[14]);
  const float Mn = max3(max3(m1, m2, m3), max3(m4, m5, acc[15]), M);
  const bool valid = Mn > 0.5f * kMaskedBias;  // some real (unmasked) column seen
  const float Me = valid ? Mn : 0.0f;
  const float off = -e * Me;
  const float scale = fast_exp2(fmaf(M, e, off));  // M = -inf -> 0
  float s0 = fast_exp2(fmaf(acc[0], e, off));
  float s1 = fast_exp2(fmaf(acc[1], e, off));
  float s2 = fast_exp2(fmaf(acc[2], e, off));
  float s3 = fast_exp2(fmaf(acc[3], e, off));
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    s0 += fast_exp2(fmaf(acc[r + 0], e, off));
    s1 += fast_exp2(fmaf(acc[r + 1], e, off));
    s2 += fast_exp2(fmaf(acc[r + 2], e, off));
    s3 += fast_exp2(fmaf(acc[r + 3], e, off));
  }
  S = fmaf(S, scale, (s0 + s1) + (s2 + s3));
  M = valid ? Mn : M;
}

// Shifted update with the row shift outside the accumulator: every term is
// exp2(e * acc + off), off = -(row shift) in log2 units.
__device__ __forceinline__ void sum_update_off(const f32x16& acc, float e, float off, float& S) {
  auto ex = [&](float a) { return fast_exp2(fmaf(a, e, off)); };
  float s0 = ex(acc[0]), s1 = ex(acc[1]), s2 = ex(acc[2]), s3 = ex(acc[3]);
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    s0 += ex(acc[r + 0]);
    s1 += ex(acc[r + 1]);
    s2 += ex(acc[r + 2]);
    s3 += ex(acc[r + 3]);
  }
  S += (s0 + s1) + (s2 + s3);
}

// Shifted update: the row shift is already inside acc (bias block), so every
// term is exp2(e * acc) with no running maximum. SCALED: e != 1 (bf16 points).
template <bool SCALED>
__device__ __forceinline__ void sum_update(const f32x16& acc, float e, float& S) {
  auto ex = [&](float a) { return fast_exp2(SCALED ? a * e : a); };
  float s0 = ex(acc[0]), s1 = ex(acc[1]), s2 = ex(acc[2]), s3 = ex(acc[3]);
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    s0 += ex(acc[r + 0]);
    s1 += ex(acc[r + 1]);
    s2 += ex(acc[r + 2]);
    s3 += ex(acc[r + 3]);
  }
  S += (s0 + s1) + (s2 + s3);
}

// Block-wide max of v (every thread of the workgroup must call it).
__device__ inline float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

constexpr float kShiftedFloor = 0x1p-60f;  // below this a shifted sum is recomputed exactly

// ---------------------------------------------------------------- column tiles
// Column operands of one 32-column tile for this lane: its half of the record
// of column (tile start + li), NKB data chunks plus the bias chunk.
template <int NKB>
struct ColTile {
  bf16x8 a[NKB];
  bf16x8 aug;
};

// Record and bias arrays are padded past the last column with masked columns
// (zero data, masked bias) for five extra tiles, so a tile load needs no
// bounds test: the loads are plain and can be issued well ahead of use.
template <int NKB>
__device__ __attribute__((always_inline)) inline void load_tile(
    ColTile<NKB>& ct, const unsigned char* __restrict__ cols, const bf16x8* __restrict__ bias,
    int jt, int li, int half) {
  const int j = jt + li;
  const bf16x8* rec = reinterpret_cast<const bf16x8*>(cols + (int64_t)j * (NKB * 32)) + half * NKB;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) ct.a[kb] = rec[kb];
  ct.aug = bias[2 * (int64_t)j + half];
}

// MFMA products of one 32-column tile against the RB row blocks.
template <int NKB, int RB>
__device__ __attribute__((always_inline)) inline void tile_mfma(
    const ColTile<NKB>& ct, const bf16x8 (&B)[RB][NKB], const bf16x8 (&Baug)[RB], f32x16 (&acc)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x16 a = {};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct.a[kb], B[rb][kb], a, 0, 0, 0);
    acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct.aug, Baug[rb], a, 0, 0, 0);
  }
}

// s_waitcnt vmcnt(N), other counters not waited on (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// One 16-byte-per-lane global-to-LDS load from a wave-uniform base address
// (SGPR pair) plus a per-lane 32-bit byte offset: lane l's 16 bytes land at
// lds_addr + 16 l. Written as inline assembly so that the compiler does not
// treat the in-flight load as aliasing every later LDS read (it would wait for
// all of them); completion is waited for explicitly with vmcnt. The uniform
// base keeps the per-stage address arithmetic on the scalar unit.
__device__ __forceinline__ void load_to_lds(const void* base, unsigned lane_off, const void* lds_dst) {
  const unsigned m0 = (unsigned)(uintptr_t)lds_dst;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base), "{m0}"(m0) : "memory");
}

// As load_to_lds with 4 bytes per lane: lane l's 4 bytes land at lds_addr + 4 l.
__device__ __forceinline__ void load_to_lds_dword(const void* base, unsigned lane_off, const void* lds_dst) {
  const unsigned m0 = (unsigned)(uintptr_t)lds_dst;
  asm volatile("global_load_lds_dword %0, %1" ::"v"(lane_off), "s"(base), "{m0}"(m0) : "memory");
}

}  // namespace dev
}  // namespace sk
