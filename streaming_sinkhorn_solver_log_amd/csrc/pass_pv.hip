// pass_pv.hip -- matrix-core transport application (P V, P^T U) and
// barycentric gradient.
//
// Both are weighted sums over columns of the half-pass scores (FlashSinkhorn
// replication review, Summary: the released primitives apply the plan to a
// matrix without forming it, and the gradient is the barycentric projection,
// i.e. an attention output with the plan's row-softmax as weights):
//
//   apply: out_i = sum_j 2^{r_i + s_ij} V_j,   r_i = log2 a_i + (f_i - |x_i|^2) log2(e) / eps
//   grad:  O_i   = sum_j 2^{s_ij} y_j / sum_j 2^{s_ij},   out_i = 2 a_i (x_i - O_i)
//
// with s_ij = e * acc_ij the score of the half-pass (column bias included,
// no row shift). A score tile comes out of the MFMA as in the half-pass; its
// entries are then the B operand of a second MFMA against the tile's values.
// In lane l (h = l / 32) register r = 8 kb + e of a score accumulator holds
// the entry of row l % 32 at tile column 16 kb + 8 (e / 4) + 4 h + e % 4, and
// a 32x32x16 B operand wants, in the same lane, K slots 8 h + e of column
// l % 32: so the accumulator, converted to bf16, IS the B operand of two K
// blocks, provided the values (the A operand, value index l % 32) are stored
// in that column order. pack_values writes them so, once per call.
//
// Precision: entries and values are split into bf16 parts (float32 points:
// three and three; the entries' leading parts are truncations, of relative
// order 1, 2^-7, 2^-14, the values' are rounded, 1, 2^-8, 2^-16, and the six
// products kept leave out terms of order 2^-22 and below: float32 accuracy;
// bf16 points: two parts of the entries (2^-16) and two of the values for
// P V, or one exact part of the bf16 points for the gradient). That is the
// form of the 1-2 block GEMM-tiled kernels and of the Hessian-vector
// product's applications; the register-resident kernel and the wide kernel
// run in the half-precision form (H): as the attention output of
// FlashAttention feeds its probabilities to the second product in 16-bit
// form, the entries are float16 parts (bf16 points: one part rounded to
// nearest, 11 significant bits, relative error <= 2^-11, within the 1e-3
// bound of bf16 inputs; float32 points: two parts, the entry and its
// remainder each rounded, 2^-22), and the values are float16 parts
// (bf16 points: two for applications, one, exact, for the gradient's points;
// float32 points: two) after an exact power-of-two scale per value column
// that puts the column's largest magnitude in [2^13, 2^14); products of
// combined order below the larger part count are kept. float16's range
// is kept by the stabilization below: the entries of a row are biased so the
// running maximum term is 2^8 and stay below 2^15; terms 2^22 below the
// maximum reach float16's subnormals, where the absolute error 2^-33 of the
// maximum per term is negligible.
//
// Stabilization: a running row maximum mu (acc units), raised only when a
// tile's maximum exceeds it by more than 2^16 in value (lazy rescaling: terms
// stay below 2^16, the accumulators are rescaled rarely). The maximum is taken
// over both halves of the wave, so one shift holds for a whole MFMA sum.
#include "sk_internal.h"
#include "sk_mfma.h"
#include "sk_gemm.h"
#include "sk_gemm_dev.h"

#include <atomic>
#include <math.h>

namespace sk {
namespace {

using namespace dev;

constexpr float kMuInit = -1.0e29f;  // no column seen yet (above any masked score)
constexpr float kLazy = 16.0f;       // raise mu when a term would exceed 2^16
// Half-precision form: terms 2^(e (acc - mu) + kHalfBias), raised when one
// would exceed 2^15 (float16's largest power of two).
constexpr float kHalfBias = 8.0f;
constexpr float kHalfLazy = 15.0f - kHalfBias;
constexpr int kVmaxCols = 4096;  // value columns of one application (the C-ABI allows k <= 4096)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Power-of-two exponent k of a value column's scale 2^k: the column's largest
// magnitude (float bits, as k_value_max writes them) times 2^k lies in
// [2^13, 2^14); 0 for an all-zero column, clamped so the scale is a normal float.
__device__ __forceinline__ int half_scale_exp(unsigned maxbits) {
  if (maxbits == 0u) return 0;
  const int be = (int)(maxbits >> 23);  // biased exponent (0: subnormal, 255: inf / nan)
  const int ex = (be == 0 ? 1 : be) - 126;  // max = m 2^ex, m in [0.5, 1) for normal values
  const int k = 14 - ex;
  return k < -126 ? -126 : (k > 126 ? 126 : k);
}

template <int NOB, int VP>
struct VTile {
  bf16x8 v[NOB][VP][2];
};

__device__ __forceinline__ const bf16x8* vfrag_at(const PvArgs& p, int64_t tile, int ob, int vp_parts,
                                                  int vp, int kb) {
  return p.vfrag + ((((tile * p.nobt + ob) * vp_parts + vp) * 2 + kb) << 6);
}

// Lane l supplies value index l % 32 of each block. Lanes past the value
// width read the fragment of the first lane of their half instead of their
// own (zero) one: the same cache lines as the live lanes, and no registers to
// clear. What they hold only reaches output rows past the value width, which
// are never stored.
template <int NOB, int VP>
__device__ __attribute__((always_inline)) inline void load_vtile(VTile<NOB, VP>& vt, const PvArgs& p,
                                                                 int64_t tile, int ob0, int lane) {
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) {
    const int src = (ob0 + ob) * 32 + (lane & 31) < p.kv ? lane : (lane & 32);
#pragma unroll
    for (int vp = 0; vp < VP; ++vp)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) vt.v[ob][vp][kb] = vfrag_at(p, tile, ob0 + ob, VP, vp, kb)[src];
  }
}

__device__ __forceinline__ float max16(const f32x16& a) {
  const float m1 = max3(a[0], a[1], a[2]);
  const float m2 = max3(a[3], a[4], a[5]);
  const float m3 = max3(a[6], a[7], a[8]);
  const float m4 = max3(a[9], a[10], a[11]);
  const float m5 = max3(a[12], a[13], a[14]);
  return max3(max3(m1, m2, m3), max3(m4, m5, a[15]), a[15]);
}

// Lazy running maximum of a row over NT score tiles; returns the exponent
// offset -e*mu (H: -e*mu + kHalfBias).
template <int NT, int NOB, bool H = false>
__device__ __attribute__((always_inline)) inline float pv_shift(const f32x16 (&acc)[NT], float e, float& mu,
                                                                float& S, f32x16 (&O)[NOB]) {
  float tm = max16(acc[0]);
#pragma unroll
  for (int t = 1; t < NT; ++t) tm = max3(tm, max16(acc[t]), tm);
  const float to = __shfl_xor(tm, 32);
  tm = max3(tm, to, to);
  const bool raise = e * (tm - mu) > (H ? kHalfLazy : kLazy);
  if (__any(raise)) {
    const float mn = raise ? tm : mu;
    const float sc = fast_exp2(e * (mu - mn));
    S *= sc;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[ob][r] *= sc;
    mu = mn;
  }
  return H ? fmaf(-e, mu, kHalfBias) : -e * mu;
}

// Two floats' upper 16 bits packed as a bf16 pair (a in the low half): the
// truncated bf16 parts, one v_perm_b32.
__device__ __forceinline__ unsigned pack_hi16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// a and b rounded to bf16 (nearest even), packed (a in the low half).
__device__ __forceinline__ unsigned pack_bf16_rne(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float trunc_bf16(float v) { return __uint_as_float(__float_as_uint(v) & 0xFFFF0000u); }

// Plan entries of one score tile (terms <= 2^16), their sum (SUM), and their
// bf16 parts as the B operands of two K blocks. All parts but the last are
// truncations (v - part is then exact), the last is rounded to nearest: two
// parts carry 16 bits (relative error <= 2^-16), three carry float32's 24.
template <int PP, bool SUM>
__device__ __attribute__((always_inline)) inline float pv_probs(const f32x16& acc, float e, float off,
                                                               bf16x8 (&P)[PP][2]) {
  u32x4 W[PP][2];
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float v0 = fast_exp2(fmaf(acc[r], e, off));
    const float v1 = fast_exp2(fmaf(acc[r + 1], e, off));
    if constexpr (SUM) {
      s0 = r == 0 ? v0 : s0 + v0;
      s1 = r == 0 ? v1 : s1 + v1;
    }
    const int kb = r >> 3, w = (r & 7) >> 1;
    if constexpr (PP == 1) {
      W[0][kb][w] = pack_bf16_rne(v0, v1);
    } else {
      W[0][kb][w] = pack_hi16(v0, v1);
      const float r0 = v0 - trunc_bf16(v0), r1 = v1 - trunc_bf16(v1);
      if constexpr (PP == 2) {
        W[1][kb][w] = pack_bf16_rne(r0, r1);
      } else {
        W[1][kb][w] = pack_hi16(r0, r1);
        W[2][kb][w] = pack_bf16_rne(r0 - trunc_bf16(r0), r1 - trunc_bf16(r1));
      }
    }
  }
#pragma unroll
  for (int pp = 0; pp < PP; ++pp)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) P[pp][kb] = __builtin_bit_cast(bf16x8, W[pp][kb]);
  return s0 + s1;
}

// Remainder v - (float)h of an entry and its float16 part h, lane half HI of
// the packed pair hp: one v_fma_mix_f32 (h * -1 + v with h read as float16
// from the selected half; exact, as the difference of v and a float16
// rounding of it). The compiler writes this as a conversion back and a
// subtraction, and converts v to float16 a second time for them.
template <int HI>
__device__ __forceinline__ float half_remainder(unsigned hp, float v) {
  float r;
  if constexpr (HI) asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hp), "v"(v));
  else asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hp), "v"(v));
  return r;
}

// Half-precision form of pv_probs: the entries (terms < 2^15) as PP float16
// parts each (v_cvt_pk_f16_f32, rounded to nearest), and their float32 sum
// (SUM). Two parts: the entry's float16 rounding and the rounded remainder,
// relative error <= 2^-22.
template <int PP, bool SUM>
__device__ __attribute__((always_inline)) inline float pv_probs_h(const f32x16& acc, float e, float off,
                                                                 f16x8 (&P)[PP][2]) {
  static_assert(PP == 1 || PP == 2, "one or two float16 parts");
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float v0 = fast_exp2(fmaf(acc[r], e, off));
    const float v1 = fast_exp2(fmaf(acc[r + 1], e, off));
    if constexpr (SUM) {
      s0 = r == 0 ? v0 : s0 + v0;
      s1 = r == 0 ? v1 : s1 + v1;
    }
    const f16x2 h = {(_Float16)v0, (_Float16)v1};
    P[0][r >> 3][r & 7] = h[0];
    P[0][r >> 3][(r & 7) + 1] = h[1];
    if constexpr (PP == 2) {
      const unsigned hp = __builtin_bit_cast(unsigned, h);
      const f16x2 l = {(_Float16)half_remainder<0>(hp, v0), (_Float16)half_remainder<1>(hp, v1)};
      P[1][r >> 3][r & 7] = l[0];
      P[1][r >> 3][(r & 7) + 1] = l[1];
    }
  }
  return s0 + s1;
}

// O[ob] += V[ob] x P in float16 over the products (pp, vp) of combined order
// below max(PP, VP) (fragments hold float16 bits in the half-precision form).
template <int NOB, int PP, int VP>
__device__ __attribute__((always_inline)) inline void pv_mfma_h(const VTile<NOB, VP>& vt, const f16x8 (&P)[PP][2],
                                                                f32x16 (&O)[NOB]) {
  constexpr int KMAX = PP > VP ? PP : VP;
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int vp = 0; vp < VP; ++vp)
        if (pp + vp < KMAX) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            O[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vt.v[ob][vp][kb]), P[pp][kb],
                                                           O[ob], 0, 0, 0);
        }
}

// Weighted plan entries of one score tile: 2^{e acc + off} * q (q: the
// weights in the accumulator layout), split into PP bf16 parts as pv_probs
// does (the weights may be negative: the truncated parts keep the sign and
// the remainders stay exact).
template <int PP>
__device__ __attribute__((always_inline)) inline void pv_probs_w(const f32x16& acc, const f32x16& q, float qo, float e,
                                                               float off, bf16x8 (&P)[PP][2]) {
  u32x4 W[PP][2];
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float v0 = fast_exp2(fmaf(acc[r], e, off)) * (q[r] + qo);
    const float v1 = fast_exp2(fmaf(acc[r + 1], e, off)) * (q[r + 1] + qo);
    const int kb = r >> 3, w = (r & 7) >> 1;
    if constexpr (PP == 1) {
      W[0][kb][w] = pack_bf16_rne(v0, v1);
    } else {
      W[0][kb][w] = pack_hi16(v0, v1);
      const float r0 = v0 - trunc_bf16(v0), r1 = v1 - trunc_bf16(v1);
      if constexpr (PP == 2) {
        W[1][kb][w] = pack_bf16_rne(r0, r1);
      } else {
        W[1][kb][w] = pack_hi16(r0, r1);
        W[2][kb][w] = pack_bf16_rne(r0 - trunc_bf16(r0), r1 - trunc_bf16(r1));
      }
    }
  }
#pragma unroll
  for (int pp = 0; pp < PP; ++pp)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) P[pp][kb] = __builtin_bit_cast(bf16x8, W[pp][kb]);
}

// O[ob] += V[ob] x P over the products (pp, vp) of combined order below max(PP, VP).
template <int NOB, int PP, int VP>
__device__ __attribute__((always_inline)) inline void pv_mfma(const VTile<NOB, VP>& vt, const bf16x8 (&P)[PP][2],
                                                              f32x16 (&O)[NOB]) {
  constexpr int KMAX = PP > VP ? PP : VP;
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int pp = 0; pp < PP; ++pp)
#pragma unroll
      for (int vp = 0; vp < VP; ++vp)
        if (pp + vp < KMAX) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            O[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt.v[ob][vp][kb], P[pp][kb], O[ob], 0, 0, 0);
        }
}

// Output element (row i, value index cc) from the merged (mu, S, T) of the row.
// Half-precision form (vmax non-null): T carries the column's value scale
// 2^k and, in the application, the entries' bias 2^kHalfBias (the gradient's
// S carries the same bias and it cancels).
__device__ __forceinline__ void pv_store(const PvArgs& p, int i, int cc, float mu, float S, float T) {
  const int64_t o = (int64_t)i * p.kv + cc;
  if (p.vmax) T = ldexpf(T, -half_scale_exp(p.vmax[cc]));
  if (p.grad) {
    float xv;
    if (p.xbf16) xv = __uint_as_float((unsigned)static_cast<const unsigned short*>(p.xrow)[o] << 16);
    else xv = static_cast<const float*>(p.xrow)[o];
    if (p.shift) xv -= p.shift[cc];
    p.out[o] = 2.0f * p.wrow[i] * (xv - T / S);
  } else {
    const float h = fmaf(p.escale, mu, p.hrow[i]);
    p.out[o] = T * fast_exp2(p.vmax ? h - kHalfBias : h);
  }
}

// End of a workgroup: with one split, every lane writes its rows' outputs;
// otherwise the partials (mu, S, T) go to the split buffer, which k_pv_merge
// combines after the launch. Lanes of inactive waves hold nothing.
template <int RB, int NOB>
__device__ __attribute__((always_inline)) inline void pv_finish(
    const PvArgs& p, bool active, int row_base, const f32x16 (&O)[RB][NOB],
    const float (&mu)[RB], const float (&S)[RB], int li, int half) {
  constexpr int CW = NOB * 32;
  const int sp = blockIdx.y, z = blockIdx.z;
  const int cbase = z * CW;
  float St[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) St[rb] = S[rb] + __shfl_xor(S[rb], 32);
  if (p.splits == 1) {
    if (!active) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = row_base + rb * 32 + li;
      if (i >= p.nr) continue;
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cc = cbase + ob * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (cc < p.kv) pv_store(p, i, cc, mu[rb], St[rb], O[rb][ob][r]);
        }
    }
    return;
  }
  const int64_t nslots = (int64_t)p.nchunks * p.splits;
  float2* part_ms = reinterpret_cast<float2*>(p.part);
  float* part_t = p.part + ((2 * nslots * p.nr + 3) & ~(int64_t)3);  // 16-byte aligned value partials
  const int64_t slot = (int64_t)z * p.splits + sp;
  if (!active) return;
  // p.pcw (a multiple of 8, at most CW) value partials per row: the columns
  // past a narrower value width are not written
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = row_base + rb * 32 + li;
    if (i >= p.nr) continue;
    if (half == 0) part_ms[slot * p.nr + i] = make_float2(mu[rb], St[rb]);
    float* T = part_t + (slot * p.nr + i) * p.pcw;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (ob * 32 + 8 * q < p.pcw)
          *reinterpret_cast<float4*>(T + ob * 32 + 8 * q + 4 * half) =
              make_float4(O[rb][ob][4 * q], O[rb][ob][4 * q + 1], O[rb][ob][4 * q + 2], O[rb][ob][4 * q + 3]);
  }
}

// Shared column stages of the register-resident kernel: the four waves of a
// workgroup sweep the same columns (each its own rows), so a stage of
// kPvStageTiles column tiles -- per tile the NKB record blocks, the bias
// chunk and the NOB x VP x 2 value fragments, 1 KB each, in the lane order
// of the operands -- is loaded once into LDS by direct global-to-LDS loads
// (the waves split the blocks) instead of once per wave: with every wave
// loading its own copy the vector memory path (texture addresser) is the
// bottleneck at d = 64. Two stages in flight, one barrier per stage.
constexpr int kPvStageTiles = 2;
template <int NKB, int NOB, int VP>
struct PvStage {
  static constexpr int kValBlocks = NOB * VP * 2;
  static constexpr int kBlocks = NKB + 1 + kValBlocks;  // per tile
  bf16x8 blk[2][kPvStageTiles][kBlocks][64];
};

// This wave's share of stage (first tile t): blocks wave, wave + 4, ... of
// the stage. Tiles past the sweep's last read the padding or the next range
// (never used); value lanes past the value width read their half's first
// lane's fragment, as load_vtile does.
template <int NKB, int NOB, int VP>
__device__ __attribute__((always_inline)) inline void pv_issue_stage(
    PvStage<NKB, NOB, VP>& L, int slot, const PvArgs& p, const unsigned char* __restrict__ cols, int64_t t,
    int ob0, int wave, int lane) {
  using Stg = PvStage<NKB, NOB, VP>;
  constexpr int NB = kPvStageTiles * Stg::kBlocks;
  const int li = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const unsigned off_rec = (unsigned)(li * (NKB * 32) + h * (NKB * 16));
  const unsigned off_bias = (unsigned)(li * 32 + h * 16);
#pragma unroll
  for (int q = 0; q < (NB + 3) / 4; ++q) {
    const int b = wv + 4 * q;
    if (b >= NB) break;  // wave-uniform: the last round has fewer blocks than waves
    const int tt = b / Stg::kBlocks, kb = b % Stg::kBlocks;
    const int64_t tile = t + tt;
    if (kb < NKB) {
      load_to_lds(cols + tile * 32 * (NKB * 32) + kb * 16, off_rec, &L.blk[slot][tt][kb][0]);
    } else if (kb == NKB) {
      load_to_lds(reinterpret_cast<const unsigned char*>(p.bias_col) + tile * 32 * 32, off_bias,
                  &L.blk[slot][tt][kb][0]);
    } else {
      const int v = kb - NKB - 1;  // (ob * VP + vp) * 2 + k
      const int ob = v / (VP * 2);
      const int src = (ob0 + ob) * 32 + li < p.kv ? lane : (lane & 32);
      load_to_lds(vfrag_at(p, tile, ob0 + ob, VP, (v / 2) % VP, v % 2), (unsigned)(src * 16),
                  &L.blk[slot][tt][kb][0]);
    }
  }
}

// Register-resident rows (record widths up to 8 K blocks): each wave keeps RB
// blocks of 32 row records and streams column tiles and their value fragments
// from memory, one tile ahead.
// Shared column stages (see PvStage) for records of four K blocks (bf16
// d = 33-64) with tiles of at most 9 blocks: two stages of two tiles, 36 KB;
// three workgroups per CU with one value block (168 registers; two value
// blocks would spill there).
template <int NKB, int NOB, int VP>
constexpr bool pv_shared() { return NKB == 4 && NKB + 1 + NOB * VP * 2 <= 9; }

template <int NKB, int RB, int NOB, int PP, int VP, bool GRAD, bool H>
__global__ __launch_bounds__(kThreads, (pv_shared<NKB, NOB, VP>() && NOB == 1 ? 3 : 2)) void k_pv_mfma(
    const PvArgs p) {
  constexpr bool kShared = pv_shared<NKB, NOB, VP>();
  constexpr int RSB = NKB * 32;
  constexpr int ROWS = 4 * RB * 32;
  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int ob0 = blockIdx.z * NOB;
  const int j0 = blockIdx.y * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int row_base = blockIdx.x * ROWS + wave * (RB * 32);
  const float e = p.escale;

  bf16x8 B[RB][NKB], Baug[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = row_base + rb * 32 + li;
    const bf16x8* rec = reinterpret_cast<const bf16x8*>(rows + (int64_t)min(i, p.nr - 1) * RSB) + half * NKB;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) B[rb][kb] = rec[kb];
    Baug[rb] = row_aug(half, 0.0f);
  }
  float mu[RB], S[RB];
  f32x16 O[RB][NOB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mu[rb] = kMuInit;
    S[rb] = 0.0f;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) O[rb][ob] = f32x16{};
  }

  // Plan entries of a scored tile, then their products with the tile's values
  // (H: the half-precision form).
  auto entries_work = [&](const f32x16 (&acc)[RB], const VTile<NOB, VP>& vt) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x16 a1[1] = {acc[rb]};
      const float off = pv_shift<1, NOB, H>(a1, e, mu[rb], S[rb], O[rb]);
      if constexpr (H) {
        f16x8 P[PP][2];
        if constexpr (GRAD) S[rb] += pv_probs_h<PP, true>(acc[rb], e, off, P);
        else pv_probs_h<PP, false>(acc[rb], e, off, P);
        pv_mfma_h<NOB, PP, VP>(vt, P, O[rb]);
      } else {
        bf16x8 P[PP][2];
        if constexpr (GRAD) S[rb] += pv_probs<PP, true>(acc[rb], e, off, P);
        else pv_probs<PP, false>(acc[rb], e, off, P);  // the application never divides by S
        pv_mfma<NOB, PP, VP>(vt, P, O[rb]);
      }
    }
  };

  const int ntiles = (j1 - j0 + 31) / 32;
  const int64_t t0 = j0 / 32;
  if constexpr (kShared) {
    using Stg = PvStage<NKB, NOB, VP>;
    __shared__ __attribute__((aligned(16))) Stg L;
    const int nstages = (ntiles + kPvStageTiles - 1) / kPvStageTiles;
    if (nstages > 0) pv_issue_stage<NKB, NOB, VP>(L, 0, p, cols, t0, ob0, wave, lane);
    for (int st = 0; st < nstages; ++st) {
      const int slot = st & 1;
      wait_vmcnt<0>();  // this wave's loads of stage st
      __syncthreads();  // everyone's; the other slot (stage st - 1) is free
      if (st + 1 < nstages)
        pv_issue_stage<NKB, NOB, VP>(L, slot ^ 1, p, cols, t0 + (st + 1) * kPvStageTiles, ob0, wave, lane);
      const int nt = min(kPvStageTiles, ntiles - st * kPvStageTiles);
#pragma unroll
      for (int tt = 0; tt < kPvStageTiles; ++tt) {
        if (tt < nt) {
          ColTile<NKB> ct;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) ct.a[kb] = L.blk[slot][tt][kb][lane];
          ct.aug = L.blk[slot][tt][NKB][lane];
          f32x16 acc[RB];
          tile_mfma<NKB, RB>(ct, B, Baug, acc);
          VTile<NOB, VP> vt;
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int vp = 0; vp < VP; ++vp)
#pragma unroll
              for (int k = 0; k < 2; ++k) vt.v[ob][vp][k] = L.blk[slot][tt][NKB + 1 + (ob * VP + vp) * 2 + k][lane];
          entries_work(acc, vt);
        }
      }
    }
    pv_finish<RB, NOB>(p, true, row_base, O, mu, S, li, half);
    return;
  }
  ColTile<NKB> c0, c1;
  VTile<NOB, VP> v0, v1;
  // Each tile is scored, then used; loads run one tile ahead (the loop reads
  // at most one tile past its last one: padding or the next range).
  auto tile_work = [&](const ColTile<NKB>& ct, const VTile<NOB, VP>& vt) {
    f32x16 acc[RB];
    tile_mfma<NKB, RB>(ct, B, Baug, acc);
    entries_work(acc, vt);
  };
  load_tile<NKB>(c0, cols, p.bias_col, j0, li, half);
  load_vtile<NOB, VP>(v0, p, t0, ob0, lane);
  for (int t = 0; t < ntiles; t += 2) {
    load_tile<NKB>(c1, cols, p.bias_col, j0 + (t + 1) * 32, li, half);
    load_vtile<NOB, VP>(v1, p, t0 + t + 1, ob0, lane);
    tile_work(c0, v0);
    if (t + 1 < ntiles) {
      load_tile<NKB>(c0, cols, p.bias_col, j0 + (t + 2) * 32, li, half);
      load_vtile<NOB, VP>(v0, p, t0 + t + 2, ob0, lane);
      tile_work(c1, v1);
    }
  }
  pv_finish<RB, NOB>(p, true, row_base, O, mu, S, li, half);
}

// GEMM-tiled variant for wide records: the score block of a 2 x 2-wave
// workgroup (128 rows x 128 columns per block, K streamed through LDS) feeds
// the value products of each wave's 64 x 64 quarter; the two column waves of
// a row pair merge their partials through LDS at the end.
template <int NOB, int PP, int VP>
__global__ __launch_bounds__(kThreads, 2) void k_pv_gemm(const PvArgs p, int nkb) {
  __shared__ __attribute__((aligned(16))) GemmLds lds;
  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int ob0 = blockIdx.z * NOB;
  const int j0 = blockIdx.y * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int r0 = blockIdx.x * kGRows;
  const float e = p.escale;

  bf16x8 Baug[2];
  float mu[2], S[2];
  f32x16 O[2][NOB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    Baug[rb] = row_aug(half, 0.0f);
    mu[rb] = kMuInit;
    S[rb] = 0.0f;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) O[rb][ob] = f32x16{};
  }

  const int nkc = nkb / kGKb;
  const int nblocks = (j1 - j0 + kGCols - 1) / kGCols;
  const int nstages = nblocks * nkc;
  GemmRegs g;
  gemm_load(g, rows, cols, nkb, p.nr, r0, j0, 0);
  gemm_store(g, lds, 0);
  __syncthreads();
  f32x16 acc[2][2];
  for (int st = 0; st < nstages; ++st) {
    const int blk = st / nkc, kc = st % nkc;
    const int buf = st & 1;
    if (st + 1 < nstages) {
      const int nb = (st + 1) / nkc, nk = (st + 1) % nkc;
      gemm_load(g, rows, cols, nkb, p.nr, r0, j0 + nb * kGCols, nk);
    }
    if (kc == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rb][ct] = f32x16{};
    }
#pragma unroll
    for (int kb = 0; kb < kGKb; ++kb) {
      bf16x8 A[2], Bm[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        A[ct] = *reinterpret_cast<const bf16x8*>(&lds.cols[buf][(wc * 64 + ct * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        Bm[rb] = *reinterpret_cast<const bf16x8*>(&lds.rows[buf][(wr * 64 + rb * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ct], Bm[rb], acc[rb][ct], 0, 0, 0);
    }
    // The next stage's operands go to LDS before the value products, so their
    // staging registers are free during them.
    if (st + 1 < nstages) gemm_store(g, lds, buf ^ 1);
    if (kc == nkc - 1) {
      const int cb = j0 + blk * kGCols + wc * 64;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x8 Aaug = p.bias_col[2 * (int64_t)(cb + ct * 32 + li) + half];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aaug, Baug[rb], acc[rb][ct], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float off = pv_shift<2, NOB>(acc[rb], e, mu[rb], S[rb], O[rb]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          bf16x8 P[PP][2];
          if (p.grad) S[rb] += pv_probs<PP, true>(acc[rb][ct], e, off, P);
          else pv_probs<PP, false>(acc[rb][ct], e, off, P);
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob) {
            VTile<1, VP> vt;
            load_vtile<1, VP>(vt, p, (cb >> 5) + ct, ob0 + ob, lane);
            f32x16 (&Oob)[1] = *reinterpret_cast<f32x16(*)[1]>(&O[rb][ob]);
            pv_mfma<1, PP, VP>(vt, P, Oob);
          }
        }
      }
    }
    __syncthreads();
  }

  // Column wave 1 hands its partials to column wave 0 of the same rows (same
  // lane layout) through the staging buffers, free after the last barrier:
  // first (mu, S), then two value blocks per round.
  constexpr int PER = 2 * (2 + 2 * 16);  // floats per lane per round
  static_assert(2 * PER * 64 * 4 <= (int)sizeof(GemmLds), "merge area exceeds the staging buffers");
  float* xl = reinterpret_cast<float*>(&lds) + wr * PER * 64 + lane;
  float f0[2], f1[2];
#pragma unroll
  for (int ob0 = 0; ob0 < NOB; ob0 += 2) {
    if (wc == 1) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        xl[(rb * 34) * 64] = mu[rb];
        xl[(rb * 34 + 1) * 64] = S[rb];
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (ob0 + q < NOB)
#pragma unroll
            for (int r = 0; r < 16; ++r) xl[(rb * 34 + 2 + q * 16 + r) * 64] = O[rb][ob0 + q][r];
      }
    }
    __syncthreads();
    if (wc == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (ob0 == 0) {
          const float mo = xl[(rb * 34) * 64];
          const float so = xl[(rb * 34 + 1) * 64];
          const float mt = fmaxf(mu[rb], mo);
          f0[rb] = fast_exp2(e * (mu[rb] - mt));
          f1[rb] = fast_exp2(e * (mo - mt));
          S[rb] = S[rb] * f0[rb] + so * f1[rb];
          mu[rb] = mt;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (ob0 + q < NOB)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              O[rb][ob0 + q][r] = O[rb][ob0 + q][r] * f0[rb] + xl[(rb * 34 + 2 + q * 16 + r) * 64] * f1[rb];
      }
    }
    __syncthreads();
  }
  pv_finish<2, NOB>(p, wc == 0, r0 + wr * 64, O, mu, S, li, half);
}

// GEMM-tiled variant for one value block (applications with k <= 32): the
// 256 x 256 workgroup tile of 8 waves of the large-d half-pass (4 row waves x
// 2 column waves, each 64 rows x 128 columns), K streamed through LDS; each
// column block's scores feed the value products of the wave's rows, and the
// two column waves of a row group merge their partials through LDS at the end.
using PvGeo = Geo<2, 4, 4>;

template <int PP, int VP, bool H>
__global__ __launch_bounds__(PvGeo::kNT, 1) void k_pv_gemm8(const PvArgs p, int nkb, int col_last) {
  using G = PvGeo;
  constexpr int WRT = 2, WCT = 4, kWaveRows = 64;
  __shared__ __attribute__((aligned(16))) TileLds<G> lds;
  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int ob0 = blockIdx.z;
  const int j0 = blockIdx.y * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int r0 = blockIdx.x * G::kRows;
  const float e = p.escale;

  bf16x8 Baug[WRT];
  float mu[WRT], S[WRT];
  f32x16 O[WRT][1];
#pragma unroll
  for (int rb = 0; rb < WRT; ++rb) {
    Baug[rb] = row_aug(half, 0.0f);
    mu[rb] = kMuInit;
    S[rb] = 0.0f;
    O[rb][0] = f32x16{};
  }

  const int nkc = nkb / kGKb;
  const int nblocks = (j1 - j0 + G::kCols - 1) / G::kCols;
  const int nstages = nblocks * nkc;
  auto load_stage = [&](TileRegs<G>& g, int st) {
    tile_load<G>(g, rows, cols, nkb, p.nr, col_last, r0, j0 + (st / nkc) * G::kCols, st % nkc);
  };
  TileRegs<G> g;
  load_stage(g, 0);
  tile_store<G>(g, lds, 0);
  if (nstages > 1) load_stage(g, 1);
  __syncthreads();
  f32x16 acc[WRT][WCT];
  for (int st = 0; st < nstages; ++st) {
    const int blk = st / nkc, kc = st % nkc;
    const int buf = st & 1;
    if (kc == 0) {
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb)
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) acc[rb][ct] = f32x16{};
    }
#pragma unroll
    for (int kb = 0; kb < kGKb; ++kb) {
      bf16x8 A[WCT], B[WRT];
#pragma unroll
      for (int ct = 0; ct < WCT; ++ct)
        A[ct] = *reinterpret_cast<const bf16x8*>(
            &lds.cols[buf][(wc * (G::kCols / 2) + ct * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb)
        B[rb] = *reinterpret_cast<const bf16x8*>(
            &lds.rows[buf][(wr * kWaveRows + rb * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb)
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ct], B[rb], acc[rb][ct], 0, 0, 0);
    }
    // the next stage's operands go to LDS before the epilogue, so their
    // staging registers are free during it
    if (st + 1 < nstages) tile_store<G>(g, lds, buf ^ 1);
    if (kc == nkc - 1) {
      const int cb = j0 + blk * G::kCols + wc * (G::kCols / 2);
#pragma unroll
      for (int ct = 0; ct < WCT; ++ct) {
        const bf16x8 Aaug = p.bias_col[2 * (int64_t)min(cb + ct * 32 + li, col_last) + half];
#pragma unroll
        for (int rb = 0; rb < WRT; ++rb)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aaug, Baug[rb], acc[rb][ct], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb) {
        const float off = pv_shift<WCT, 1, H>(acc[rb], e, mu[rb], S[rb], O[rb]);
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
          // a column block can overhang the padded columns by up to 7 tiles:
          // those columns are masked, so any zero-valued tile serves, here
          // the last padded one
          VTile<1, VP> vt;
          if constexpr (H) {
            f16x8 P[PP][2];
            if (p.grad) S[rb] += pv_probs_h<PP, true>(acc[rb][ct], e, off, P);
            else pv_probs_h<PP, false>(acc[rb][ct], e, off, P);
            load_vtile<1, VP>(vt, p, min((cb >> 5) + ct, col_last >> 5), ob0, lane);
            pv_mfma_h<1, PP, VP>(vt, P, O[rb]);
          } else {
            bf16x8 P[PP][2];
            if (p.grad) S[rb] += pv_probs<PP, true>(acc[rb][ct], e, off, P);
            else pv_probs<PP, false>(acc[rb][ct], e, off, P);
            load_vtile<1, VP>(vt, p, min((cb >> 5) + ct, col_last >> 5), ob0, lane);
            pv_mfma<1, PP, VP>(vt, P, O[rb]);
          }
        }
      }
    }
    if (st + 2 < nstages) load_stage(g, st + 2);
    __syncthreads();
  }

  // Column wave 1 hands (mu, S, O) to column wave 0 of the same rows (same
  // lane layout) through the staging buffers, free after the last barrier.
  constexpr int PER = WRT * (2 + 16);  // floats per lane
  static_assert(G::kNT / 128 * PER * 64 * 4 <= (int)sizeof(TileLds<G>), "merge area exceeds the staging buffers");
  float* xl = reinterpret_cast<float*>(&lds) + wr * PER * 64 + lane;
  if (wc == 1) {
#pragma unroll
    for (int rb = 0; rb < WRT; ++rb) {
      xl[(rb * 18) * 64] = mu[rb];
      xl[(rb * 18 + 1) * 64] = S[rb];
#pragma unroll
      for (int r = 0; r < 16; ++r) xl[(rb * 18 + 2 + r) * 64] = O[rb][0][r];
    }
  }
  __syncthreads();
  if (wc == 0) {
#pragma unroll
    for (int rb = 0; rb < WRT; ++rb) {
      const float mo = xl[(rb * 18) * 64];
      const float so = xl[(rb * 18 + 1) * 64];
      const float mt = fmaxf(mu[rb], mo);
      const float f0 = fast_exp2(e * (mu[rb] - mt)), f1 = fast_exp2(e * (mo - mt));
      S[rb] = S[rb] * f0 + so * f1;
      mu[rb] = mt;
#pragma unroll
      for (int r = 0; r < 16; ++r) O[rb][0][r] = O[rb][0][r] * f0 + xl[(rb * 18 + 2 + r) * 64] * f1;
    }
  }
  __syncthreads();
  pv_finish<WRT, 1>(p, wc == 0, r0 + wr * kWaveRows, O, mu, S, li, half);
}

// GEMM-tiled variant for wide value chunks (the gradient at large d: value
// width d up to 4 * NOBW * 32 per chunk). Each 64 x 128 score block is
// computed once: the four waves form it together (wave w: row tile w & 1,
// column tiles 2 (w >> 1) and 2 (w >> 1) + 1), agree on the rows' lazy shift
// through LDS, and write the plan entries' bf16 parts to LDS; each wave then
// applies all 64 x 128 entries to its own NOBW value blocks. The score work is
// thereby done once per value chunk instead of once per NOB = 4 blocks
// (k_pv_gemm).
//
// The score operands stream through a ring of LDS stages that direct
// global-to-LDS loads fill several stages ahead, one K chunk (4 K blocks, 128
// bytes per record) of the 64 row and 128 column records (and of the rows'
// tangent records) per stage. Each load instruction reads 8 whole 128-byte
// record chunks (coalesced) into 1 KB of LDS; within record r's 128 bytes the
// 16-byte piece c (K block c / 2, half c % 2) is stored at position
// c ^ ((r / 2) % 8), so that an MFMA operand read (records 32 t + li, one
// piece each) is free of bank conflicts: the LDS serves a 16-byte read 16
// lanes at a time (256 bytes, all 64 banks), and of 16 consecutive records the
// even ones start at bank 0 and the odd ones at bank 32, each group of eight
// meeting every piece position once (with c ^ (r % 8), records r and r + 8
// collided). Each stage's fragments are read right after the barrier that
// publishes it, while the previous stage's MFMAs still run.
constexpr int kPvwRows = 64;
constexpr int kPvwCols = 128;

template <int WQ>
struct PvwStage {
  static constexpr int kColOff = kPvwRows * 128;             // byte offsets within a stage
  static constexpr int kTanOff = (kPvwRows + kPvwCols) * 128;
  static constexpr int kBytes = (kPvwRows + kPvwCols + WQ * kPvwRows) * 128;
  static constexpr int kPerWave = kBytes / 1024 / 4;         // 1 KB load instructions per wave
  static constexpr int kRing = WQ > 0 ? 3 : 4;               // stages (tangent records take the room of one)
  static_assert(kBytes % 4096 == 0, "stage loads split evenly over four waves");
};

template <int PP, int WQ>
struct PvwLds {
  unsigned char ring[PvwStage<WQ>::kRing][PvwStage<WQ>::kBytes];
  bf16x8 P[2][4][PP][2][64];   // entries: row tile, column tile, part, K block, lane
  float tmax[2][2][32];        // per column half and row tile: each row's maximum over the block
  float ssum[2][2][32];        // per column half and row tile: partial row sums (gradient)
};

// This wave's loads of a stage: K chunk kc of rows [r0, r0 + 64), columns
// [c0, c0 + 128) and the rows' tangent records, into `dst`. Load q = 4 u +
// wave covers records [8 q', 8 q' + 8) of its region (rows for u < 2, columns
// for u < 6, then the tangent arrays; q' and q have the same parity); lane l
// reads piece (l % 8) ^ ((r / 2) % 8) of record r = 8 q' + l / 8, i.e. piece
// (l % 8) ^ (4 (q % 2) + l / 16), which lands at position l % 8 of that
// record's LDS chunk. Row indices clamp to the last row, column indices to
// the last padded (masked) column. The uniform part of each address is on the
// scalar unit.
template <int WQ>
__device__ __attribute__((always_inline)) inline void pvw_issue_stage(
    unsigned char* dst, const PvArgs& p, int nkb, int col_last, int r0, int c0, int kc, int wave, int lane) {
  using Stg = PvwStage<WQ>;
  static_assert(Stg::kPerWave == 6 + 2 * WQ, "load q = 4 u + wave: u < 2 rows, u < 6 columns, then tangents");
  const int64_t rsb = (int64_t)nkb * 32;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 3;
  const unsigned piece = (unsigned)(((lane & 7) ^ (((wv & 1) << 2) | (g >> 1))) * 16);
  const int64_t kco = (int64_t)kc * 128;
  const unsigned char* rows = static_cast<const unsigned char*>(p.rows) + (int64_t)r0 * rsb + kco;
  const unsigned char* cols = static_cast<const unsigned char*>(p.cols) + (int64_t)c0 * rsb + kco;
#pragma unroll
  for (int u = 0; u < Stg::kPerWave; ++u) {
    const int q = 4 * u + wv;
    if (u < 2) {
      const int rec = min(r0 + 8 * q + g, p.nr - 1) - r0;
      load_to_lds(rows, (unsigned)(rec * rsb) + piece, dst + q * 1024);
    } else if (u < 6) {
      const int q2 = q - 8;
      const int rec = min(c0 + 8 * q2 + g, col_last) - c0;
      load_to_lds(cols, (unsigned)(rec * rsb) + piece, dst + q * 1024);
    } else {
      const int q3 = q - 24;  // tangent array q3 / 8, records 8 (q3 % 8) ...
      const unsigned char* tan = reinterpret_cast<const unsigned char*>(p.wrec) +
                                 (int64_t)(q3 >> 3) * p.wrec_stride * 16 + (int64_t)r0 * rsb + kco;
      const int rec = min(r0 + 8 * (q3 & 7) + g, p.nr - 1) - r0;
      load_to_lds(tan, (unsigned)(rec * rsb) + piece, dst + q * 1024);
    }
  }
}

template <int PP, int VP, int NOBW, int WQ, bool H>
__global__ __launch_bounds__(kThreads, 1) void k_pv_wide(const PvArgs p, int nkb, int col_last) {
  static_assert(!(H && WQ > 0), "the weighted application keeps bf16 parts");
  using Stg = PvwStage<WQ>;
  constexpr int R = Stg::kRing;
  constexpr int PER = Stg::kPerWave;
  __shared__ __attribute__((aligned(16))) PvwLds<PP, WQ> lds;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int srt = wave & 1;   // row tile of this wave's scores
  const int sch = wave >> 1;  // column half of this wave's scores
  const int ob0 = blockIdx.z * (4 * NOBW) + wave * NOBW;  // this wave's first value block
  const int j0 = blockIdx.y * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int r0 = blockIdx.x * kPvwRows;
  const float e = p.escale;
  const bf16x8 Baug = row_aug(half, 0.0f);

  float mu[2] = {kMuInit, kMuInit};  // lazy row maxima (acc units) of the lane's row in each row tile
  float Sp = 0.0f;                   // partial row sum over this wave's score tiles
  f32x16 O[2][NOBW];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ob = 0; ob < NOBW; ++ob) O[rt][ob] = f32x16{};

  const int nkc = nkb / kGKb;
  const int nblocks = (j1 - j0 + kPvwCols - 1) / kPvwCols;
  const int nstages = nblocks * nkc;
  auto issue = [&](int st) {
    pvw_issue_stage<WQ>(lds.ring[st % R], p, nkb, col_last, r0, j0 + (st / nkc) * kPvwCols, st % nkc, wave, lane);
  };
  // Waits until this wave's loads of stage st have landed, the stages after
  // it up to `last` (at most R - 2 of them) being still in flight.
  auto wait_stage = [&](int st, int last) {
    const int younger = min(last, nstages - 1) - st;
    if (R > 3 && younger >= 2) wait_vmcnt<(R > 3 ? 2 * PER : 0)>();
    else if (younger >= 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
  };
  // operand fragments of a stage (row tile srt, column tiles 2 sch + ct)
  bf16x8 Bs[kGKb], As[kGKb][2], Ws[WQ > 0 ? WQ : 1][kGKb];
  auto read_frags = [&](int st) {
    const unsigned char* rg = lds.ring[st % R];
#pragma unroll
    for (int kb = 0; kb < kGKb; ++kb) {
      const int pos = (((2 * kb + half) ^ ((li >> 1) & 7)) * 16) + li * 128;  // piece 2 kb + h of record 32 t + li
      Bs[kb] = *reinterpret_cast<const bf16x8*>(rg + srt * 32 * 128 + pos);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        As[kb][ct] = *reinterpret_cast<const bf16x8*>(rg + Stg::kColOff + (2 * sch + ct) * 32 * 128 + pos);
      if constexpr (WQ > 0) {
#pragma unroll
        for (int qq = 0; qq < WQ; ++qq)
          Ws[qq][kb] = *reinterpret_cast<const bf16x8*>(rg + Stg::kTanOff + qq * (kPvwRows * 128) + srt * 32 * 128 + pos);
      }
    }
  };
  // Advances the ring past stage st: refills the slot of stage st - 1 (its
  // readers all passed the previous barrier) with stage st + R - 1, waits for
  // this wave's loads of stage st + 1, publishes it and reads its fragments
  // while the MFMAs of stage st still run.
  auto advance = [&](int st) {
    if (st + R - 1 < nstages) issue(st + R - 1);
    if (st + 1 < nstages) wait_stage(st + 1, st + R - 1);
    __syncthreads();
    if (st + 1 < nstages) read_frags(st + 1);
  };

  for (int s2 = 0; s2 < R - 1 && s2 < nstages; ++s2) issue(s2);
  if (nstages > 0) wait_stage(0, R - 2);
  float qoff[2] = {0.0f, 0.0f};
  if constexpr (WQ > 0) {
    if (p.qoff) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) qoff[rt] = p.qoff[min(r0 + rt * 32 + li, p.nr - 1)];
    }
  }
  __syncthreads();
  if (nstages > 0) read_frags(0);
  f32x16 acc[2], accq[2];
  // value fragments of the block's column tiles, one tile ahead (the first
  // tile's loads go out with the block's last K chunk), where the registers
  // allow it; three-part values at four blocks per wave load at their use
  constexpr bool PF = !(VP == 3 && NOBW == 4);
  VTile<NOBW, VP> vb0, vb1;
  // Blocks of 128 columns, each a run of K chunks then the epilogue; the K
  // loop leaves the value accumulators alone, so they stay in their
  // registers across it.
  for (int blk = 0; blk < nblocks; ++blk) {
    const int cb = j0 + blk * kPvwCols;
    acc[0] = f32x16{};
    acc[1] = f32x16{};
    if constexpr (WQ > 0) {
      accq[0] = f32x16{};
      accq[1] = f32x16{};
    }
    for (int kc = 0; kc < nkc; ++kc) {
      if (PF && kc == nkc - 1) {
        load_vtile<NOBW, VP>(vb0, p, min(cb >> 5, col_last >> 5), ob0, lane);
        // keep the loads here, a whole K chunk and the epilogue ahead of their
        // use (the scheduler would otherwise sink them next to the MFMAs)
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kb = 0; kb < kGKb; ++kb) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(As[kb][ct], Bs[kb], acc[ct], 0, 0, 0);
          if constexpr (WQ > 0) {
#pragma unroll
            for (int qq = 0; qq < WQ; ++qq)
              accq[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(As[kb][ct], Ws[qq][kb], accq[ct], 0, 0, 0);
          }
        }
      }
      if (kc + 1 < nkc) advance(blk * nkc + kc);
    }
    {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x8 Aaug = p.bias_col[2 * (int64_t)min(cb + (2 * sch + ct) * 32 + li, col_last) + half];
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aaug, Baug, acc[ct], 0, 0, 0);
      }
      float tm = max3(max16(acc[0]), max16(acc[1]), kMuInit);
      tm = max3(tm, __shfl_xor(tm, 32), tm);
      if (half == 0) lds.tmax[sch][srt][li] = tm;
      __syncthreads();
      // the same lazy shift in every wave: raise a row's maximum only when a
      // term would exceed 2^16 (H: 2^15 with the bias 2^kHalfBias)
      float sc[2];
      bool raised = false;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float t = fmaxf(lds.tmax[0][rt][li], lds.tmax[1][rt][li]);
        const bool raise = e * (t - mu[rt]) > (H ? kHalfLazy : kLazy);
        const float mn = raise ? t : mu[rt];
        sc[rt] = fast_exp2(e * (mu[rt] - mn));
        mu[rt] = mn;
        raised |= raise;
      }
      if (__any(raised)) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[rt][ob][r] *= sc[rt];
        Sp *= sc[srt];
      }
      const float off = H ? fmaf(-e, mu[srt], kHalfBias) : -e * mu[srt];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        if constexpr (H) {
          f16x8 P[PP][2];
          if (p.grad) Sp += pv_probs_h<PP, true>(acc[ct], e, off, P);
          else pv_probs_h<PP, false>(acc[ct], e, off, P);
#pragma unroll
          for (int pp = 0; pp < PP; ++pp)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              lds.P[srt][2 * sch + ct][pp][kb][lane] = __builtin_bit_cast(bf16x8, P[pp][kb]);
        } else {
          bf16x8 P[PP][2];
          if constexpr (WQ > 0) pv_probs_w<PP>(acc[ct], accq[ct], qoff[srt], e, off, P);
          else if (p.grad) Sp += pv_probs<PP, true>(acc[ct], e, off, P);
          else pv_probs<PP, false>(acc[ct], e, off, P);
#pragma unroll
          for (int pp = 0; pp < PP; ++pp)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) lds.P[srt][2 * sch + ct][pp][kb][lane] = P[pp][kb];
        }
      }
      __syncthreads();
      // a column block can overhang the padded columns by up to 3 tiles:
      // those columns are masked, so any zero-valued tile serves, here the
      // last padded one
      constexpr int KMAX = PP > VP ? PP : VP;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        VTile<NOBW, VP>& cur = (ct & 1) ? vb1 : vb0;
        VTile<NOBW, VP>& nxt = (ct & 1) ? vb0 : vb1;
        if constexpr (PF) {
          if (ct + 1 < 4) {
            load_vtile<NOBW, VP>(nxt, p, min((cb >> 5) + ct + 1, col_last >> 5), ob0, lane);
            __builtin_amdgcn_sched_barrier(0);  // issued one tile of MFMAs ahead of their use
          }
        } else {
          load_vtile<NOBW, VP>(cur, p, min((cb >> 5) + ct, col_last >> 5), ob0, lane);
        }
        bf16x8 Pf[2][PP][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int pp = 0; pp < PP; ++pp)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) Pf[rt][pp][kb] = lds.P[rt][ct][pp][kb][lane];
#pragma unroll
        for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int pp = 0; pp < PP; ++pp)
#pragma unroll
              for (int vp = 0; vp < VP; ++vp)
                if (pp + vp < KMAX) {
#pragma unroll
                  for (int kb = 0; kb < 2; ++kb) {
                    if constexpr (H)
                      O[rt][ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, cur.v[ob][vp][kb]),
                                                                         __builtin_bit_cast(f16x8, Pf[rt][pp][kb]),
                                                                         O[rt][ob], 0, 0, 0);
                    else
                      O[rt][ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.v[ob][vp][kb], Pf[rt][pp][kb],
                                                                          O[rt][ob], 0, 0, 0);
                  }
                }
      }
    }
    advance(blk * nkc + nkc - 1);
    // the value accumulators cross the back edge in the accumulation
    // registers (else the compiler carries a vector-register copy of all of
    // them and moves it on every trip)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ob = 0; ob < NOBW; ++ob) asm volatile("" : "+a"(O[rt][ob]));
  }

  // Row sums: the two column halves' partials (both halves of each wave).
  const float Sw = Sp + __shfl_xor(Sp, 32);
  if (half == 0) lds.ssum[sch][srt][li] = Sw;
  __syncthreads();
  float S[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) S[rt] = lds.ssum[0][rt][li] + lds.ssum[1][rt][li];

  constexpr int CW = 4 * NOBW * 32;  // value columns per chunk
  const int z = blockIdx.z;
  const int cbase = z * CW + wave * NOBW * 32;  // this wave's first value column
  if (p.splits == 1) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int i = r0 + rt * 32 + li;
      if (i >= p.nr) continue;
#pragma unroll
      for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cc = cbase + ob * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (cc < p.kv) pv_store(p, i, cc, mu[rt], S[rt], O[rt][ob][r]);
        }
    }
    return;
  }
  // Split partials (mu, S, values), combined by k_pv_merge after the launch.
  const int64_t nslots = (int64_t)p.nchunks * p.splits;
  float2* part_ms = reinterpret_cast<float2*>(p.part);
  float* part_t = p.part + ((2 * nslots * p.nr + 3) & ~(int64_t)3);
  const int64_t slot = (int64_t)z * p.splits + blockIdx.y;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int i = r0 + rt * 32 + li;
    if (i >= p.nr) continue;
    if (wave == 0 && half == 0) part_ms[slot * p.nr + i] = make_float2(mu[rt], S[rt]);
    float* T = part_t + (slot * p.nr + i) * CW + wave * NOBW * 32;
#pragma unroll
    for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(T + ob * 32 + 8 * q + 4 * half) =
            make_float4(O[rt][ob][4 * q], O[rt][ob][4 * q + 1], O[rt][ob][4 * q + 2], O[rt][ob][4 * q + 3]);
  }
}

// Split partials of the transport kernels, combined in split order (bitwise
// repeatable): for element (i, c) of value chunk z, M = max_s M_s and, with
// f_s = 2^(e (M_s - M)), S = sum_s S_s f_s and T = sum_s T_s f_s, then the
// output as in a single-split launch. cw: value columns per chunk.
__global__ __launch_bounds__(256) void k_pv_merge(const PvArgs p, int cw) {
  // four consecutive value columns per thread (cw is a multiple of 8): one
  // 16-byte partial load per split, the split weights formed once per four
  const int64_t nslots = (int64_t)p.nchunks * p.splits;
  const float2* part_ms = reinterpret_cast<const float2*>(p.part);
  const float* part_t = p.part + ((2 * nslots * p.nr + 3) & ~(int64_t)3);
  const int cq = cw >> 2;
  const int64_t total = (int64_t)p.nchunks * p.nr * cq;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int c = (int)(q % cq) * 4;
    const int64_t t = q / cq;
    const int i = (int)(t % p.nr);
    const int z = (int)(t / p.nr);
    const int cc = z * cw + c;
    if (cc >= p.kv) continue;
    const int64_t s0 = (int64_t)z * p.splits * p.nr + i;  // slot (z, 0) of row i
    // (unrolled so that the partials' loads are in flight together; the sums
    // still run in split order)
    float Mt = kMuInit;
#pragma unroll 8
    for (int s2 = 0; s2 < p.splits; ++s2) Mt = fmaxf(Mt, part_ms[s0 + (int64_t)s2 * p.nr].x);
    float St = 0.0f;
    float Tt[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int s2 = 0; s2 < p.splits; ++s2) {
      const int64_t sl = s0 + (int64_t)s2 * p.nr;
      const float2 ms = part_ms[sl];
      const float f = fast_exp2(p.escale * (ms.x - Mt));
      St = fmaf(ms.y, f, St);
      const float4 v = *reinterpret_cast<const float4*>(part_t + sl * cw + c);
      Tt[0] = fmaf(v.x, f, Tt[0]);
      Tt[1] = fmaf(v.y, f, Tt[1]);
      Tt[2] = fmaf(v.z, f, Tt[2]);
      Tt[3] = fmaf(v.w, f, Tt[3]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (cc + u < p.kv) pv_store(p, i, cc + u, Mt, St, Tt[u]);
  }
}

// Largest magnitude of each value column (as float bits; (src - shift) for
// the gradient's points) into vmax, which k_value_max_init zeroed. Maxima of
// non-negative floats order as their bits, so the atomics are exact and the
// result does not depend on their order.
__global__ __launch_bounds__(256) void k_value_max_init(int kv, unsigned* vmax) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < kv) vmax[i] = 0u;
}

// The grid's thread count is a multiple of kv, so each thread stays on one
// column; a workgroup combines its threads' maxima in LDS, then issues one
// global atomic per column.
__global__ __launch_bounds__(256) void k_value_max(const void* src, int src_bf16, int64_t nv, int kv,
                                                   const float* shift, unsigned* vmax) {
  __shared__ unsigned smax[kVmaxCols];
  for (int c = threadIdx.x; c < kv; c += 256) smax[c] = 0u;
  __syncthreads();
  const int64_t total = nv * kv;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cc = (int)(idx % kv);
  unsigned m = 0u;
  for (; idx < total; idx += stride) {
    float v = src_bf16 ? __uint_as_float((unsigned)static_cast<const unsigned short*>(src)[idx] << 16)
                       : static_cast<const float*>(src)[idx];
    if (shift) v -= shift[cc];
    const unsigned bits = __float_as_uint(v) & 0x7FFFFFFFu;
    m = bits > m ? bits : m;
  }
  if (m) atomicMax(&smax[cc], m);
  __syncthreads();
  for (int c = threadIdx.x; c < kv; c += 256)
    if (smax[c]) atomicMax(&vmax[c], smax[c]);
}

// Value fragment (tile t, value block ob, part vp, K block kb) in lane l
// (h = l / 32): the values of index 32 ob + l % 32 at the eight points
// 32 t + 16 kb + 8 (e / 4) + 4 h + e % 4, e = 0..7 -- the column order of a
// score accumulator. Part vp of the three-part bf16 split, or with vmax (the
// half-precision form) of the two-part float16 split of the value times its
// column's scale 2^k (exact); zeros past nv / kv.
__global__ __launch_bounds__(256) void k_pack_values(const void* src, int src_bf16, int64_t nv, int kv,
                                                     const float* shift, int vp_parts, int nobt,
                                                     int64_t ntiles, const unsigned* vmax, bf16x8* out) {
  const int64_t total = ntiles * nobt * vp_parts * 2 * 64;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    int64_t q = idx >> 6;
    const int kb = (int)(q & 1);
    q >>= 1;
    const int vp = (int)(q % vp_parts);
    q /= vp_parts;
    const int ob = (int)(q % nobt);
    const int64_t t = q / nobt;
    const int h = lane >> 5;
    const int cc = ob * 32 + (lane & 31);
    const int k = (vmax && cc < kv) ? half_scale_exp(vmax[cc]) : 0;
    bf16x8 r = {};
    f16x8 rh = {};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t j = t * 32 + kb * 16 + 8 * (e >> 2) + 4 * h + (e & 3);
      float v = 0.0f;
      if (j < nv && cc < kv) {
        if (src_bf16) v = __uint_as_float((unsigned)static_cast<const unsigned short*>(src)[j * kv + cc] << 16);
        else v = static_cast<const float*>(src)[j * kv + cc];
        if (shift) v -= shift[cc];
      }
      if (vmax) {
        const float vs = ldexpf(v, k);
        const _Float16 hi = (_Float16)vs;
        rh[e] = vp == 0 ? hi : (_Float16)(vs - (float)hi);
      } else {
        __bf16 a, b, c;
        split3(v, a, b, c);
        r[e] = vp == 0 ? a : (vp == 1 ? b : c);
      }
    }
    out[idx] = vmax ? __builtin_bit_cast(bf16x8, rh) : r;
  }
}

// Tangent records of the rows for the weighted application, in the GEMM-tiled
// record order: float32 points, one record in the row form of the six-slot
// split (scale 1, so its product with a column record is t_i.y_j to float32
// accuracy); bf16 points, two records holding the bf16 parts of t (t - hi
// rounded again), whose products with the exact bf16 column records sum to
// t_i.y_j within 2^-16. qoff_i = t_i.shift adds back the centering of float32
// columns (q uses the points as given).
__global__ __launch_bounds__(256) void k_pack_tangent(const float* __restrict__ T, int bf16pts, int64_t n, int d,
                                                      int nkb, const float* __restrict__ shift, bf16x8* out,
                                                      int64_t part_stride, float* __restrict__ qoff) {
  const int chunks = nkb * 2;
  const int64_t total = n * chunks;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / chunks;
    const int q = (int)(c % chunks);
    bf16x8 a = {}, b = {};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s2 = q * 8 + e;
      if (bf16pts) {
        if (s2 < d) {
          const float v = T[r * d + s2];
          const __bf16 hi = (__bf16)v;
          a[e] = hi;
          b[e] = (__bf16)(v - (float)hi);
        }
      } else if (s2 < 6 * d) {
        const int k = s2 / 6, w = s2 % 6;
        __bf16 v1, v2, v3;
        split3(T[r * d + k], v1, v2, v3);
        a[e] = (w == 2 || w == 4) ? v2 : (w == 5 ? v3 : v1);
      }
    }
    const int64_t at = r * chunks + (q % nkb) * 2 + q / nkb;
    out[at] = a;
    if (bf16pts) out[part_stride + at] = b;
    if (qoff && q == 0) {
      float acc = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(T[r * d + k], shift ? shift[k] : 0.0f, acc);
      qoff[r] = acc;
    }
  }
}

// Row blocks per wave of the resident kernel: two where registers allow.
constexpr int pv_rb(int nkb, int nob, int vp) { return (nkb <= 4 && nob * vp <= 2) ? 2 : 1; }

// The form, the part counts and the gradient / application choice are
// template arguments (no branch in the tile loop). Instantiated: the half
// form's bf16-point application (1, 2) and gradient (1, 1) and float32-point
// application and gradient (2, 2); the bf16-part form's bf16-point
// application (2, 2), which the Hessian-vector product's CG uses.
template <int NKB, int RB, int NOB, int PP, int VP, bool GRAD, bool H>
bool try_pv_mfma(const PvArgs& a, int pp, int vp, bool half, const dim3& grid, hipStream_t s) {
  if constexpr (pv_rb(NKB, NOB, VP) != RB) {
    return false;
  } else {
    if (pp != PP || vp != VP || half != H || (a.grad != 0) != GRAD) return false;
    k_pv_mfma<NKB, RB, NOB, PP, VP, GRAD, H><<<grid, kThreads, 0, s>>>(a);
    return true;
  }
}

template <int NKB, int RB, int NOB>
hipError_t run_pv_mfma(const PvArgs& a, int pp, int vp, bool half, const dim3& grid, hipStream_t s) {
  if (try_pv_mfma<NKB, RB, NOB, 1, 2, false, true>(a, pp, vp, half, grid, s) ||
      try_pv_mfma<NKB, RB, NOB, 1, 1, true, true>(a, pp, vp, half, grid, s) ||
      try_pv_mfma<NKB, RB, NOB, 2, 2, false, true>(a, pp, vp, half, grid, s) ||
      try_pv_mfma<NKB, RB, NOB, 2, 2, true, true>(a, pp, vp, half, grid, s) ||
      try_pv_mfma<NKB, RB, NOB, 2, 2, false, false>(a, pp, vp, half, grid, s))
    return hipGetLastError();
  return hipErrorInvalidValue;
}

// Emitted though never launched: without it the compiler allocates
// k_pv_gemm8<2, 2, true>'s registers differently and spills more in its
// main loop (P V at n = m = 20k, d = 512 float32: 4.70 -> 5.51 ms).
template __global__ void k_pv_gemm8<3, 3, false>(const PvArgs, int, int);

hipError_t run_pv_gemm8(const PvArgs& a, int nkb, int pp, int vp, bool half, const dim3& grid, hipStream_t s) {
  const int col_last = (int)(mfma_padded_count(a.nc) - 1);
  if (half && pp == 2 && vp == 2) k_pv_gemm8<2, 2, true><<<grid, PvGeo::kNT, 0, s>>>(a, nkb, col_last);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Instantiated: the weighted application (bf16 parts); the half form's
// bf16-point gradient (1, 1) and application (1, 2) and float32-point ones
// (2, 2); the bf16-part form's bf16-point application (2, 2) (the Hessian-
// vector product's CG).
template <int NOBW>
hipError_t run_pv_wide(const PvArgs& a, int nkb, int pp, int vp, bool half, int wq, const dim3& grid,
                       hipStream_t s) {
  const int col_last = (int)(mfma_padded_count(a.nc) - 1);
  if constexpr (NOBW <= 2) {
    if (wq == 1 && pp == 3 && vp == 3 && !half) {  // float32 points: one six-slot tangent record
      k_pv_wide<3, 3, NOBW, 1, false><<<grid, kThreads, 0, s>>>(a, nkb, col_last);
      return hipGetLastError();
    }
    if (wq == 2 && pp == 2 && vp == 1 && !half) {  // bf16 points: two bf16 parts of the tangent
      k_pv_wide<2, 1, NOBW, 2, false><<<grid, kThreads, 0, s>>>(a, nkb, col_last);
      return hipGetLastError();
    }
  }
  if (wq != 0) return hipErrorInvalidValue;
  if (half) {
    if (pp == 1 && vp == 1) k_pv_wide<1, 1, NOBW, 0, true><<<grid, kThreads, 0, s>>>(a, nkb, col_last);
    else if (pp == 1 && vp == 2) k_pv_wide<1, 2, NOBW, 0, true><<<grid, kThreads, 0, s>>>(a, nkb, col_last);
    else if (pp == 2 && vp == 2) k_pv_wide<2, 2, NOBW, 0, true><<<grid, kThreads, 0, s>>>(a, nkb, col_last);
    else return hipErrorInvalidValue;
  } else {
    if (pp == 2 && vp == 2) k_pv_wide<2, 2, NOBW, 0, false><<<grid, kThreads, 0, s>>>(a, nkb, col_last);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NOB>
hipError_t run_pv_gemm(const PvArgs& a, int nkb, int pp, int vp, const dim3& grid, hipStream_t s) {
  // float32 points' applications and gradients of 33-64 values, bf16 points'
  // applications of up to 64 values (their gradients run on the wide kernel)
  if (pp == 3 && vp == 3) k_pv_gemm<NOB, 3, 3><<<grid, kThreads, 0, s>>>(a, nkb);
  else if (pp == 2 && vp == 2) k_pv_gemm<NOB, 2, 2><<<grid, kThreads, 0, s>>>(a, nkb);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

void pv_parts(int dtype, bool grad, bool half_kernel, bool precise, int& pp, int& vp, bool& half) {
  // precise: bf16 points keep two bf16 parts (2^-16) rather than one float16
  // part; float32 points' two float16 parts (2^-22) already match the
  // three-part bf16 split
  half = half_kernel && !(precise && dtype != 0);
  if (half) {  // float16 parts
    pp = dtype == 0 ? 2 : 1;
    vp = (dtype != 0 && grad) ? 1 : 2;
  } else if (dtype == 0) {
    pp = 3;
    vp = 3;
  } else {
    pp = 2;
    vp = grad ? 1 : 2;
  }
}

int pv_nob(bool gemm, int nobt, int vp) {
  // GEMM-tiled, more than two value blocks: the wide kernel, whose four waves
  // carry NOBW blocks each (a chunk of 4 NOBW blocks, up to 512 values).
  if (gemm && nobt > 2) return pv_wide_nob(nobt, vp, false);
  return nobt >= 2 ? 2 : 1;
}

namespace {
// Resident workgroups of the GEMM-tiled kernel carrying nob value blocks.
int pv_gemm_resident(int nob) {
  // Per device and value blocks per chunk, computed once; concurrent first
  // calls compute the same value.
  constexpr int kDevices = 16;
  static std::atomic<int> cached[kDevices][17];
  if (nob < 1 || nob > 16) return 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::atomic<int>* slot = (dev >= 0 && dev < kDevices) ? &cached[dev][nob] : nullptr;
  int v = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    int cus = 0, per_cu = 0;
    hipError_t e = hipErrorInvalidValue;
    if (nob == 1) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pv_gemm<1, 3, 3>, kThreads, 0);
    if (nob == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pv_gemm<2, 3, 3>, kThreads, 0);
    if (nob == 4) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pv_wide<3, 3, 1, 1, false>, kThreads, 0);
    if (nob == 8) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pv_wide<3, 3, 2, 1, false>, kThreads, 0);
    if (nob == 16) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pv_wide<2, 2, 4, 0, false>, kThreads, 0);
    if (e != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    v = per_cu * cus;
    if (slot) slot->store(v, std::memory_order_relaxed);
  }
  return v;
}
}  // namespace

namespace {
// one value block on the GEMM path: the 8-wave tile for float32 points in
// the float16 form (bf16 points stay on the 128 x 128 tile: 0.73 ms there
// at d = 512, n = m = 20k, the same in the float16 form on the 8-wave tile,
// 1.3 ms in bf16 parts)
bool pv_tile8(bool gemm, int nob, int vp, bool half) { return gemm && nob == 1 && vp == 2 && half; }

// Resident workgroups of the 8-wave GEMM-tiled kernel (per device, computed once).
int pv_gemm8_resident() {
  constexpr int kDevices = 16;
  static std::atomic<int> cached[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::atomic<int>* slot = (dev >= 0 && dev < kDevices) ? &cached[dev] : nullptr;
  int v = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    int cus = 0, per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pv_gemm8<2, 2, true>, PvGeo::kNT, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    v = per_cu * cus;
    if (slot) slot->store(v, std::memory_order_relaxed);
  }
  return v;
}
}  // namespace

PassPlan plan_pv(bool gemm, int64_t nr, int64_t nc, int nkb, int nob, int vp, int nchunks, bool half) {
  PassPlan pl{};
  // GEMM-tiled with one value block and float32 points: the 256 x 256 tile
  // of 8 waves (k_pv_gemm8). Its epilogue spills, which only the long K loop
  // of the six-part float32 records amortizes (d = 512: P V 10.1 -> 6.2 ms
  // in bf16 parts, 5.3 -> 4.7 ms in the float16 form, which spills less);
  // bf16 records stay on the 128 x 128 tile.
  const bool tile8 = pv_tile8(gemm, nob, vp, half);
  const bool wide = gemm && nob >= 4;
  pl.rows_per_block = tile8 ? PvGeo::kRows : (wide ? kPvwRows : (gemm ? kGRows : 4 * pv_rb(nkb, nob, vp) * 32));
  pl.row_blocks = (int)((nr + pl.rows_per_block - 1) / pl.rows_per_block);
  if (gemm) {
    int64_t max_splits = nc / 512 > 1 ? nc / 512 : 1;
    if (max_splits > 64) max_splits = 64;
    int64_t cps = 0;
    const int64_t units = (int64_t)pl.row_blocks * (nchunks > 0 ? nchunks : 1);
    pl.splits = (int)round_filling_splits(units, nc, tile8 ? PvGeo::kCols : (wide ? kPvwCols : kGCols),
                                          max_splits, tile8 ? pv_gemm8_resident() : pv_gemm_resident(nob), cps);
    pl.cols_per_split = (int)cps;
    return pl;
  }
  const int64_t target = 2048 / (nchunks > 0 ? nchunks : 1);
  int64_t splits = (target + pl.row_blocks - 1) / pl.row_blocks;
  const int64_t min_cols = 1024;
  const int64_t max_splits = nc / min_cols > 1 ? nc / min_cols : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  const int64_t unit = 64;
  int64_t cps = (nc + splits - 1) / splits;
  cps = (cps + unit - 1) / unit * unit;
  pl.cols_per_split = (int)cps;
  pl.splits = (int)((nc + cps - 1) / cps);
  return pl;
}

hipError_t launch_pv_main(const PvArgs& a, bool gemm, int nkb, int nob, int pp, int vp, bool half,
                          const PassPlan& pl, hipStream_t s) {
  const dim3 grid(pl.row_blocks, pl.splits, a.nchunks);
  if (gemm) {
    if (pv_tile8(gemm, nob, vp, half)) return run_pv_gemm8(a, nkb, pp, vp, half, grid, s);
    if (nob == 1) return run_pv_gemm<1>(a, nkb, pp, vp, grid, s);
    if (nob == 2) return run_pv_gemm<2>(a, nkb, pp, vp, grid, s);
    const int wq = a.wrec ? (pp == 3 ? 1 : 2) : 0;
    if (nob == 4) return run_pv_wide<1>(a, nkb, pp, vp, half, wq, grid, s);
    if (nob == 8) return run_pv_wide<2>(a, nkb, pp, vp, half, wq, grid, s);
    if (nob == 16) return run_pv_wide<4>(a, nkb, pp, vp, half, wq, grid, s);
    return hipErrorInvalidValue;
  }
  const int rb = pv_rb(nkb, nob, vp);
  const int key = nkb * 100 + rb * 10 + nob;
  switch (key) {
    case 111: return run_pv_mfma<1, 1, 1>(a, pp, vp, half, grid, s);
    case 121: return run_pv_mfma<1, 2, 1>(a, pp, vp, half, grid, s);
    case 122: return run_pv_mfma<1, 2, 2>(a, pp, vp, half, grid, s);
    case 112: return run_pv_mfma<1, 1, 2>(a, pp, vp, half, grid, s);
    case 221: return run_pv_mfma<2, 2, 1>(a, pp, vp, half, grid, s);
    case 222: return run_pv_mfma<2, 2, 2>(a, pp, vp, half, grid, s);
    case 211: return run_pv_mfma<2, 1, 1>(a, pp, vp, half, grid, s);
    case 212: return run_pv_mfma<2, 1, 2>(a, pp, vp, half, grid, s);
    case 421: return run_pv_mfma<4, 2, 1>(a, pp, vp, half, grid, s);
    case 422: return run_pv_mfma<4, 2, 2>(a, pp, vp, half, grid, s);
    case 411: return run_pv_mfma<4, 1, 1>(a, pp, vp, half, grid, s);
    case 412: return run_pv_mfma<4, 1, 2>(a, pp, vp, half, grid, s);
    case 811: return run_pv_mfma<8, 1, 1>(a, pp, vp, half, grid, s);
    case 812: return run_pv_mfma<8, 1, 2>(a, pp, vp, half, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pv(const PvArgs& a, bool gemm, int nkb, int nob, int pp, int vp, bool half,
                     const PassPlan& pl, hipStream_t s) {
  if (half && gemm && nob == 2) return hipErrorInvalidValue;  // k_pv_gemm: bf16 parts
  // value partials per (slot, row): a single chunk of the register-resident
  // or the 1-2 block GEMM-tiled kernels keeps only the value width (rounded
  // to 8); the wide kernel writes whole chunks
  PvArgs b = a;
  const int cw = nob * 32;
  const bool wide = gemm && nob >= 4;
  b.pcw = (!wide && a.nchunks == 1 && ((a.kv + 7) & ~7) < cw) ? ((a.kv + 7) & ~7) : cw;
  hipError_t e = launch_pv_main(b, gemm, nkb, nob, pp, vp, half, pl, s);
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t total = (int64_t)b.nchunks * b.nr * (b.pcw / 4);  // four columns per thread
  const int64_t blocks = (total + 255) / 256;
  k_pv_merge<<<(int)(blocks < 16384 ? blocks : 16384), 256, 0, s>>>(b, b.pcw);
  return hipGetLastError();
}

hipError_t launch_pack_tangent(const float* T, bool bf16pts, int64_t n, int d, int nkb, const float* shift,
                               bf16x8* out, int64_t part_stride, float* qoff, hipStream_t s) {
  const int64_t total = n * nkb * 2;
  const int64_t blocks = (total + 255) / 256;
  k_pack_tangent<<<(int)(blocks < 8192 ? blocks : 8192), 256, 0, s>>>(T, bf16pts ? 1 : 0, n, d, nkb, shift, out,
                                                                      part_stride, qoff);
  return hipGetLastError();
}

hipError_t launch_pack_values(const void* src, bool src_bf16, int64_t nv, int kv, const float* shift,
                              int vp, int nobt, int64_t ntiles, unsigned* vmax, bf16x8* out, hipStream_t s) {
  if (vmax) {
    k_value_max_init<<<(kv + 255) / 256, 256, 0, s>>>(kv, vmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (kv < 1 || kv > kVmaxCols) return hipErrorInvalidValue;
    // a grid whose thread count is a multiple of kv: blocks a multiple of kv / gcd(kv, 256)
    int g = kv, r = 256;
    while (r) { const int t = g % r; g = r; r = t; }
    const int64_t unit = kv / g;
    const int64_t total = nv * kv;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256) blocks = 256;
    blocks = blocks / unit * unit;
    if (blocks < unit) blocks = unit;
    k_value_max<<<(int)blocks, 256, 0, s>>>(src, src_bf16 ? 1 : 0, nv, kv, shift, vmax);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t total = ntiles * nobt * vp * 2 * 64;
  const int64_t blocks = (total + 255) / 256;
  k_pack_values<<<(int)(blocks < 8192 ? blocks : 8192), 256, 0, s>>>(src, src_bf16 ? 1 : 0, nv, kv, shift,
                                                                     vp, nobt, ntiles, vmax, out);
  return hipGetLastError();
}

}  // namespace sk
