// pass_mfma.hip -- matrix-core half-pass for moderate dimension.
//
// The biased score of a (row i, column j) pair is a dot product plus a column
// bias (FlashSinkhorn replication review, Summary: the cost has the form
// alpha_i + beta_j - Q_i.K_j, so the update is a row-wise LSE of biased
// dot-product scores). Here both parts run on the MFMA units:
//
//   acc_ij = s * p_i . q_j + h_j / e         (exponent in log2 units: e * acc)
//
// where c2 = 2 log2(e) / eps and (s, e) = (c2, 1) for float32 points (c2 is
// folded into the row records before they are split) or (1, c2) for bf16
// points (records stay exact, the bias is stored divided by c2).
// with v_mfma_f32_32x32x16_bf16. Points are packed once per call into "records"
// of bf16 slots whose slot-wise products sum to the dot product:
//   * bf16 storage: slot k holds coordinate k (exact);
//   * float32 storage: each coordinate v is split as v1 + v2 + v3 (three bf16,
//     v1 = bf16(v), v2 = bf16(v - v1), v3 = bf16(v - v1 - v2)); the row record
//     holds (x1, x1, x2, x1, x2, x3) and the column record (y1, y2, y1, y3, y2,
//     y1), so the slot products are the six terms of (x1+x2+x3)(y1+y2+y3) down
//     to relative order 2^-24, float32 accuracy.
// The column bias rides in one extra K block: the column side holds the three
// bf16 parts of h~_j, the row side holds ones. The vector ALU is left with the
// per-pair work the log-sum-exp itself needs: a running maximum, one fma into
// the base-2 exponent, one exp2 and one add.
//
// MFMA layout (32x32x16, wave64): lane l (half h = l/32, li = l%32) supplies
// A[row li][k = 8h..8h+7] and B[k = 8h..8h+7][col li]; the accumulator holds
// D[row 8(r/4) + 4h + r%4][col li] in register r. Columns of the transport
// problem are the MFMA rows (A) and rows are the MFMA columns (B), so each lane
// accumulates 16 column scores of one row in registers, and the two halves of
// the wave are merged once at the end. Record slot s is MFMA k-slot
// (s mod 8) of K block (s / 8) mod NKB in half s / (8 NKB): each lane loads its
// half of a record with contiguous 16-byte loads.
//
// Column records (and their bias blocks) are staged through LDS, double
// buffered, 64 columns per stage; each wave keeps RB blocks of 32 row records
// in registers for the whole pass.
#include "sk_internal.h"
#include "sk_mfma.h"

#include <math.h>

namespace sk {
namespace {

constexpr int kStageCols = 64;
constexpr float kMaskedBias = -1.0e30f;  // bias of a column that contributes nothing

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ T load_coherent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool arrive_last(unsigned* counter, int splits) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1u) == (unsigned)(splits - 1));
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// Three-part bf16 split of v (v ~= hi + mid + lo to float32 precision).
__device__ __forceinline__ void split3(float v, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = (__bf16)v;
  const float r1 = v - (float)hi;
  mid = (__bf16)r1;
  lo = (__bf16)(r1 - (float)mid);
}

// Bias record of one column: half 0 = (hi, mid, lo, 0...), half 1 = zeros.
__device__ __forceinline__ void write_bias_record(bf16x8* rec, float htilde) {
  float v = htilde < kMaskedBias ? kMaskedBias : htilde;  // -inf (zero weight) -> masked; NaN kept
  bf16x8 h0 = {}, h1 = {};
  __bf16 a, b, c;
  split3(v, a, b, c);
  h0[0] = a;
  h0[1] = b;
  h0[2] = c;
  rec[0] = h0;
  rec[1] = h1;
}

__device__ __forceinline__ void finish_row_mfma(const MfmaPassArgs& p, int i, float L) {
  const float al = p.alpha[i];
  float v = fmaf(p.neg_eps_ln2, L, al);
  if (p.symmetric) v = 0.5f * (p.pot[i] + v);
  p.pot[i] = v;
  const float h = fmaf(kLog2e, p.lw[i], (v - al) * p.log2e_over_eps);
  write_bias_record(p.bias_out + 2 * (int64_t)i, h * p.bias_scale);
  if (p.Lout) p.Lout[i] = L;
}

// Online update of a lane's running (M, S) with one 32x32 tile (16 scores per lane).
// M is in accumulator units; the exponent of a score is e * (acc - M).
// max(a, b, c) in one instruction. Written as inline assembly because the
// compiler otherwise quiets each MFMA result before a max (IEEE mode), which
// costs an extra instruction per score; a NaN score still reaches the sum
// through exp2 and propagates.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ void lse_update(const f32x16& acc, float c2, float& M, float& S) {
  // c2 here is the exponent scale e
  const float m1 = max3(acc[0], acc[1], acc[2]);
  const float m2 = max3(acc[3], acc[4], acc[5]);
  const float m3 = max3(acc[6], acc[7], acc[8]);
  const float m4 = max3(acc[9], acc[10], acc[11]);
  const float m5 = max3(acc[12], acc[13], acc[14]);
  const float Mn = max3(max3(m1, m2, m3), max3(m4, m5, acc[15]), M);
  const bool valid = Mn > 0.5f * kMaskedBias;  // some real (unmasked) column seen
  const float Me = valid ? Mn : 0.0f;
  const float off = -c2 * Me;
  const float scale = fast_exp2(fmaf(M, c2, off));  // M = -inf -> 0
  float s0 = fast_exp2(fmaf(acc[0], c2, off));
  float s1 = fast_exp2(fmaf(acc[1], c2, off));
  float s2 = fast_exp2(fmaf(acc[2], c2, off));
  float s3 = fast_exp2(fmaf(acc[3], c2, off));
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    s0 += fast_exp2(fmaf(acc[r + 0], c2, off));
    s1 += fast_exp2(fmaf(acc[r + 1], c2, off));
    s2 += fast_exp2(fmaf(acc[r + 2], c2, off));
    s3 += fast_exp2(fmaf(acc[r + 3], c2, off));
  }
  S = fmaf(S, scale, (s0 + s1) + (s2 + s3));
  M = valid ? Mn : M;
}

// Registers holding one stage of column records in flight (global -> LDS).
template <int CPT>
struct StageRegs {
  u32x4 d[CPT];
  bf16x8 aug;
};

// Thread t moves data chunks t, t + 256, ... and bias chunk t % 128 of a stage.
// Loads are unconditional (indices clamped into range) so the staged values
// stay in registers while the current stage is computed; a column past the end
// of the range gets the masked bias, which makes its terms zero.
template <int NKB, int CPT>
__device__ __attribute__((always_inline)) inline void load_stage(
    StageRegs<CPT>& sr, const unsigned char* __restrict__ cols, const bf16x8* __restrict__ bias,
    int s0, int j1, const bf16x8& masked) {
  constexpr int RSB = NKB * 32;
  constexpr int CHUNKS = kStageCols * NKB * 2;
  constexpr int ACHUNKS = kStageCols * 2;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    int ch = threadIdx.x + c * kThreads;
    if constexpr (CHUNKS % kThreads != 0) ch = min(ch, CHUNKS - 1);
    const int col = ch / (NKB * 2), part = ch % (NKB * 2);
    const int j = min(s0 + col, j1 - 1);
    sr.d[c] = *reinterpret_cast<const u32x4*>(cols + (int64_t)j * RSB + part * 16);
  }
  const int ach = threadIdx.x & (ACHUNKS - 1);
  const int j = s0 + (ach >> 1);
  const bf16x8 v = bias[2 * (int64_t)min(j, j1 - 1) + (ach & 1)];
  sr.aug = (j < j1) ? v : masked;
}

template <int NKB, int CPT>
__device__ __attribute__((always_inline)) inline void store_stage(const StageRegs<CPT>& sr,
                                                                  unsigned char* dat, bf16x8* aug) {
  constexpr int LDS_ROW = NKB * 32 + 16;
  constexpr int CHUNKS = kStageCols * NKB * 2;
  constexpr int ACHUNKS = kStageCols * 2;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * kThreads;
    if (CHUNKS % kThreads == 0 || ch < CHUNKS) {
      const int col = ch / (NKB * 2), part = ch % (NKB * 2);
      *reinterpret_cast<u32x4*>(dat + col * LDS_ROW + part * 16) = sr.d[c];
    }
  }
  if (threadIdx.x < ACHUNKS) aug[threadIdx.x] = sr.aug;
}

template <int NKB, int RB>
__global__ __launch_bounds__(kThreads, 2) void k_lse_mfma(const MfmaPassArgs p) {
  constexpr int RS = NKB * 16;                 // bf16 slots per record (both halves)
  constexpr int RSB = RS * 2;                  // bytes per record
  constexpr int LDS_ROW = RSB + 16;            // padded LDS row (bytes) against bank conflicts
  constexpr int CHUNKS = kStageCols * NKB * 2; // 16-byte chunks of column data per stage
  constexpr int ACHUNKS = kStageCols * 2;      // 16-byte chunks of bias records per stage
  constexpr int CPT = (CHUNKS + kThreads - 1) / kThreads;
  static_assert(ACHUNKS <= kThreads, "bias chunks: one per thread");

  __shared__ __attribute__((aligned(16))) unsigned char lds_dat[2][kStageCols * LDS_ROW];
  __shared__ __attribute__((aligned(16))) bf16x8 lds_aug[2][kStageCols * 2];

  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const bf16x8* __restrict__ bias = p.bias_col;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int sp = blockIdx.y;
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int row_base = blockIdx.x * (4 * RB * 32) + wave * (RB * 32);

  // Row operands (B): this lane's half of the records of rows row_base + rb*32 + li.
  bf16x8 B[RB][NKB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = row_base + rb * 32 + li;
    const bf16x8* rec = reinterpret_cast<const bf16x8*>(rows + (int64_t)min(i, p.nr - 1) * RSB) + half * NKB;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) B[rb][kb] = rec[kb];
  }
  bf16x8 Baug = {};
  if (half == 0) {
    Baug[0] = (__bf16)1.0f;
    Baug[1] = (__bf16)1.0f;
    Baug[2] = (__bf16)1.0f;
  }
  float M[RB], S[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    M[rb] = -INFINITY;
    S[rb] = 0.0f;
  }

  StageRegs<CPT> sr;
  bf16x8 masked = {};
  if ((threadIdx.x & 1) == 0) masked[0] = (__bf16)kMaskedBias;

  const int nstages = (j1 - j0 + kStageCols - 1) / kStageCols;
  load_stage<NKB, CPT>(sr, cols, bias, j0, j1, masked);
  store_stage<NKB, CPT>(sr, &lds_dat[0][0], &lds_aug[0][0]);
  __syncthreads();
  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstages) load_stage<NKB, CPT>(sr, cols, bias, j0 + (st + 1) * kStageCols, j1, masked);
#pragma unroll
    for (int t = 0; t < kStageCols / 32; ++t) {
      const int col = t * 32 + li;
      bf16x8 A[NKB];
      const bf16x8* arow = reinterpret_cast<const bf16x8*>(&lds_dat[buf][col * LDS_ROW]) + half * NKB;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) A[kb] = arow[kb];
      const bf16x8 Aaug = lds_aug[buf][2 * col + half];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x16 acc = {};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[kb], B[rb][kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aaug, Baug, acc, 0, 0, 0);
        lse_update(acc, p.escale, M[rb], S[rb]);
      }
    }
    if (st + 1 < nstages) store_stage<NKB, CPT>(sr, &lds_dat[buf ^ 1][0], &lds_aug[buf ^ 1][0]);
    __syncthreads();
  }

  // Merge the two halves of each row (lanes li and li + 32), convert to log2 units.
  float Lm[RB], Ls[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float Mo = __shfl_xor(M[rb], 32);
    const float So = __shfl_xor(S[rb], 32);
    const float Mt = fmaxf(M[rb], Mo);
    const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
    Ls[rb] = S[rb] * fast_exp2(p.escale * (M[rb] - Me)) + So * fast_exp2(p.escale * (Mo - Me));
    Lm[rb] = p.escale * Mt;
  }

  if (p.splits == 1) {
    if (half == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int i = row_base + rb * 32 + li;
        if (i < p.nr) finish_row_mfma(p, i, Lm[rb] + fast_log2(Ls[rb]));
      }
    }
    return;
  }
  if (half == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = row_base + rb * 32 + li;
      if (i < p.nr) p.part[(int64_t)sp * p.nr + i] = make_float2(Lm[rb], Ls[rb]);
    }
  }
  if (!arrive_last(p.counters + blockIdx.x, p.splits)) return;
  // The completing workgroup merges the splits of its 4 * RB * 32 rows in split order.
  for (int r = threadIdx.x; r < 4 * RB * 32; r += kThreads) {
    const int i = blockIdx.x * (4 * RB * 32) + r;
    if (i >= p.nr) continue;
    float Mt = -INFINITY;
    for (int s2 = 0; s2 < p.splits; ++s2) Mt = fmaxf(Mt, load_coherent(&p.part[(int64_t)s2 * p.nr + i].x));
    const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
    float St = 0.0f;
    for (int s2 = 0; s2 < p.splits; ++s2) {
      const float Mp = load_coherent(&p.part[(int64_t)s2 * p.nr + i].x);
      const float Sp = load_coherent(&p.part[(int64_t)s2 * p.nr + i].y);
      St = fmaf(Sp, fast_exp2(Mp - Me), St);
    }
    finish_row_mfma(p, i, Mt + fast_log2(St));
  }
  if (threadIdx.x == 0) atomicExch(p.counters + blockIdx.x, 0u);
}

// ---------------------------------------------------------------- record prep
// Slot s of a record: data slots first (coordinate-major), then zeros.
// bf16 storage: one slot per coordinate. float32 storage: six slots per coordinate.
__global__ __launch_bounds__(256) void k_pack_records(const void* pts, int dtype, int64_t n, int d,
                                                      const float* shift, int nkb, float c2,
                                                      bf16x8* row_rec, bf16x8* col_rec) {
  const int chunks = nkb * 2;  // 16-byte chunks per record
  const int64_t total = n * chunks;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / chunks;
    const int q = (int)(c % chunks);
    bf16x8 rv = {}, cv = {};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = q * 8 + e;
      if (dtype == 1) {
        if (s < d) {
          const unsigned short bits = static_cast<const unsigned short*>(pts)[r * d + s];
          const __bf16 v = __builtin_bit_cast(__bf16, bits);
          rv[e] = v;
          cv[e] = v;
        }
      } else if (s < 6 * d) {
        const int k = s / 6, w = s % 6;
        float v = static_cast<const float*>(pts)[r * d + k];
        if (shift) v -= shift[k];
        __bf16 v1, v2, v3, u1, u2, u3;
        split3(c2 * v, v1, v2, v3);  // row form carries the exponent scale
        split3(v, u1, u2, u3);
        // products (row x col): x1y1, x1y2, x2y1, x1y3, x2y2, x3y1
        rv[e] = (w == 2 || w == 4) ? v2 : (w == 5 ? v3 : v1);
        cv[e] = (w == 1 || w == 4) ? u2 : (w == 3 ? u3 : u1);
      }
    }
    row_rec[c] = rv;
    col_rec[c] = cv;
  }
}

// Norms (of the values the records represent), log-weights, starting potentials
// and the initial bias records. One thread per point.
__global__ __launch_bounds__(256) void k_prep_side_mfma(const void* pts, int dtype, int64_t n, int d,
                                                        const float* shift, const float* w,
                                                        const float* pot, float* pot_zero,
                                                        float* alpha, float* lw, bf16x8* bias,
                                                        float log2e_over_eps, float bias_scale) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  float nrm = 0.0f;
  for (int k = 0; k < d; ++k) {
    float v;
    if (dtype == 1) {
      const unsigned short bits = static_cast<const unsigned short*>(pts)[r * d + k];
      v = __uint_as_float(static_cast<unsigned>(bits) << 16);
    } else {
      v = static_cast<const float*>(pts)[r * d + k];
      if (shift) v -= shift[k];
    }
    nrm = fmaf(v, v, nrm);
  }
  const float l = logf(w[r]);
  const float pv = pot ? pot[r] : 0.0f;
  if (pot_zero) pot_zero[r] = 0.0f;
  alpha[r] = nrm;
  lw[r] = l;
  write_bias_record(bias + 2 * r, (kLog2e * l + (pv - nrm) * log2e_over_eps) * bias_scale);
}

template <int NKB, int RB>
hipError_t run_lse(const MfmaPassArgs& a, const PassPlan& pl, hipStream_t s) {
  k_lse_mfma<NKB, RB><<<dim3(pl.row_blocks, pl.splits), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int mfma_nkb(int dtype, int d) {
  const int slots = (dtype == 1) ? d : 6 * d;
  const int nkb = (slots + 15) / 16;
  if (nkb <= 1) return 1;
  if (nkb <= 2) return 2;
  if (nkb <= 4) return 4;
  if (nkb <= 8) return 8;
  return 0;  // not served by the register-resident kernel
}

int mfma_rb(int nkb) { return nkb <= 4 ? 2 : 1; }

PassPlan plan_mfma_pass(int64_t nr, int64_t nc, int nkb) {
  PassPlan pl;
  pl.rows_per_block = 4 * mfma_rb(nkb) * 32;
  pl.row_blocks = (int)((nr + pl.rows_per_block - 1) / pl.rows_per_block);
  const int64_t target = 2048;
  int64_t splits = (target + pl.row_blocks - 1) / pl.row_blocks;
  const int64_t max_splits = nc / 1024 > 1 ? nc / 1024 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  int64_t cps = (nc + splits - 1) / splits;
  cps = (cps + kStageCols - 1) / kStageCols * kStageCols;
  pl.cols_per_split = (int)cps;
  pl.splits = (int)((nc + cps - 1) / cps);
  return pl;
}

hipError_t launch_lse_mfma(const MfmaPassArgs& a, int nkb, const PassPlan& pl, hipStream_t s) {
  switch (nkb) {
    case 1: return run_lse<1, 2>(a, pl, s);
    case 2: return run_lse<2, 2>(a, pl, s);
    case 4: return run_lse<4, 2>(a, pl, s);
    case 8: return run_lse<8, 1>(a, pl, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prep_mfma(const MfmaPrepSide& xs, const MfmaPrepSide& ys, int dtype, int d,
                            int nkb, bool center, double* centroid_part, float* shift,
                            unsigned* counters, int n_counters, float log2e_over_eps,
                            float c2, hipStream_t s) {
  const float* sh = nullptr;
  if (center && dtype == 0) {
    hipError_t e = launch_centroid(xs.pts, xs.n, ys.pts, ys.n, dtype, d, centroid_part, shift, s);
    if (e != hipSuccess) return e;
    sh = shift;
  }
  hipError_t ez = launch_zero_u32(counters, n_counters, s);
  if (ez != hipSuccess) return ez;
  for (const MfmaPrepSide* side : {&xs, &ys}) {
    const int64_t chunks = side->n * nkb * 2;
    const int blocks = (int)((chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096);
    k_pack_records<<<blocks, 256, 0, s>>>(side->pts, dtype, side->n, d, sh, nkb, c2,
                                          side->row_rec, side->col_rec);
    k_prep_side_mfma<<<(int)((side->n + 255) / 256), 256, 0, s>>>(
        side->pts, dtype, side->n, d, sh, side->w, side->pot, side->pot_zero, side->alpha, side->lw,
        side->bias, log2e_over_eps, mfma_bias_scale(dtype, c2));
  }
  return hipGetLastError();
}

}  // namespace sk
