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
// Each wave keeps RB blocks of 32 row records in registers for the whole pass
// and streams the column records of its range from memory.
#include "sk_internal.h"
#include "sk_mfma.h"
#include "sk_mfma_dev.h"

#include <math.h>

#include <type_traits>

namespace sk {
namespace {

using namespace dev;

template <int RB, bool SHIFTED, bool SCALED>
__device__ __attribute__((always_inline)) inline void tile_valu(const f32x16 (&acc)[RB], float e,
                                                                float (&M)[RB], float (&S)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (SHIFTED) sum_update<SCALED>(acc[rb], e, S[rb]);
    else lse_update(acc[rb], e, M[rb], S[rb]);
  }
}

// One sweep of a wave over columns [j0, j1). SHIFTED: the row shift is folded
// into Baug and the sums need no running maximum; otherwise online
// max/sum-exp. Each wave streams its column records straight from memory (the
// four waves of a workgroup read the same columns, so the L1 cache serves the
// reuse), keeps two tiles of loads in flight ahead of use, and issues the
// MFMAs of tile t+1 before the exp/sum work of tile t. There is no LDS staging
// and no barrier, so waves never wait for each other.
template <int NKB, int RB, bool SHIFTED, bool SCALED>
__device__ __attribute__((always_inline)) inline void sweep(
    const MfmaPassArgs& p, int j0, int j1, const bf16x8 (&B)[RB][NKB], const bf16x8 (&Baug)[RB],
    float (&M)[RB], float (&S)[RB], int li, int half) {
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const bf16x8* __restrict__ bias = p.bias_col;
  const int ntiles = (j1 - j0 + 31) / 32;
  ColTile<NKB> c0, c1;
  f32x16 acc0[RB], acc1[RB];
  // Prefetch loads run up to four tiles past the range: they read the next
  // range's columns or the padding, and their products are never summed.
  load_tile<NKB>(c0, cols, bias, j0, li, half);
  load_tile<NKB>(c1, cols, bias, j0 + 32, li, half);
  tile_mfma<NKB, RB>(c0, B, Baug, acc0);
  load_tile<NKB>(c0, cols, bias, j0 + 64, li, half);
  for (int t = 0; t < ntiles; t += 2) {
    // here: acc0 = tile t (issued), c1 = tile t+1, c0 = tile t+2 (loads in flight)
    tile_mfma<NKB, RB>(c1, B, Baug, acc1);
    load_tile<NKB>(c1, cols, bias, j0 + (t + 3) * 32, li, half);
    tile_valu<RB, SHIFTED, SCALED>(acc0, p.escale, M, S);
    tile_mfma<NKB, RB>(c0, B, Baug, acc0);
    load_tile<NKB>(c0, cols, bias, j0 + (t + 4) * 32, li, half);
    if (t + 1 < ntiles) tile_valu<RB, SHIFTED, SCALED>(acc1, p.escale, M, S);
  }
}

// LDS-staged variant of the sweep for wide records (NKB >= 4): the workgroup
// stages 64 columns at a time through LDS (double buffered, one barrier per
// stage), so the four waves share one copy of each column record instead of
// each pulling it through the L1 cache.
constexpr int kStageCols = 64;

template <int NKB>
struct StageLds {
  static constexpr int kRow = NKB * 32 + 16;  // padded record row (bytes) against bank conflicts
  unsigned char dat[2][kStageCols * kRow];
  bf16x8 aug[2][2 * kStageCols];             // [buffer][half * 64 + column]
};

template <int CPT>
struct StageRegs {
  u32x4 d[CPT];
  bf16x8 aug;
};

// Thread t moves data chunks t, t + 256, ... and bias chunk t % 128 of a stage.
// Columns past the range read the padding or the next range (never summed).
template <int NKB, int CPT>
__device__ __attribute__((always_inline)) inline void load_stage(
    StageRegs<CPT>& sr, const unsigned char* __restrict__ cols, const bf16x8* __restrict__ bias, int s0) {
  constexpr int CHUNKS = kStageCols * NKB * 2;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    int ch = threadIdx.x + c * kThreads;
    if constexpr (CHUNKS % kThreads != 0) ch = min(ch, CHUNKS - 1);
    const int col = ch / (NKB * 2), part = ch % (NKB * 2);
    sr.d[c] = *reinterpret_cast<const u32x4*>(cols + (int64_t)(s0 + col) * (NKB * 32) + part * 16);
  }
  const int ach = threadIdx.x & (2 * kStageCols - 1);
  sr.aug = bias[2 * (int64_t)(s0 + (ach >> 1)) + (ach & 1)];
}

template <int NKB, int CPT>
__device__ __attribute__((always_inline)) inline void store_stage(const StageRegs<CPT>& sr,
                                                                  StageLds<NKB>& L, int buf) {
  constexpr int CHUNKS = kStageCols * NKB * 2;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * kThreads;
    if (CHUNKS % kThreads == 0 || ch < CHUNKS) {
      const int col = ch / (NKB * 2), part = ch % (NKB * 2);
      *reinterpret_cast<u32x4*>(&L.dat[buf][col * StageLds<NKB>::kRow + part * 16]) = sr.d[c];
    }
  }
  if (threadIdx.x < 2 * kStageCols)
    L.aug[buf][(threadIdx.x & 1) * kStageCols + (threadIdx.x >> 1)] = sr.aug;
}

template <int NKB, int RB, bool SHIFTED, bool SCALED>
__device__ __attribute__((always_inline)) inline void sweep_lds(
    const MfmaPassArgs& p, StageLds<NKB>& L, int j0, int j1, const bf16x8 (&B)[RB][NKB],
    const bf16x8 (&Baug)[RB], float (&M)[RB], float (&S)[RB], int li, int half) {
  constexpr int CPT = (kStageCols * NKB * 2 + kThreads - 1) / kThreads;
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  StageRegs<CPT> sr;
  const int nstages = (j1 - j0 + kStageCols - 1) / kStageCols;
  load_stage<NKB, CPT>(sr, cols, p.bias_col, j0);
  store_stage<NKB, CPT>(sr, L, 0);
  __syncthreads();
  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstages) load_stage<NKB, CPT>(sr, cols, p.bias_col, j0 + (st + 1) * kStageCols);
#pragma unroll
    for (int t = 0; t < kStageCols / 32; ++t) {
      const int col = t * 32 + li;
      ColTile<NKB> ct;
      const bf16x8* arow = reinterpret_cast<const bf16x8*>(&L.dat[buf][col * StageLds<NKB>::kRow]) + half * NKB;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) ct.a[kb] = arow[kb];
      ct.aug = L.aug[buf][half * kStageCols + col];
      f32x16 acc[RB];
      tile_mfma<NKB, RB>(ct, B, Baug, acc);
      tile_valu<RB, SHIFTED, SCALED>(acc, p.escale, M, S);
    }
    if (st + 1 < nstages) store_stage<NKB, CPT>(sr, L, buf ^ 1);
    __syncthreads();
  }
}

// Per record width, the sweep that serves it best: narrow records stream
// per wave, wide records are staged through LDS.
template <int NKB>
constexpr bool kUseLds = NKB >= 4;

template <int NKB>
struct SweepLds {
  StageLds<NKB> s;
};
struct NoLds {};

// One half-pass. SHIFTED (every pass after a side's first): the row shift
// M_i = L_i(previous pass) + max_j (change of h_j since then) bounds every
// term by 1, so the sum cannot overflow; a row whose sum falls below 2^-60
// (shift far too high) is recomputed by an exact online-max sweep over all
// columns, done by the workgroup that completes the row's block.
template <int NKB, int RB, bool SHIFTED, bool SCALED>
__global__ __launch_bounds__(kThreads, 2) void k_lse_mfma(const MfmaPassArgs p) {
  constexpr int RSB = NKB * 32;
  constexpr int ROWS = 4 * RB * 32;
  __shared__ float red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) std::conditional_t<kUseLds<NKB>, StageLds<NKB>, NoLds> lds;

  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int sp = blockIdx.y;
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int row_base = blockIdx.x * ROWS + wave * (RB * 32);

  bf16x8 B[RB][NKB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = row_base + rb * 32 + li;
    const bf16x8* rec = reinterpret_cast<const bf16x8*>(rows + (int64_t)min(i, p.nr - 1) * RSB) + half * NKB;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) B[rb][kb] = rec[kb];
  }
  float M[RB], S[RB];
  bf16x8 Baug[RB];
  float shift_row[RB];
  if constexpr (SHIFTED) {
    // largest change of a column bias since this side's previous pass
    float dm = -INFINITY;
    for (int q = threadIdx.x; q < p.n_dmax_in; q += kThreads) dm = fmaxf(dm, p.dmax_in[q]);
    const float dmax = block_max(dm, red);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = min(row_base + rb * 32 + li, p.nr - 1);
      shift_row[rb] = p.Lin[i] + dmax;  // log2 units
      Baug[rb] = row_aug(half, -shift_row[rb] / p.escale);
      M[rb] = 0.0f;
      S[rb] = 0.0f;
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      Baug[rb] = row_aug(half, 0.0f);
      M[rb] = -INFINITY;
      S[rb] = 0.0f;
      shift_row[rb] = 0.0f;
    }
  }

  if constexpr (kUseLds<NKB>) sweep_lds<NKB, RB, SHIFTED, SCALED>(p, lds, j0, j1, B, Baug, M, S, li, half);
  else sweep<NKB, RB, SHIFTED, SCALED>(p, j0, j1, B, Baug, M, S, li, half);

  // Per row (lanes of half 0): (Lm, Ls) with L = Lm + log2 Ls, Lm in log2 units.
  float Lm[RB], Ls[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float So = __shfl_xor(S[rb], 32);
    if constexpr (SHIFTED) {
      Ls[rb] = S[rb] + So;
      Lm[rb] = shift_row[rb];
    } else {
      const float Mo = __shfl_xor(M[rb], 32);
      const float Mt = fmaxf(M[rb], Mo);
      const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
      Ls[rb] = S[rb] * fast_exp2(p.escale * (M[rb] - Me)) + So * fast_exp2(p.escale * (Mo - Me));
      Lm[rb] = p.escale * Mt;
    }
  }

  float dh = -INFINITY;  // this thread's largest bias change over the rows it finishes
  bool need_exact = false;
  if (p.splits == 1) {
    bool bad = false;
    if constexpr (SHIFTED) {
      if (half == 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          bad |= (row_base + rb * 32 + li < p.nr) && !(Ls[rb] >= kShiftedFloor);
      need_exact = __syncthreads_or(bad);
    }
    if (!need_exact && half == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int i = row_base + rb * 32 + li;
        if (i < p.nr) dh = fmaxf(dh, finish_row_mfma(p, i, Lm[rb] + fast_log2(Ls[rb])));
      }
    }
  } else {
    if (half == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int i = row_base + rb * 32 + li;
        if (i < p.nr) p.part[(int64_t)sp * p.nr + i] = make_float2(Lm[rb], Ls[rb]);
      }
    }
    if (!arrive_last(p.counters + blockIdx.x, p.splits)) return;
    // The completing workgroup merges the splits of its rows in split order.
    float Lr = 0.0f;
    bool bad = false;
    const int i = blockIdx.x * ROWS + (int)threadIdx.x;
    const bool mine = (int)threadIdx.x < ROWS && i < p.nr;
    if (mine) {
      float Mt = -INFINITY;
      for (int s2 = 0; s2 < p.splits; ++s2) Mt = fmaxf(Mt, load_coherent(&p.part[(int64_t)s2 * p.nr + i].x));
      const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
      float St = 0.0f;
      for (int s2 = 0; s2 < p.splits; ++s2) {
        const float Mp = load_coherent(&p.part[(int64_t)s2 * p.nr + i].x);
        const float Sp = load_coherent(&p.part[(int64_t)s2 * p.nr + i].y);
        St = fmaf(Sp, fast_exp2(Mp - Me), St);
      }
      Lr = Mt + fast_log2(St);
      bad = SHIFTED && !(St >= kShiftedFloor);
    }
    if constexpr (SHIFTED) need_exact = __syncthreads_or(bad);
    if (!need_exact && mine) dh = finish_row_mfma(p, i, Lr);
    if (threadIdx.x == 0) atomicExch(p.counters + blockIdx.x, 0u);
  }

  if constexpr (SHIFTED) {
    if (need_exact) {
      // Exact recomputation of this workgroup's rows over all columns.
      if (threadIdx.x == 0 && p.exact_count) atomicAdd(p.exact_count, 1u);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        Baug[rb] = row_aug(half, 0.0f);
        M[rb] = -INFINITY;
        S[rb] = 0.0f;
      }
      if constexpr (kUseLds<NKB>) sweep_lds<NKB, RB, false, SCALED>(p, lds, 0, p.nc, B, Baug, M, S, li, half);
      else sweep<NKB, RB, false, SCALED>(p, 0, p.nc, B, Baug, M, S, li, half);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float So = __shfl_xor(S[rb], 32);
        const float Mo = __shfl_xor(M[rb], 32);
        const float Mt = fmaxf(M[rb], Mo);
        const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
        const float St = S[rb] * fast_exp2(p.escale * (M[rb] - Me)) + So * fast_exp2(p.escale * (Mo - Me));
        const int i = row_base + rb * 32 + li;
        if (half == 0 && i < p.nr) dh = fmaxf(dh, finish_row_mfma(p, i, p.escale * Mt + fast_log2(St)));
      }
    }
  }
  const float bmax = block_max(dh, red);
  if (threadIdx.x == 0) p.dmax_out[blockIdx.x] = bmax;
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
                                                        float* hval, float log2e_over_eps,
                                                        float bias_scale) {
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
  const float h = kLog2e * l + (pv - nrm) * log2e_over_eps;
  hval[r] = h;
  write_bias_record(bias + 2 * r, h * bias_scale);
}

// Masked padding columns [n, n_pad) of a side: zero records, masked bias in both buffers.
__global__ __launch_bounds__(256) void k_pad_columns(int64_t n, int64_t n_pad, int nkb, bf16x8* col_rec,
                                                     bf16x8* bias0, bf16x8* bias1) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)nkb * 2;
  if (t < (n_pad - n) * per) col_rec[n * per + t] = bf16x8{};
  if (t < (n_pad - n) * 2) {
    const int64_t q = n * 2 + t;
    bf16x8 v = {};
    if ((q & 1) == 0) {
      v[0] = (__bf16)kMaskedBias;
      v[3] = (__bf16)1.0f;
      v[4] = (__bf16)1.0f;
      v[5] = (__bf16)1.0f;
    }
    bias0[q] = v;
    bias1[q] = v;
  }
}

template <int NKB, int RB>
hipError_t run_lse(const MfmaPassArgs& a, bool shifted, bool scaled, const PassPlan& pl, hipStream_t s) {
  const dim3 grid(pl.row_blocks, pl.splits);
  if (shifted) {
    if (scaled) k_lse_mfma<NKB, RB, true, true><<<grid, kThreads, 0, s>>>(a);
    else k_lse_mfma<NKB, RB, true, false><<<grid, kThreads, 0, s>>>(a);
  } else {
    if (scaled) k_lse_mfma<NKB, RB, false, true><<<grid, kThreads, 0, s>>>(a);
    else k_lse_mfma<NKB, RB, false, false><<<grid, kThreads, 0, s>>>(a);
  }
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

int64_t mfma_padded_count(int64_t n) { return (n + 31) / 32 * 32 + 5 * 32; }

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
  cps = (cps + 63) / 64 * 64;  // whole 64-column stages: a split never reads into the next one
  pl.cols_per_split = (int)cps;
  pl.splits = (int)((nc + cps - 1) / cps);
  return pl;
}

hipError_t launch_lse_mfma(const MfmaPassArgs& a, int nkb, bool shifted, bool scaled,
                           const PassPlan& pl, hipStream_t s) {
  switch (nkb) {
    case 1: return run_lse<1, 2>(a, shifted, scaled, pl, s);
    case 2: return run_lse<2, 2>(a, shifted, scaled, pl, s);
    case 4: return run_lse<4, 2>(a, shifted, scaled, pl, s);
    case 8: return run_lse<8, 1>(a, shifted, scaled, pl, s);
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
    const int64_t npad = mfma_padded_count(side->n);
    const int64_t pad_work = (npad - side->n) * nkb * 2;
    k_pad_columns<<<(int)((pad_work + 255) / 256), 256, 0, s>>>(side->n, npad, nkb, side->col_rec,
                                                                side->bias, side->bias_alt);
    k_prep_side_mfma<<<(int)((side->n + 255) / 256), 256, 0, s>>>(
        side->pts, dtype, side->n, d, sh, side->w, side->pot, side->pot_zero, side->alpha, side->lw,
        side->bias, side->hval, log2e_over_eps, mfma_bias_scale(dtype, c2));
  }
  return hipGetLastError();
}

}  // namespace sk
