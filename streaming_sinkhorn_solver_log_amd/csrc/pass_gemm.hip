// pass_gemm.hip -- matrix-core half-pass for wide records (large dimension).
//
// Same arithmetic as the register-resident half-pass (pass_mfma.hip): scores
// p_i . q_j plus the column bias (and, after a side's first pass, minus the
// row shift) come out of v_mfma_f32_32x32x16_bf16, and the vector ALU only
// forms exp2 and sums. For large d the row records no longer fit in
// registers, so both operands stream through LDS in chunks of the K dimension,
// GEMM style: a workgroup of 2 x 2 waves owns 128 rows and sweeps its column
// range in blocks of 128 columns; for each block it runs the K loop (4 K blocks
// per LDS stage, double buffered, one barrier per stage) into 2 x 2 32x32
// accumulators per wave, applies the bias block, and folds the 4096 scores of
// each accumulator tile into per-row sums before the next block. Tiles of
// both operands are re-read once per (row block, column block): the
// n m d (1/128 + 1/128) re-read term of the IO bound (FlashSinkhorn
// replication review, Summary: Theorem 2's n m d^2 / M term, here with
// M ~ 128 records per side in LDS).
#include "sk_internal.h"
#include "sk_mfma.h"
#include "sk_gemm.h"
#include "sk_gemm_dev.h"

#include <math.h>
#include <stdint.h>

namespace sk {
namespace {

using namespace dev;

// One sweep of the workgroup over columns [j0, j1) (j1 - j0 a multiple of 128,
// or ending in the padding). Wave (wr, wc) accumulates rows wr*64 + rb*32 + li
// against columns wc*64 + ct*32 of each block. Ends with a barrier.
template <bool SHIFTED, bool SCALED>
__device__ __attribute__((always_inline)) inline void gemm_sweep(
    const MfmaPassArgs& p, GemmLds& L, int nkb, int j0, int j1, const bf16x8 (&Baug)[2],
    float (&M)[2], float (&S)[2], int wr, int wc, int li, int half) {
  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const int nkc = nkb / kGKb;
  const int nblocks = (j1 - j0 + kGCols - 1) / kGCols;
  const int nstages = nblocks * nkc;
  const int r0 = blockIdx.x * kGRows;
  GemmRegs g;
  gemm_load(g, rows, cols, nkb, p.nr, r0, j0, 0);
  gemm_store(g, L, 0);
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
      bf16x8 A[2], B[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        A[ct] = *reinterpret_cast<const bf16x8*>(&L.cols[buf][(wc * 64 + ct * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        B[rb] = *reinterpret_cast<const bf16x8*>(&L.rows[buf][(wr * 64 + rb * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ct], B[rb], acc[rb][ct], 0, 0, 0);
    }
    if (kc == nkc - 1) {
      // bias block (and row shift), then fold the block's scores into the row sums
      const int cb = j0 + blk * kGCols + wc * 64;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x8 Aaug = p.bias_col[2 * (int64_t)(cb + ct * 32 + li) + half];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aaug, Baug[rb], acc[rb][ct], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          if constexpr (SHIFTED) sum_update<SCALED>(acc[rb][ct], p.escale, S[rb]);
          else lse_update(acc[rb][ct], p.escale, M[rb], S[rb]);
        }
    }
    if (st + 1 < nstages) gemm_store(g, L, buf ^ 1);
    __syncthreads();
  }
}

template <bool SHIFTED, bool SCALED>
__global__ __launch_bounds__(kThreads, 2) void k_lse_gemm(const MfmaPassArgs p, int nkb) {
  __shared__ __attribute__((aligned(16))) GemmLds lds;
  __shared__ float red[kThreads / 64];
  __shared__ float sm_m[2][kGRows];  // per column-wave partials of each row
  __shared__ float sm_s[2][kGRows];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int sp = blockIdx.y;
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int row0 = blockIdx.x * kGRows;

  float M[2], S[2];
  bf16x8 Baug[2];
  float shift_row[2];
  if constexpr (SHIFTED) {
    float dm = -INFINITY;
    for (int q = threadIdx.x; q < p.n_dmax_in; q += kThreads) dm = fmaxf(dm, p.dmax_in[q]);
    const float dmax = block_max(dm, red);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int i = min(row0 + wr * 64 + rb * 32 + li, p.nr - 1);
      shift_row[rb] = p.Lin[i] + dmax;
      Baug[rb] = row_aug(half, -shift_row[rb] / p.escale);
      M[rb] = 0.0f;
      S[rb] = 0.0f;
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      Baug[rb] = row_aug(half, 0.0f);
      M[rb] = -INFINITY;
      S[rb] = 0.0f;
      shift_row[rb] = 0.0f;
    }
  }

  // Per row: (Lm, Ls) with L = Lm + log2 Ls (log2 units), merged over the two
  // column waves and the two halves of each wave; thread t < 128 owns row t.
  auto merge_rows = [&](bool shifted) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float So = __shfl_xor(S[rb], 32);
      float lm, ls;
      if (shifted) {
        lm = shift_row[rb];
        ls = S[rb] + So;
      } else {
        const float Mo = __shfl_xor(M[rb], 32);
        const float Mt = fmaxf(M[rb], Mo);
        const float Me = (Mt == -INFINITY) ? 0.0f : Mt;
        ls = S[rb] * fast_exp2(p.escale * (M[rb] - Me)) + So * fast_exp2(p.escale * (Mo - Me));
        lm = p.escale * Mt;
      }
      if (half == 0) {
        sm_m[wc][wr * 64 + rb * 32 + li] = lm;
        sm_s[wc][wr * 64 + rb * 32 + li] = ls;
      }
    }
    __syncthreads();
  };
  auto row_result = [&](int r, float& lm, float& ls) {
    const float m0 = sm_m[0][r], m1 = sm_m[1][r];
    const float mt = fmaxf(m0, m1);
    const float me = (mt == -INFINITY) ? 0.0f : mt;
    ls = sm_s[0][r] * fast_exp2(m0 - me) + sm_s[1][r] * fast_exp2(m1 - me);
    lm = mt;
  };

  gemm_sweep<SHIFTED, SCALED>(p, lds, nkb, j0, j1, Baug, M, S, wr, wc, li, half);
  merge_rows(SHIFTED);

  const int r = threadIdx.x;
  const int i = row0 + r;
  const bool mine = r < kGRows && i < p.nr;
  float dh = -INFINITY;
  bool need_exact = false;
  float Lr = 0.0f;
  bool bad = false;
  if (p.splits == 1) {
    if (mine) {
      float lm, ls;
      row_result(r, lm, ls);
      Lr = lm + fast_log2(ls);
      bad = SHIFTED && !(ls >= kShiftedFloor);
    }
  } else {
    if (mine) {
      float lm, ls;
      row_result(r, lm, ls);
      store_coherent(&p.part[(int64_t)sp * p.nr + i], make_float2(lm, ls));
    }
    if (!arrive_last(p.counters + blockIdx.x, p.splits)) return;
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
    if (threadIdx.x == 0) atomicExch(p.counters + blockIdx.x, 0u);
  }
  if constexpr (SHIFTED) need_exact = __syncthreads_or(bad);
  if (!need_exact && mine) dh = finish_row_mfma(p, i, Lr);
  if constexpr (SHIFTED) {
    if (need_exact) {
      if (threadIdx.x == 0 && p.exact_count) atomicAdd(p.exact_count, 1u);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        Baug[rb] = row_aug(half, 0.0f);
        M[rb] = -INFINITY;
        S[rb] = 0.0f;
      }
      gemm_sweep<false, SCALED>(p, lds, nkb, 0, p.nc, Baug, M, S, wr, wc, li, half);
      merge_rows(false);
      if (mine) {
        float lm, ls;
        row_result(r, lm, ls);
        dh = finish_row_mfma(p, i, lm + fast_log2(ls));
      }
    }
  }
  const float bmax = block_max(dh, red);
  if (threadIdx.x == 0) p.dmax_out[blockIdx.x] = bmax;
}

}  // namespace

int64_t round_filling_splits(int64_t units, int64_t nc, int64_t unit_cols, int64_t max_splits,
                             int64_t resident, int64_t& cols_per_split) {
  // Workgroups run in rounds of `resident`; a round costs about one split's
  // columns. Take the split count with the fewest column-rounds (ties: fewer
  // splits), so the last round is not left mostly empty.
  if (max_splits < 1) max_splits = 1;
  if (resident < 1) resident = 1;
  int64_t best = 1, best_cps = 0, best_cost = INT64_MAX;
  for (int64_t s = 1; s <= max_splits; ++s) {
    int64_t cps = (nc + s - 1) / s;
    cps = (cps + unit_cols - 1) / unit_cols * unit_cols;
    const int64_t se = (nc + cps - 1) / cps;
    if (se < s) continue;  // same split as a smaller s
    const int64_t rounds = (units * se + resident - 1) / resident;
    const int64_t cost = rounds * cps;
    if (cost < best_cost) {
      best_cost = cost;
      best = se;
      best_cps = cps;
    }
  }
  cols_per_split = best_cps;
  return best;
}

namespace {
int gemm_resident() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0, per_cu = 0, most = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    // the four instantiations share the LDS footprint that binds occupancy
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_gemm<true, true>, kThreads, 0) == hipSuccess)
      most = per_cu;
    if (most < 1) most = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    cached = most * cus;
  }
  return cached;
}
}  // namespace

PassPlan plan_gemm_pass(int64_t nr, int64_t nc) {
  PassPlan pl{};
  pl.rows_per_block = kGRows;
  pl.row_blocks = (int)((nr + kGRows - 1) / kGRows);
  int64_t max_splits = nc / 512 > 1 ? nc / 512 : 1;
  if (max_splits > 64) max_splits = 64;
  int64_t cps = 0;
  pl.splits = (int)round_filling_splits(pl.row_blocks, nc, kGCols, max_splits, gemm_resident(), cps);
  pl.cols_per_split = (int)cps;
  return pl;
}

int gemm_nkb(int dtype, int d) {
  const int slots = (dtype == 1) ? d : 6 * d;
  const int nkb = (slots + 15) / 16;
  return (nkb + kGKb - 1) / kGKb * kGKb;  // whole K chunks
}

hipError_t launch_lse_gemm(const MfmaPassArgs& a, int nkb, bool shifted, bool scaled,
                           const PassPlan& pl, hipStream_t s) {
  const dim3 grid(pl.row_blocks, pl.splits);
  if (shifted) {
    if (scaled) k_lse_gemm<true, true><<<grid, kThreads, 0, s>>>(a, nkb);
    else k_lse_gemm<true, false><<<grid, kThreads, 0, s>>>(a, nkb);
  } else {
    if (scaled) k_lse_gemm<false, true><<<grid, kThreads, 0, s>>>(a, nkb);
    else k_lse_gemm<false, false><<<grid, kThreads, 0, s>>>(a, nkb);
  }
  return hipGetLastError();
}

}  // namespace sk
