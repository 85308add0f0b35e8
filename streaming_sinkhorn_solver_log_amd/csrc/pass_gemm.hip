// pass_gemm.hip -- matrix-core half-pass for wide records (large dimension).
//
// Same arithmetic as the register-resident half-pass (pass_mfma.hip): scores
// p_i . q_j plus the column bias (and, after a side's first pass, minus the
// row shift) come out of v_mfma_f32_32x32x16_bf16, and the vector ALU only
// forms exp2 and sums. For large d the row records no longer fit in
// registers, so both operands stream through LDS in chunks of the K dimension,
// GEMM style: a workgroup of 2 x 2 waves owns a block of rows and sweeps its
// column range in column blocks; for each block it runs the K loop (4 K blocks
// per LDS stage, double buffered, one barrier per stage) into the waves'
// 32x32 accumulators, applies the bias block, and folds the scores into
// per-row sums before the next block. Tiles of both operands are re-read once
// per (row block, column block): the n m d (1/R + 1/C) re-read term of the IO
// bound (FlashSinkhorn replication review, Summary: Theorem 2's n m d^2 / M
// term, here with M ~ R + C records in LDS).
//
// Each MFMA of a 2 x 2 wave tile needs one 1 KB LDS fragment; measured on
// gfx950, a register/LDS-only loop at that ratio reaches 57% of the MFMA
// peak (62-67% at one fragment per two MFMAs, 89% with no LDS reads).
#include "sk_internal.h"
#include "sk_mfma.h"
#include "sk_gemm.h"
#include "sk_gemm_dev.h"

#include <atomic>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

namespace sk {
namespace {

using namespace dev;

// One sweep of the workgroup over columns [j0, j1). Wave (wr, wc)
// accumulates rows wr * kRows/WGR + rb * 32 + li against columns
// wc * kCols/2 + ct * 32 of each block. Ends with a barrier.
template <bool SHIFTED, bool SCALED, class G, int WRT, int WCT>
__device__ __attribute__((always_inline)) inline void gemm_sweep(
    const MfmaPassArgs& p, TileLds<G>& L, int nkb, int col_last, int r0, int j0, int j1,
    const bf16x8 (&Baug)[WRT], float (&M)[WRT], float (&S)[WRT], int wr, int wc, int li, int half) {
  static_assert(G::kRows == 32 * WRT * (G::kNT / 128) && G::kCols == 64 * WCT, "wave tile matches the geometry");
  constexpr int kWaveRows = G::kRows / (G::kNT / 128);
  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const int nkc = nkb / kGKb;
  const int nblocks = (j1 - j0 + G::kCols - 1) / G::kCols;
  const int nstages = nblocks * nkc;
  auto load_stage = [&](TileRegs<G>& g, int st) {
    tile_load<G>(g, rows, cols, nkb, p.nr, col_last, r0, j0 + (st / nkc) * G::kCols, st % nkc);
  };
  TileRegs<G> g;
  load_stage(g, 0);
  tile_store<G>(g, L, 0);
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
            &L.cols[buf][(wc * (G::kCols / 2) + ct * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb)
        B[rb] = *reinterpret_cast<const bf16x8*>(
            &L.rows[buf][(wr * kWaveRows + rb * 32 + li) * kGRow + half * 64 + kb * 16]);
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb)
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[ct], B[rb], acc[rb][ct], 0, 0, 0);
    }
    if (kc == nkc - 1) {
      // bias block (and row shift), then fold the block's scores into the row sums
      const int cb = j0 + blk * G::kCols + wc * (G::kCols / 2);
#pragma unroll
      for (int ct = 0; ct < WCT; ++ct) {
        const int j = min(cb + ct * 32 + li, col_last);
        const bf16x8 Aaug = p.bias_col[2 * (int64_t)j + half];
#pragma unroll
        for (int rb = 0; rb < WRT; ++rb)
          acc[rb][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aaug, Baug[rb], acc[rb][ct], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb)
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
          if constexpr (SHIFTED) sum_update<SCALED>(acc[rb][ct], p.escale, S[rb]);
          else lse_update(acc[rb][ct], p.escale, M[rb], S[rb]);
        }
    }
    // stage st + 1 into the other buffer (its previous stage was consumed
    // before the last barrier), then fetch stage st + 2
    if (st + 1 < nstages) tile_store<G>(g, L, buf ^ 1);
    if (st + 2 < nstages) load_stage(g, st + 2);
    __syncthreads();
  }
}

// Workgroup-wide maximum over NT threads (every thread must call it).
template <int NT>
__device__ inline float wg_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

template <bool SHIFTED, bool SCALED, int WRT, int WCT, int WGR>
__global__ __launch_bounds__((Geo<WRT, WCT, WGR>::kNT), (Geo<WRT, WCT, WGR>::kOcc)) void k_lse_gemm(
    const MfmaPassArgs p, int nkb, int col_last) {
  using G = Geo<WRT, WCT, WGR>;
  constexpr int kNT = G::kNT;
  constexpr int kWaveRows = G::kRows / WGR;
  __shared__ __attribute__((aligned(16))) TileLds<G> lds;
  __shared__ float red[kNT / 64];
  __shared__ float sm_m[2][G::kRows];  // per column-wave partials of each row
  __shared__ float sm_s[2][G::kRows];
  // Wide tiles keep their accumulators in AGPRs: an (empty) use of one lets
  // the compiler allocate them.
  if constexpr (WRT * WCT >= 16) asm volatile("" ::: "a0");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5;
  const int li = lane & 31;
  // Workgroups are dispatched to the 8 XCDs round robin; the virtual index v
  // gives each XCD a contiguous range, in groups of kGroupRows row blocks:
  // within a group, v runs over the row blocks, then the splits. The
  // workgroups an XCD runs together thus cover a few row blocks times several
  // column splits, and its L2 serves both operands' re-reads (numbered
  // split-major, every resident workgroup had rows of its own, which the L2
  // could not hold).
  constexpr int kGroupRows = 4;
  int sp, rblk;
  {
    const int nwg = p.row_blocks * p.splits;
    const int h = blockIdx.x, xcd = h & 7, q = nwg >> 3, rem = nwg & 7;
    const int v = xcd * q + min(xcd, rem) + (h >> 3);
    const int gsz = kGroupRows * p.splits;
    const int grp = v / gsz;
    const int gr = min(kGroupRows, p.row_blocks - grp * kGroupRows);  // row blocks in this group
    const int off = v - grp * gsz;
    sp = off / gr;
    rblk = grp * kGroupRows + (off - sp * gr);
  }
  const int j0 = sp * p.cols_per_split;
  const int j1 = min(p.nc, j0 + p.cols_per_split);
  const int row0 = rblk * G::kRows;

  float M[WRT], S[WRT];
  bf16x8 Baug[WRT];
  float shift_row[WRT];
  if constexpr (SHIFTED) {
    float dm = -INFINITY;
    for (int q = threadIdx.x; q < p.n_dmax_in; q += kNT) dm = fmaxf(dm, p.dmax_in[q]);
    const float dmax = wg_max<kNT>(dm, red);
#pragma unroll
    for (int rb = 0; rb < WRT; ++rb) {
      const int i = min(row0 + wr * kWaveRows + rb * 32 + li, p.nr - 1);
      shift_row[rb] = p.Lin[i] + dmax;
      Baug[rb] = row_aug(half, -shift_row[rb] / p.escale);
      M[rb] = 0.0f;
      S[rb] = 0.0f;
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < WRT; ++rb) {
      Baug[rb] = row_aug(half, 0.0f);
      M[rb] = -INFINITY;
      S[rb] = 0.0f;
      shift_row[rb] = 0.0f;
    }
  }

  // Per row: (Lm, Ls) with L = Lm + log2 Ls (log2 units), merged over the two
  // column waves and the two halves of each wave.
  auto merge_rows = [&](bool shifted) {
#pragma unroll
    for (int rb = 0; rb < WRT; ++rb) {
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
        sm_m[wc][wr * kWaveRows + rb * 32 + li] = lm;
        sm_s[wc][wr * kWaveRows + rb * 32 + li] = ls;
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

  gemm_sweep<SHIFTED, SCALED, G, WRT, WCT>(p, lds, nkb, col_last, row0, j0, j1, Baug, M, S, wr, wc, li, half);
  merge_rows(SHIFTED);

  // thread t owns rows t, t + 256, ... of the block
  constexpr int kRowsPerThread = (G::kRows + kNT - 1) / kNT;
  float dh = -INFINITY;
  bool need_exact = false;
  float Lr[kRowsPerThread];
  bool bad = false;
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) Lr[u] = 0.0f;
  if (p.splits == 1) {
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int r = threadIdx.x + u * kNT, i = row0 + r;
      if (r < G::kRows && i < p.nr) {
        float lm, ls;
        row_result(r, lm, ls);
        Lr[u] = lm + fast_log2(ls);
        bad |= SHIFTED && !(ls >= kShiftedFloor);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int r = threadIdx.x + u * kNT, i = row0 + r;
      if (r < G::kRows && i < p.nr) {
        float lm, ls;
        row_result(r, lm, ls);
        store_coherent(&p.part[(int64_t)sp * p.nr + i], make_float2(lm, ls));
      }
    }
    if (!arrive_last(p.counters + rblk, p.splits)) return;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int r = threadIdx.x + u * kNT, i = row0 + r;
      if (r < G::kRows && i < p.nr) {
        float Mt, St;
        merge_partials(p.part + i, p.nr, p.splits, Mt, St);
        Lr[u] = Mt + fast_log2(St);
        bad |= SHIFTED && !(St >= kShiftedFloor);
      }
    }
    if (threadIdx.x == 0) atomicExch(p.counters + rblk, 0u);
  }
  if constexpr (SHIFTED) need_exact = __syncthreads_or(bad || p.force_exact != 0);
  if (!need_exact) {
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int r = threadIdx.x + u * kNT, i = row0 + r;
      if (r < G::kRows && i < p.nr) dh = fmaxf(dh, finish_row_mfma(p, i, Lr[u]));
    }
  }
  if constexpr (SHIFTED) {
    if (need_exact) {
      if (threadIdx.x == 0 && p.exact_count) atomicAdd(p.exact_count, 1u);
#pragma unroll
      for (int rb = 0; rb < WRT; ++rb) {
        Baug[rb] = row_aug(half, 0.0f);
        M[rb] = -INFINITY;
        S[rb] = 0.0f;
      }
      gemm_sweep<false, SCALED, G, WRT, WCT>(p, lds, nkb, col_last, row0, 0, p.nc, Baug, M, S, wr, wc, li, half);
      merge_rows(false);
#pragma unroll
      for (int u = 0; u < kRowsPerThread; ++u) {
        const int r = threadIdx.x + u * kNT, i = row0 + r;
        if (r < G::kRows && i < p.nr) {
          float lm, ls;
          row_result(r, lm, ls);
          dh = fmaxf(dh, finish_row_mfma(p, i, lm + fast_log2(ls)));
        }
      }
    }
  }
  const float bmax = wg_max<kNT>(dh, red);
  if (threadIdx.x == 0) p.dmax_out[rblk] = bmax;
}

// Tile shapes: 128 x 128 for bf16 records (two workgroups per CU hide the
// exp2 epilogue behind the other's MFMAs) and 128 x 256 for the six-part
// float32 records, whose long K loop favours fewer operand reads per MFMA
// (0.75 instead of 1 LDS fragment per MFMA; measured 3.4-3.7 ms against
// 4.2 ms at d = 512).
// Workgroup tiles: 256 x 256 with eight waves (the default), and two smaller
// ones for the re-read study of the pass (the operand re-read traffic scales
// with 1/R + 1/C) and for tests: 128 x 128 (four waves, two workgroups per
// CU) and 128 x 256 (four waves).
using Tile256 = Geo<2, 4, 4>;
using Tile128 = Geo<2, 2, 2>;
using Tile128x256 = Geo<2, 4, 2>;

template <class G, bool SHIFTED, bool SCALED>
void launch_geo(const MfmaPassArgs& a, int nkb, int col_last, dim3 grid, hipStream_t s) {
  k_lse_gemm<SHIFTED, SCALED, G::kWRT, G::kWCT, G::kWGR><<<grid, G::kNT, 0, s>>>(a, nkb, col_last);
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
template <class G>
int occupancy_of() {
  int per_cu = 0;
  // the instantiations of one tile share the LDS footprint that binds occupancy
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, k_lse_gemm<true, true, G::kWRT, G::kWCT, G::kWGR>, G::kNT, 0);
  return (e != hipSuccess || per_cu < 1) ? 1 : per_cu;
}

int gemm_resident(int tile) {
  // Per device and tile, computed once; concurrent first calls compute the
  // same value.
  constexpr int kDevices = 16;
  static std::atomic<int> cached[kDevices][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::atomic<int>* slot = (dev >= 0 && dev < kDevices) ? &cached[dev][tile] : nullptr;
  int v = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    const int per_cu = tile == 1 ? occupancy_of<Tile128>() : (tile == 2 ? occupancy_of<Tile128x256>()
                                                                         : occupancy_of<Tile256>());
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    v = per_cu * cus;
    if (slot) slot->store(v, std::memory_order_relaxed);
  }
  return v;
}
}  // namespace

int gemm_tile_choice() {
  const char* v = getenv("FLASHSK_GEMM_TILE");
  if (v && !strcmp(v, "128x128")) return 1;
  if (v && !strcmp(v, "128x256")) return 2;
  return 0;
}

PassPlan plan_gemm_pass(int64_t nr, int64_t nc) {
  PassPlan pl{};
  pl.tile = gemm_tile_choice();
  const int rows = pl.tile == 0 ? Tile256::kRows : (pl.tile == 1 ? Tile128::kRows : Tile128x256::kRows);
  const int cols = pl.tile == 0 ? Tile256::kCols : (pl.tile == 1 ? Tile128::kCols : Tile128x256::kCols);
  pl.rows_per_block = rows;
  pl.row_blocks = (int)((nr + rows - 1) / rows);
  int64_t max_splits = nc / 512 > 1 ? nc / 512 : 1;
  if (max_splits > 64) max_splits = 64;
  int64_t cps = 0;
  pl.splits = (int)round_filling_splits(pl.row_blocks, nc, cols, max_splits, gemm_resident(pl.tile), cps);
  pl.cols_per_split = (int)cps;
  return pl;
}

int gemm_nkb(int dtype, int d) {
  const int slots = (dtype == 1) ? d : 6 * d;
  const int nkb = (slots + 15) / 16;
  return (nkb + kGKb - 1) / kGKb * kGKb;  // whole K chunks
}

namespace {
template <class G>
void launch_tile(const MfmaPassArgs& a, int nkb, bool shifted, bool scaled, int col_last, dim3 grid, hipStream_t s) {
  if (shifted) {
    if (scaled) launch_geo<G, true, true>(a, nkb, col_last, grid, s);
    else launch_geo<G, true, false>(a, nkb, col_last, grid, s);
  } else {
    if (scaled) launch_geo<G, false, true>(a, nkb, col_last, grid, s);
    else launch_geo<G, false, false>(a, nkb, col_last, grid, s);
  }
}
}  // namespace

hipError_t launch_lse_gemm(const MfmaPassArgs& args, int nkb, bool shifted, bool scaled, const PassPlan& pl,
                           hipStream_t s) {
  MfmaPassArgs a = args;
  a.row_blocks = pl.row_blocks;
  a.splits = pl.splits;
  const dim3 grid((unsigned)(pl.row_blocks * pl.splits));
  const int col_last = (int)(mfma_padded_count(a.nc) - 1);
  if (pl.tile == 1) launch_tile<Tile128>(a, nkb, shifted, scaled, col_last, grid, s);
  else if (pl.tile == 2) launch_tile<Tile128x256>(a, nkb, shifted, scaled, col_last, grid, s);
  else launch_tile<Tile256>(a, nkb, shifted, scaled, col_last, grid, s);
  return hipGetLastError();
}

}  // namespace sk
