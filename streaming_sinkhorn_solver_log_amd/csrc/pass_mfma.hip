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

#include <atomic>
#include <math.h>

#include <type_traits>

namespace sk {
namespace {

using namespace dev;

// bf16 points with a separate bias record: the column bias enters as the
// first MFMA's float32 accumulator input (h~ from MfmaPassArgs::hcol) and the
// row shift as the exponent's offset, exp2(e * acc - shift), folded into the
// multiply by e that bf16 points need anyway: one MFMA per tile and row block
// fewer than a bias K block. float32 records keep the bias block (an offset
// would cost them an add per pair).
template <bool SCALED, bool MERGED>
constexpr bool kFloatBias = SCALED && !MERGED;

template <int RB, bool SHIFTED, bool SCALED, bool FB>
__device__ __attribute__((always_inline)) inline void tile_valu(const f32x16 (&acc)[RB], float e,
                                                                const float (&off)[RB], float (&M)[RB],
                                                                float (&S)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (SHIFTED && FB) sum_update_off(acc[rb], e, off[rb], S[rb]);
    else if constexpr (SHIFTED) sum_update<SCALED>(acc[rb], e, S[rb]);
    else lse_update(acc[rb], e, M[rb], S[rb]);
  }
}

// ---------------------------------------------------------------- column staging
// Column records stream into LDS by direct global-to-LDS loads
// (global_load_lds_dwordx4), four tiles (128 columns) per stage, in a ring of
// stages. A tile's image in LDS is NKB + 1 blocks of 1 KB; block kb holds, at
// lane l's 16 bytes, exactly the A operand lane l needs (its half l / 32 of
// K block kb of column tile + l % 32; block NKB is the bias chunk), so the
// compute waves read it back with conflict-free 16-byte reads. With float
// biases (kFloatBias) the last block is instead the tile's 32 float32 biases
// (one global_load_lds_dword; lanes 32-63 load a second copy), read back as
// broadcast 16-byte reads. The four waves of the workgroup share the loads
// (one per block) and one barrier per stage.
constexpr int kStageTiles = 4;
constexpr int kStageCols = kStageTiles * 32;
template <int NKB>
constexpr int kRing = NKB >= 4 ? 2 : 3;  // stages in flight (LDS: ring x 4 x blocks KB)

// LDS blocks per tile: the record's K blocks, plus the bias chunk unless it
// is merged into the record.
template <int NKB, bool MERGED>
constexpr int kBlocks = MERGED ? NKB : NKB + 1;

template <int NKB, bool MERGED, bool FB>
struct StageRing {
  bf16x8 blk[kRing<NKB>][kStageTiles][kBlocks<NKB, MERGED>][64];
};
template <int NKB, bool MERGED>
struct StageRing<NKB, MERGED, true> {
  bf16x8 blk[kRing<NKB>][kStageTiles][NKB][64];
  float hb[kRing<NKB>][kStageTiles][64];  // column biases of the tile, twice
};

// Column operands of one tile with float biases: the data K blocks and the
// tile's biases in LDS, which each row block loads straight into its
// accumulator (no registers held for them).
template <int NKB>
struct ColTileF {
  bf16x8 a[NKB];
  const float* hb;
};

// The accumulator input of a tile: lane (h, li) gets the biases of columns
// 8q + 4h + t in register 4q + t (the accumulator layout), four broadcast
// 16-byte LDS reads.
__device__ __forceinline__ f32x16 bias_tile(const float* hb, int half) {
  const float4* hb4 = reinterpret_cast<const float4*>(hb);
  f32x16 c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = hb4[2 * q + half];  // columns 8q + 4h .. 8q + 4h + 3
    c[4 * q + 0] = v.x;
    c[4 * q + 1] = v.y;
    c[4 * q + 2] = v.z;
    c[4 * q + 3] = v.w;
  }
  return c;
}

// This wave's share of stage [c0, c0 + 128): blocks wave, wave + 4, ... of the
// stage's blocks. Columns past the range read the padding (masked) or the
// next range; they are never summed.
template <int NKB, bool MERGED, bool FB>
__device__ __attribute__((always_inline)) inline void issue_stage(
    StageRing<NKB, MERGED, FB>& L, int slot, const unsigned char* __restrict__ cols, const bf16x8* __restrict__ bias,
    const float* __restrict__ hcol, int c0, int wave, int lane) {
  constexpr int NBT = kBlocks<NKB, MERGED>;
  constexpr int NB = kStageTiles * NBT;
  static_assert(NB % 4 == 0, "blocks of a stage split evenly over four waves");
  const int li = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: block choice on the scalar unit
  // lane (li, h) reads its half h of column (tile start + li)
  const unsigned off_rec = (unsigned)(li * (NKB * 32) + h * (NKB * 16));
  const unsigned off_bias = (unsigned)(li * 32 + h * 16);
#pragma unroll
  for (int q = 0; q < NB / 4; ++q) {
    const int b = wv + 4 * q;
    const int tt = b / NBT, kb = b % NBT;
    const int64_t c = (int64_t)c0 + tt * 32;  // first column of the tile
    if (kb < NKB) {
      load_to_lds(cols + c * (NKB * 32) + kb * 16, off_rec, &L.blk[slot][tt][kb][0]);
    } else if constexpr (FB) {
      load_to_lds_dword(reinterpret_cast<const unsigned char*>(hcol) + c * 4, (unsigned)(li * 4), &L.hb[slot][tt][0]);
    } else {
      load_to_lds(reinterpret_cast<const unsigned char*>(bias) + c * 32, off_bias, &L.blk[slot][tt][kb][0]);
    }
  }
}

// Score tile against the RB row blocks: data K blocks, then (separate layout)
// the bias block.
template <int NKB, int RB, bool MERGED>
__device__ __attribute__((always_inline)) inline void tile_scores(
    const ColTileF<NKB>& ct, const bf16x8 (&B)[RB][NKB], const bf16x8 (&)[RB], f32x16 (&acc)[RB]) {
  // float biases: the first MFMA adds them as its accumulator input
  const int half = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x16 a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct.a[0], B[rb][0], bias_tile(ct.hb, half), 0, 0, 0);
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct.a[kb], B[rb][kb], a, 0, 0, 0);
    acc[rb] = a;
  }
}

template <int NKB, int RB, bool MERGED>
__device__ __attribute__((always_inline)) inline void tile_scores(
    const ColTile<NKB>& ct, const bf16x8 (&B)[RB][NKB], const bf16x8 (&Baug)[RB], f32x16 (&acc)[RB]) {
  if constexpr (MERGED) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x16 a = {};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct.a[kb], B[rb][kb], a, 0, 0, 0);
      acc[rb] = a;
    }
  } else {
    tile_mfma<NKB, RB>(ct, B, Baug, acc);
  }
}

// One sweep of the workgroup over columns [j0, j1), j0 a multiple of 128.
// SHIFTED: the row shift is folded into the row side's bias block (float
// biases: off = -shift in the exponent) and the sums need no running maximum;
// otherwise online max/sum-exp. Ends with a barrier (LDS reusable).
template <int NKB, int RB, bool SHIFTED, bool SCALED, bool MERGED>
__device__ __attribute__((always_inline)) inline void sweep(
    const MfmaPassArgs& p, StageRing<NKB, MERGED, kFloatBias<SCALED, MERGED>>& L, int j0, int j1,
    const bf16x8 (&B)[RB][NKB], const bf16x8 (&Baug)[RB], const float (&off)[RB], float (&M)[RB],
    float (&S)[RB], int lane, int wave) {
  constexpr bool FB = kFloatBias<SCALED, MERGED>;
  using Tile = std::conditional_t<FB, ColTileF<NKB>, ColTile<NKB>>;
  constexpr int R = kRing<NKB>;
  constexpr int PER = kStageTiles * kBlocks<NKB, MERGED> / 4;  // loads per wave per stage
  const unsigned char* __restrict__ cols = static_cast<const unsigned char*>(p.cols);
  const int nstages = (j1 - j0 + kStageCols - 1) / kStageCols;
  // Software pipeline over the whole sweep: the MFMAs of tile g are issued
  // before the exp/sum work of tile g - 1, across stage boundaries (tile g's
  // scores live in acc[g & 1]; a stage holds an even number of tiles). The
  // slot read before the first tile holds -inf scores, which add nothing.
  static_assert(kStageTiles % 2 == 0, "tile parity carries across stages");
  f32x16 acc[2][RB];
  if constexpr (NKB <= 4) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1][rb][r] = -INFINITY;
  }
  // Every earlier load (row records, shifts) completes here. Otherwise the
  // compiler waits for them at their first use inside the stage loop, with a
  // full vmcnt(0) that would also wait, every stage, for the loads just
  // issued for the stages ahead.
  wait_vmcnt<0>();
#pragma unroll
  for (int q = 0; q < R - 1; ++q)
    if (q < nstages) issue_stage<NKB, MERGED, FB>(L, q, cols, p.bias_col, p.hcol, j0 + q * kStageCols, wave, lane);
  for (int st = 0; st < nstages; ++st) {
    // this wave's loads of stage st are done once at most the later stages'
    // loads are outstanding; the barrier then covers every wave's loads
    if constexpr (R == 3) {
      if (st + 1 < nstages) wait_vmcnt<PER>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    // slot (st - 1) % R is free: every wave finished stage st - 1 before the barrier
    if (st + R - 1 < nstages)
      issue_stage<NKB, MERGED, FB>(L, (st + R - 1) % R, cols, p.bias_col, p.hcol, j0 + (st + R - 1) * kStageCols,
                                   wave, lane);
    const int slot = st % R;
    auto stage_tile = [&](Tile& ct, int tt) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) ct.a[kb] = L.blk[slot][tt][kb][lane];
      if constexpr (FB) {
        ct.hb = &L.hb[slot][tt][0];
      } else if constexpr (!MERGED) {
        ct.aug = L.blk[slot][tt][NKB][lane];
      }
    };
    if constexpr (NKB <= 4) {
      Tile ct;
#pragma unroll
      for (int tt = 0; tt < kStageTiles; ++tt) {
        stage_tile(ct, tt);
        tile_scores<NKB, RB, MERGED>(ct, B, Baug, acc[tt & 1]);
        tile_valu<RB, SHIFTED, SCALED, FB>(acc[(tt + 1) & 1], p.escale, off, M, S);
      }
    } else {
      // wide records: registers do not allow a second tile of accumulators
#pragma unroll
      for (int tt = 0; tt < kStageTiles; ++tt) {
        Tile ct;
        stage_tile(ct, tt);
        f32x16 one[RB];
        tile_scores<NKB, RB, MERGED>(ct, B, Baug, one);
        tile_valu<RB, SHIFTED, SCALED, FB>(one, p.escale, off, M, S);
      }
    }
  }
  if constexpr (NKB <= 4)
    if (nstages > 0) tile_valu<RB, SHIFTED, SCALED, FB>(acc[1], p.escale, off, M, S);  // the last tile
  __syncthreads();
}

// ---------------------------------------------------------------- work split
// The pass is R row blocks x T stages (128 columns) = U units, ordered chunk
// by chunk: the columns are cut into C chunks, and within a chunk the units
// run row block by row block. Workgroup v of W takes units [v U / W,
// (v + 1) U / W): every workgroup gets the same amount of work (within one
// unit) and the grid is one wave of resident workgroups. Workgroups are
// dispatched to the 8 XCDs round robin; numbering them so that each XCD
// holds a contiguous range of v makes the workgroups of one XCD share about
// 1/C of the columns, which its L2 cache keeps. A row block is merged from
// the partials of its contributors by the last one to arrive, in (chunk,
// workgroup) order, so results do not depend on timing.
struct UnitMap {
  int64_t R, T, C, U, W;
  __host__ __device__ int64_t cs(int64_t c) const { return c * T / C; }   // first stage of chunk c
  __host__ __device__ int64_t off(int64_t c) const { return R * cs(c); }  // first unit of chunk c
  __host__ __device__ int64_t begin(int64_t v) const { return v * U / W; }
  __host__ __device__ int64_t owner(int64_t u) const { return ((u + 1) * W - 1) / U; }
  __host__ __device__ int64_t chunk_of(int64_t u) const {
    int64_t c = u * C / U;
    while (c + 1 < C && off(c + 1) <= u) ++c;
    while (c > 0 && off(c) > u) --c;
    return c;
  }
  // workgroups that contribute to row block r within chunk c
  __host__ __device__ int64_t contrib(int64_t c, int64_t r) const {
    const int64_t tc = cs(c + 1) - cs(c);
    if (tc == 0) return 0;
    const int64_t a = off(c) + r * tc;
    return owner(a + tc - 1) - owner(a) + 1;
  }
};

// Column chunks of a pass: the fewest (1, 2, 4 or 8) whose share of the
// column bytes fits one XCD's 4 MB L2, so that the XCDs sweeping a chunk keep
// it cached. More chunks than needed cost more row-block segments per
// workgroup (row loads, partials, merges): measured at n = m = 50k, eight
// chunks instead of one made the d = 3 half-pass 8% slower.
int64_t chunks_for(int64_t T, int64_t W, int64_t col_bytes) {
  constexpr int64_t kL2Bytes = int64_t(4) << 20;
  if (W % 8 != 0) return 1;
  int64_t c = 1;
  while (c < 8 && c < T && col_bytes / c > kL2Bytes) c *= 2;
  return c;
}

// Row results of one row block: (Lm, Ls) per row with L = Lm + log2 Ls (log2
// units), in lanes of half 0.
template <int RB, bool SHIFTED>
__device__ __forceinline__ void row_sums(const MfmaPassArgs& p, const float (&M)[RB], const float (&S)[RB],
                                         const float (&shift_row)[RB], float (&Lm)[RB], float (&Ls)[RB]) {
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
}

// One half-pass. SHIFTED (every pass after a side's first): the row shift
// M_i = L_i(previous pass) + max_j (change of h_j since then) bounds every
// term by 1, so the sum cannot overflow; a row block with a sum below 2^-60
// (shift far too high) is recomputed by an exact online-max sweep over all
// columns, by the workgroup that completes it.
// Waves per SIMD the register allocation must allow: 4 for the one-block
// layouts (d = 3 float32, small bf16), 3 up to four K blocks (d = 64 bf16:
// at most 168 VGPRs), 2 for wide records (their LDS ring allows two
// workgroups per CU anyway).
template <int NKB, bool MERGED>
constexpr int kMinWaves = (MERGED || NKB == 1) ? 4 : (NKB <= 4 ? 3 : 2);

// PAIR: two independent half-passes (the averaged schedule's F and G maps,
// both of the previous pair) share one launch: workgroups below w0 run p0's
// pass over its own plan, the others p1's. Otherwise p1 and w0 are unused.
template <int NKB, int RB, bool SHIFTED, bool SCALED, bool MERGED, bool PAIR>
__global__ __launch_bounds__(kThreads, (kMinWaves<NKB, MERGED>)) void k_lse_mfma(const MfmaPassArgs p0,
                                                                                 const MfmaPassArgs p1, int w0) {
  const bool second = PAIR && (int)blockIdx.x >= w0;
  const MfmaPassArgs& p = second ? p1 : p0;
  constexpr int RSB = NKB * 32;
  constexpr int ROWS = 4 * RB * 32;
  static_assert(ROWS <= kThreads, "the partial merge finishes one row per thread");
  __shared__ float red[kThreads / 64];
  constexpr bool FB = kFloatBias<SCALED, MERGED>;
  __shared__ __attribute__((aligned(16))) StageRing<NKB, MERGED, FB> lds;
  // Row side of the bias block: (1, 1, 1, -shift parts) meeting the column's
  // (bias parts, 1, 1, 1). Separate layout: its own K block (Baug); merged
  // layout: the free last chunk of the row record (half 1, K block NKB - 1).
  auto set_row_aug = [&](bf16x8 (&Bx)[NKB], bf16x8& Baugx, float neg_m, int half_) {
    if constexpr (MERGED) {
      if (half_ == 1) Bx[NKB - 1] = row_aug(0, neg_m);
    } else {
      Baugx = row_aug(half_, neg_m);
    }
  };

  const unsigned char* __restrict__ rows = static_cast<const unsigned char*>(p.rows);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int li = lane & 31;
  const int64_t W = PAIR ? (second ? (int64_t)gridDim.x - w0 : w0) : (int64_t)gridDim.x;
  const int64_t w = second ? (int64_t)blockIdx.x - w0 : (int64_t)blockIdx.x;
  const int64_t T = p.stages;
  const UnitMap um{p.row_blocks, T, p.chunks > 0 ? p.chunks : 1, (int64_t)p.row_blocks * T, W};
  const int64_t v = (W % 8 == 0) ? (w % 8) * (W / 8) + w / 8 : w;  // XCD-contiguous numbering
  const int64_t u_end = um.begin(v + 1);

  // Largest change of a column bias since this side's previous pass: the
  // loads start here, the workgroup maximum is taken after the first row
  // segment's loads are issued (their latencies overlap).
  float dmax = 0.0f, dm = -INFINITY;
  bool dmax_ready = !SHIFTED;
  if constexpr (SHIFTED)
    for (int q = threadIdx.x; q < p.n_dmax_in; q += kThreads) dm = fmaxf(dm, p.dmax_in[q]);

  for (int64_t u = um.begin(v); u < u_end;) {
    const int64_t c = um.chunk_of(u);
    const int64_t tc = um.cs(c + 1) - um.cs(c);
    const int64_t local = u - um.off(c);
    const int r = (int)(local / tc);
    const int s0 = (int)(um.cs(c) + local % tc);
    const int64_t seg_end = min(u_end, um.off(c) + (int64_t)(r + 1) * tc);
    const int s1 = (int)(s0 + (seg_end - u));
    u = seg_end;
    const int row_base = r * ROWS + wave * (RB * 32);

    bf16x8 B[RB][NKB], Baug[RB];
    float M[RB], S[RB], shift_row[RB], off[RB], lin[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = min(row_base + rb * 32 + li, p.nr - 1);
      const bf16x8* rec = reinterpret_cast<const bf16x8*>(rows + (int64_t)i * RSB) + half * NKB;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) B[rb][kb] = rec[kb];
      if constexpr (SHIFTED) lin[rb] = p.Lin[i];
    }
    if (!dmax_ready) {  // the workgroup's first segment (uniform)
      dmax = block_max(dm, red);
      dmax_ready = true;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (SHIFTED) {
        shift_row[rb] = lin[rb] + dmax;  // log2 units
        if constexpr (!FB) set_row_aug(B[rb], Baug[rb], -shift_row[rb] / p.escale, half);
        off[rb] = -shift_row[rb];
        M[rb] = 0.0f;
      } else {
        shift_row[rb] = 0.0f;
        if constexpr (!FB) set_row_aug(B[rb], Baug[rb], 0.0f, half);
        off[rb] = 0.0f;
        M[rb] = -INFINITY;
      }
      S[rb] = 0.0f;
    }

    sweep<NKB, RB, SHIFTED, SCALED, MERGED>(p, lds, s0 * kStageCols, min(p.nc, s1 * kStageCols), B, Baug, off,
                                             M, S, lane, wave);
    float Lm[RB], Ls[RB];
    row_sums<RB, SHIFTED>(p, M, S, shift_row, Lm, Ls);

    // Finish the row block here if this workgroup holds all of it, else leave
    // a partial and let the last contributor merge.
    float dh = -INFINITY;  // largest bias change over the rows this thread finishes
    bool need_exact = false;
    if (s0 == 0 && s1 == T) {
      bool bad = false;
      if constexpr (SHIFTED) {
        if (half == 0)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            bad |= (row_base + rb * 32 + li < p.nr) && !(Ls[rb] >= kShiftedFloor);
        bad |= p.force_exact != 0;
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
      int contributors = 0;
      int64_t slot = 0;
      for (int64_t c2 = 0; c2 < um.C; ++c2) {
        const int64_t n2 = um.contrib(c2, r);
        if (c2 < c) slot += n2;
        contributors += (int)n2;
      }
      slot += v - um.owner(um.off(c) + (int64_t)r * tc);
      if (half == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = row_base + rb * 32 + li;
          if (i < p.nr) store_coherent(&p.part[slot * p.nr + i], make_float2(Lm[rb], Ls[rb]));
        }
      }
      if (!arrive_last(p.counters + r, contributors)) continue;
      // the last contributor merges the partials of the row block in workgroup order
      float Lr = 0.0f;
      bool bad = false;
      const int i = r * ROWS + (int)threadIdx.x;
      const bool mine = (int)threadIdx.x < ROWS && i < p.nr;
      RowIn rin{};
      if (mine) {
        rin = load_row_in(p, i);
        float Mt, St;
        merge_partials(p.part + i, p.nr, contributors, Mt, St);
        Lr = Mt + fast_log2(St);
        bad = SHIFTED && !(St >= kShiftedFloor);
      }
      if constexpr (SHIFTED) need_exact = __syncthreads_or(bad || p.force_exact != 0);
      if (!need_exact && mine) dh = finish_row_mfma(p, i, Lr, rin);
      if (threadIdx.x == 0) atomicExch(p.counters + r, 0u);
    }

    if constexpr (SHIFTED) {
      if (need_exact) {
        // exact recomputation of this row block over all columns
        if (threadIdx.x == 0 && p.exact_count) atomicAdd(p.exact_count, 1u);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (!FB) set_row_aug(B[rb], Baug[rb], 0.0f, half);
          M[rb] = -INFINITY;
          S[rb] = 0.0f;
        }
        sweep<NKB, RB, false, SCALED, MERGED>(p, lds, 0, p.nc, B, Baug, off, M, S, lane, wave);
        row_sums<RB, false>(p, M, S, shift_row, Lm, Ls);
        dh = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = row_base + rb * 32 + li;
          if (half == 0 && i < p.nr) dh = fmaxf(dh, finish_row_mfma(p, i, Lm[rb] + fast_log2(Ls[rb])));
        }
      }
    }
    const float bmax = block_max(dh, red);
    if (threadIdx.x == 0) p.dmax_out[r] = bmax;
  }
}

// ---------------------------------------------------------------- record prep
// Slot s of a record: data slots first (coordinate-major), then zeros.
// bf16 storage: one slot per coordinate. float32 storage: six slots per coordinate.
// Records of the GEMM-tiled kernels (interleave) are stored K block by K
// block: chunk (half h, K block kb) at position 2 kb + h instead of h nkb + kb.
__global__ __launch_bounds__(256) void k_pack_records(const void* pts, int dtype, int64_t n, int d,
                                                      const float* shift, int nkb, float c2, int interleave,
                                                      bf16x8* row_rec, bf16x8* col_rec) {
  const int chunks = nkb * 2;  // 16-byte chunks per record
  const int64_t total = n * chunks;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / chunks;
    const int q = (int)(c % chunks);
    bf16x8 rv = {}, cv = {};
    if (dtype == 1 && (d & 7) == 0 && q * 8 < d) {
      // eight whole coordinates: one 16-byte load (rows are 16-byte aligned)
      const bf16x8 v = reinterpret_cast<const bf16x8*>(static_cast<const unsigned short*>(pts) + r * d)[q];
      if (shift) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          rv[e] = (__bf16)((float)v[e] - shift[q * 8 + e]);  // exact (prep.hip)
      } else {
        rv = v;
      }
      cv = rv;
      const int64_t at = interleave ? r * chunks + (q % nkb) * 2 + q / nkb : c;
      row_rec[at] = rv;
      col_rec[at] = cv;
      continue;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = q * 8 + e;
      if (dtype == 1) {
        if (s < d) {
          const unsigned short bits = static_cast<const unsigned short*>(pts)[r * d + s];
          __bf16 v = __builtin_bit_cast(__bf16, bits);
          if (shift) v = (__bf16)(__uint_as_float((unsigned)bits << 16) - shift[s]);  // exact (prep.hip)
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
    const int64_t at = interleave ? r * chunks + (q % nkb) * 2 + q / nkb : c;
    row_rec[at] = rv;
    col_rec[at] = cv;
  }
}

// Norms (of the values the records represent), log-weights, starting potentials
// and the initial bias chunks (at bias + r * bias_stride). Separate layout
// (bias_alt non-null): the half-1 chunks of both bias buffers are zeroed here
// once; the passes only rewrite half-0 chunks. G threads per point: one for
// small d, a wave for large d (coordinates k = lane, lane + 64, ...: coalesced
// loads, the norm summed over the wave).
template <int G>
__global__ __launch_bounds__(256) void k_prep_side_mfma(const void* pts, int dtype, int64_t n, int d,
                                                        const float* shift, const float* w,
                                                        const float* pot, float* pot_zero,
                                                        float* alpha, float* lw, bf16x8* bias, int bias_stride,
                                                        bf16x8* bias_alt, float* hval, float log2e_over_eps,
                                                        float bias_scale, float* hacc) {
  static_assert(G == 1 || G == 64, "a thread or a wave per point");
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = t / G;
  const int sub = (int)(t % G);
  if (r >= n) return;  // G = 64: the whole wave
  float nrm = 0.0f;
#pragma unroll 4
  for (int k = sub; k < d; k += G) {
    float v;
    if (dtype == 1) {
      const unsigned short bits = static_cast<const unsigned short*>(pts)[r * d + k];
      v = __uint_as_float(static_cast<unsigned>(bits) << 16);
      if (shift) v -= shift[k];
    } else {
      v = static_cast<const float*>(pts)[r * d + k];
      if (shift) v -= shift[k];
    }
    nrm = fmaf(v, v, nrm);
  }
  if constexpr (G > 1) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) nrm += __shfl_xor(nrm, o, G);
    if (sub != 0) return;
  }
  const float l = logf(w[r]);
  const float pv = pot ? pot[r] : 0.0f;
  if (pot_zero) pot_zero[r] = 0.0f;
  alpha[r] = nrm;
  lw[r] = l;
  const float h = kLog2e * l + (pv - nrm) * log2e_over_eps;
  hval[r] = h;
  write_bias_chunk(bias + r * bias_stride, h * bias_scale);
  if (hacc) hacc[r] = masked_bias(h * bias_scale);
  if (bias_alt) {
    bias[r * bias_stride + 1] = bf16x8{};
    bias_alt[2 * r + 1] = bf16x8{};
  }
}

// Masked padding columns [n, n_pad) of a side. Separate layout: zero records,
// masked bias records in both buffers. Merged layout: zero records whose
// last chunk is a masked bias chunk. Float bias buffers (if given): masked.
__global__ __launch_bounds__(256) void k_pad_columns(int64_t n, int64_t n_pad, int nkb, int merged,
                                                     bf16x8* col_rec, bf16x8* bias0, bf16x8* bias1,
                                                     float* hacc0, float* hacc1) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)nkb * 2;
  bf16x8 masked = {};
  masked[0] = (__bf16)kMaskedBias;
  masked[3] = (__bf16)1.0f;
  masked[4] = (__bf16)1.0f;
  masked[5] = (__bf16)1.0f;
  if (t < (n_pad - n) * per) col_rec[n * per + t] = (merged && t % per == per - 1) ? masked : bf16x8{};
  if (!merged && t < (n_pad - n) * 2) {
    const int64_t q = n * 2 + t;
    const bf16x8 v = ((q & 1) == 0) ? masked : bf16x8{};
    bias0[q] = v;
    bias1[q] = v;
  }
  if (t < n_pad - n) {
    if (hacc0) hacc0[n + t] = kMaskedBias;
    if (hacc1) hacc1[n + t] = kMaskedBias;
  }
}

template <int NKB, int RB, bool MERGED>
hipError_t run_lse(const MfmaPassArgs& a, const PassPlan& pl, const MfmaPassArgs& a1, const PassPlan* pl1,
                   bool shifted, bool scaled, hipStream_t s) {
  const int w0 = pl.grid;
  const dim3 grid(pl.grid + (pl1 ? pl1->grid : 0));
  if (pl1) {
    // the averaged schedule, which never uses the merged layout
    if constexpr (MERGED) {
      return hipErrorInvalidValue;
    } else {
      if (shifted) {
        if (scaled) k_lse_mfma<NKB, RB, true, true, false, true><<<grid, kThreads, 0, s>>>(a, a1, w0);
        else k_lse_mfma<NKB, RB, true, false, false, true><<<grid, kThreads, 0, s>>>(a, a1, w0);
      } else {
        if (scaled) k_lse_mfma<NKB, RB, false, true, false, true><<<grid, kThreads, 0, s>>>(a, a1, w0);
        else k_lse_mfma<NKB, RB, false, false, false, true><<<grid, kThreads, 0, s>>>(a, a1, w0);
      }
      return hipGetLastError();
    }
  }
  if (shifted) {
    if (scaled) k_lse_mfma<NKB, RB, true, true, MERGED, false><<<grid, kThreads, 0, s>>>(a, a, w0);
    else k_lse_mfma<NKB, RB, true, false, MERGED, false><<<grid, kThreads, 0, s>>>(a, a, w0);
  } else {
    if (scaled) k_lse_mfma<NKB, RB, false, true, MERGED, false><<<grid, kThreads, 0, s>>>(a, a, w0);
    else k_lse_mfma<NKB, RB, false, false, MERGED, false><<<grid, kThreads, 0, s>>>(a, a, w0);
  }
  return hipGetLastError();
}

// Workgroups of the shifted kernel of a record width that fit on the device at once.
int resident_workgroups(int nkb, bool merged) {
  // Per device and record width, computed once; concurrent first calls
  // compute the same value.
  constexpr int kDevices = 16;
  static std::atomic<int> cached[kDevices][9][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (nkb < 1 || nkb > 8) return 0;
  std::atomic<int>* slot = (dev >= 0 && dev < kDevices) ? &cached[dev][nkb][merged ? 1 : 0] : nullptr;
  int v = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    int per_cu = 0, cus = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (nkb * 2 + (merged ? 1 : 0)) {
      case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_mfma<1, 2, true, true, false, false>, kThreads, 0); break;
      case 3: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_mfma<1, 2, true, true, true, false>, kThreads, 0); break;
      case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_mfma<2, 2, true, false, false, false>, kThreads, 0); break;
      case 5: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_mfma<2, 2, true, false, true, false>, kThreads, 0); break;
      case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_mfma<4, 2, true, true, false, false>, kThreads, 0); break;
      case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_lse_mfma<8, 1, true, true, false, false>, kThreads, 0); break;
      default: break;
    }
    if (e != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    v = per_cu * cus;
    if (slot) slot->store(v, std::memory_order_relaxed);
  }
  return v;
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

bool mfma_merged(int dtype, int d, int nkb) {
  const int slots = (dtype == 1) ? d : 6 * d;
  const int data_chunks = (slots + 7) / 8;
  return nkb <= 2 && data_chunks <= 2 * nkb - 1;
}

int64_t mfma_padded_count(int64_t n) { return (n + 31) / 32 * 32 + 5 * 32; }

PassPlan plan_mfma_pass(int64_t nr, int64_t nc, int nkb, bool merged, bool scaled, int share) {
  PassPlan pl{};
  pl.rows_per_block = 4 * mfma_rb(nkb) * 32;
  pl.row_blocks = (int)((nr + pl.rows_per_block - 1) / pl.rows_per_block);
  pl.stages = (int)((nc + kStageCols - 1) / kStageCols);
  const int64_t units = (int64_t)pl.row_blocks * pl.stages;
  // A pass sharing its launch with another gets 1/share of the resident
  // workgroups (a multiple of 8, so both keep the XCD-contiguous numbering)
  // where its units are few; with at least 32 units a workgroup each keeps
  // all of them, and a pass of its own with at least 64 gets twice the
  // resident count: the launch then runs two rounds, and workgroups of the
  // second fill the slots the first frees unevenly (n = m = 50k: averaged
  // d = 3, 541 -> 515 us per iteration; alternating d = 64, 399 -> 392 us and
  // d = 3, 241 -> 236 us per half-pass; at 10k the shared grid is faster, 35
  // against 40 us per iteration).
  int64_t grid = resident_workgroups(nkb, merged);
  if (share > 1 && units < 32 * grid) grid = grid / share / 8 * 8 > 0 ? grid / share / 8 * 8 : 1;
  else if (share == 1 && units >= 64 * grid) grid *= 2;
  const int64_t min_units = 4;  // at least 512 columns of one row block per workgroup
  if (grid > units / min_units) grid = units / min_units;
  if (grid < 1) grid = 1;
  pl.grid = (int)grid;
  // column bytes a sweep streams: the records, plus (separate layout) the
  // float32 biases (bf16 points) or the 32-byte bias records
  const int64_t col_bytes = nc * ((int64_t)nkb * 32 + (merged ? 0 : (scaled ? 4 : 32)));
  pl.chunks = (int)chunks_for(pl.stages, grid, col_bytes);
  // partial slots per row: the most contributors any row block has
  const UnitMap um{pl.row_blocks, pl.stages, pl.chunks, units, grid};
  int64_t most = 1;
  for (int64_t r = 0; r < pl.row_blocks; ++r) {
    int64_t n = 0;
    for (int64_t c = 0; c < um.C; ++c) n += um.contrib(c, r);
    if (n > most) most = n;
  }
  pl.splits = (int)most;
  pl.cols_per_split = kStageCols;
  return pl;
}

hipError_t launch_lse_mfma(const MfmaPassArgs& a, int nkb, bool shifted, bool scaled, bool merged,
                           const PassPlan& pl, hipStream_t s) {
  return launch_lse_mfma_pair(a, pl, a, nullptr, nkb, shifted, scaled, merged, s);
}

hipError_t launch_lse_mfma_pair(const MfmaPassArgs& a0, const PassPlan& pl0, const MfmaPassArgs& a1,
                                const PassPlan* pl1, int nkb, bool shifted, bool scaled, bool merged,
                                hipStream_t s) {
  if (merged) {
    switch (nkb) {
      case 1: return run_lse<1, 2, true>(a0, pl0, a1, pl1, shifted, scaled, s);
      case 2: return run_lse<2, 2, true>(a0, pl0, a1, pl1, shifted, scaled, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (nkb) {
    case 1: return run_lse<1, 2, false>(a0, pl0, a1, pl1, shifted, scaled, s);
    case 2: return run_lse<2, 2, false>(a0, pl0, a1, pl1, shifted, scaled, s);
    case 4: return run_lse<4, 2, false>(a0, pl0, a1, pl1, shifted, scaled, s);
    case 8: return run_lse<8, 1, false>(a0, pl0, a1, pl1, shifted, scaled, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prep_mfma(const MfmaPrepSide& xs, const MfmaPrepSide& ys, int dtype, int d,
                            int nkb, bool merged, bool center, double* centroid_part, float* shift,
                            unsigned* counters, int n_counters, float log2e_over_eps,
                            float c2, bool interleave, hipStream_t s) {
  const float* sh = nullptr;
  if (center) {
    hipError_t e = dtype == 0 ? launch_centroid(xs.pts, xs.n, ys.pts, ys.n, dtype, d, centroid_part, shift, s)
                              : launch_bf16_shift(xs.pts, xs.n, ys.pts, ys.n, d, centroid_part, shift, s);
    if (e != hipSuccess) return e;
    sh = shift;
  }
  hipError_t ez = launch_zero_u32(counters, n_counters, s);
  if (ez != hipSuccess) return ez;
  for (const MfmaPrepSide* side : {&xs, &ys}) {
    const int64_t chunks = side->n * nkb * 2;
    const int blocks = (int)((chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096);
    k_pack_records<<<blocks, 256, 0, s>>>(side->pts, dtype, side->n, d, sh, nkb, c2, interleave ? 1 : 0,
                                          side->row_rec, side->col_rec);
    const int64_t npad = mfma_padded_count(side->n);
    const int64_t pad_work = (npad - side->n) * nkb * 2;
    k_pad_columns<<<(int)((pad_work + 255) / 256), 256, 0, s>>>(side->n, npad, nkb, merged ? 1 : 0,
                                                                side->col_rec, side->bias, side->bias_alt,
                                                                side->hacc, side->hacc_alt);
    // merged: the bias chunk is the last chunk of the column record
    bf16x8* bias0 = merged ? side->col_rec + (2 * nkb - 1) : side->bias;
    if (d >= 32) {
      k_prep_side_mfma<64><<<(int)((side->n * 64 + 255) / 256), 256, 0, s>>>(
          side->pts, dtype, side->n, d, sh, side->w, side->pot, side->pot_zero, side->alpha, side->lw,
          bias0, merged ? 2 * nkb : 2, merged ? nullptr : side->bias_alt, side->hval, log2e_over_eps,
          mfma_bias_scale(dtype, c2), side->hacc);
    } else {
      k_prep_side_mfma<1><<<(int)((side->n + 255) / 256), 256, 0, s>>>(
          side->pts, dtype, side->n, d, sh, side->w, side->pot, side->pot_zero, side->alpha, side->lw,
          bias0, merged ? 2 * nkb : 2, merged ? nullptr : side->bias_alt, side->hval, log2e_over_eps,
          mfma_bias_scale(dtype, c2), side->hacc);
    }
  }
  return hipGetLastError();
}

}  // namespace sk
