// sk_gemm_dev.h -- LDS staging of the GEMM-tiled kernels (library-internal;
// included by pass_gemm.hip and pass_pv.hip).
#pragma once

#include "sk_mfma_dev.h"

namespace sk {
namespace dev {

// ---------------------------------------------------------------- GEMM-tiled staging
constexpr int kGKb = 4;       // K blocks (16 slots) per LDS stage
constexpr int kGRow = kGKb * 2 * 16 + 16;  // LDS bytes per record per stage (both halves + pad)

// The GEMM-tiled kernels read records stored K block by K block: the 16-byte
// chunk of half h and K block kb sits at chunk position 2 kb + h (the
// register-resident kernels keep each half's run together instead), so the
// four K blocks of a stage are 128 contiguous bytes of a record, one cache
// line, and eight threads load it whole.
__device__ __forceinline__ int64_t gemm_chunk_off(int hh, int kc, int part) {
  return (int64_t)((kc * kGKb + part) * 2 + hh) * 16;
}


// Workgroups of 2 x 2 waves own 128 rows and sweep columns in blocks of 128;
// both operands stream through LDS in chunks of 4 K blocks.
constexpr int kGRows = 128;   // rows per workgroup
constexpr int kGCols = 128;   // columns per block

struct GemmLds {
  unsigned char rows[2][kGRows * kGRow];
  unsigned char cols[2][kGCols * kGRow];
};

struct GemmRegs {
  u32x4 r[4];  // 1024 row chunks / 256 threads
  u32x4 c[4];  // 1024 column chunks / 256 threads
};

// Stage s of the flattened (column block, K chunk) sequence: chunk (kc) of the
// K dimension for rows [r0, r0+128) and columns [c0, c0+128). A chunk is, per
// record, the 128 bytes [kc * 128, +128) (both halves of 4 K blocks).
__device__ __attribute__((always_inline)) inline void gemm_load(
    GemmRegs& g, const unsigned char* __restrict__ rows, const unsigned char* __restrict__ cols,
    int nkb, int nr, int r0, int c0, int kc) {
  const int64_t rsb = (int64_t)nkb * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = threadIdx.x + q * kThreads;  // 0..1023: record (ch >> 3), half ((ch >> 2) & 1), part (ch & 3)
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    const int64_t off = gemm_chunk_off(hh, kc, part);
    g.r[q] = *reinterpret_cast<const u32x4*>(rows + (int64_t)min(r0 + rec, nr - 1) * rsb + off);
    g.c[q] = *reinterpret_cast<const u32x4*>(cols + (int64_t)(c0 + rec) * rsb + off);
  }
}

__device__ __attribute__((always_inline)) inline void gemm_store(const GemmRegs& g, GemmLds& L, int buf) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = threadIdx.x + q * kThreads;
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    const int o = rec * kGRow + hh * 64 + part * 16;
    *reinterpret_cast<u32x4*>(&L.rows[buf][o]) = g.r[q];
    *reinterpret_cast<u32x4*>(&L.cols[buf][o]) = g.c[q];
  }
}

// ---------------------------------------------------------------- 256 x 256 tiles of 8 waves
// Workgroup tile: WGR x 2 waves (row waves x column waves), each wave
// WRT x WCT accumulator tiles of 32 x 32, i.e. 32 WRT WGR rows and 64 WCT
// columns per workgroup.
template <int WRT, int WCT, int WGR>
struct Geo {
  static constexpr int kWRT = WRT, kWCT = WCT, kWGR = WGR;
  static constexpr int kNT = 128 * WGR;  // threads
  static constexpr int kRows = 32 * WRT * WGR;
  static constexpr int kCols = 64 * WCT;
  static constexpr int kRowLoads = kRows * 8 / kNT;  // 16-byte chunks per thread per stage
  static constexpr int kColLoads = kCols * 8 / kNT;
  static constexpr int kOcc = (WRT * WCT * WGR > 8) ? 1 : 2;  // workgroups per CU
  static_assert(kRows * 8 % kNT == 0 && kCols * 8 % kNT == 0, "stage loads split evenly");
};

template <class G>
struct TileLds {
  unsigned char rows[2][G::kRows * kGRow];
  unsigned char cols[2][G::kCols * kGRow];
};

template <class G>
struct TileRegs {
  u32x4 r[G::kRowLoads];
  u32x4 c[G::kColLoads];
};

// Stage (kc) of the K dimension for rows [r0, r0 + kRows) and columns
// [c0, c0 + kCols): per record, the 128 bytes [kc * 128, +128) (both halves
// of 4 K blocks). Row indices clamp to the last row, column indices to the
// last padded (masked) column.
template <class G>
__device__ __attribute__((always_inline)) inline void tile_load(
    TileRegs<G>& g, const unsigned char* __restrict__ rows, const unsigned char* __restrict__ cols,
    int nkb, int nr, int col_last, int r0, int c0, int kc) {
  const int64_t rsb = (int64_t)nkb * 32;
#pragma unroll
  for (int q = 0; q < G::kRowLoads; ++q) {
    const int ch = threadIdx.x + q * G::kNT;  // record (ch >> 3), half ((ch >> 2) & 1), part (ch & 3)
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    const int64_t off = gemm_chunk_off(hh, kc, part);
    g.r[q] = *reinterpret_cast<const u32x4*>(rows + (int64_t)min(r0 + rec, nr - 1) * rsb + off);
  }
#pragma unroll
  for (int q = 0; q < G::kColLoads; ++q) {
    const int ch = threadIdx.x + q * G::kNT;
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    const int64_t off = gemm_chunk_off(hh, kc, part);
    g.c[q] = *reinterpret_cast<const u32x4*>(cols + (int64_t)min(c0 + rec, col_last) * rsb + off);
  }
}

template <class G>
__device__ __attribute__((always_inline)) inline void tile_store(const TileRegs<G>& g, TileLds<G>& L, int buf) {
#pragma unroll
  for (int q = 0; q < G::kRowLoads; ++q) {
    const int ch = threadIdx.x + q * G::kNT;
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    *reinterpret_cast<u32x4*>(&L.rows[buf][rec * kGRow + hh * 64 + part * 16]) = g.r[q];
  }
#pragma unroll
  for (int q = 0; q < G::kColLoads; ++q) {
    const int ch = threadIdx.x + q * G::kNT;
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    *reinterpret_cast<u32x4*>(&L.cols[buf][rec * kGRow + hh * 64 + part * 16]) = g.c[q];
  }
}

}  // namespace dev
}  // namespace sk
