// sk_gemm_dev.h -- LDS staging of the GEMM-tiled kernels (library-internal;
// included by pass_gemm.hip and pass_pv.hip).
#pragma once

#include "sk_mfma_dev.h"

namespace sk {
namespace dev {

// ---------------------------------------------------------------- GEMM-tiled staging
// Workgroups of 2 x 2 waves own 128 rows and sweep columns in blocks of 128;
// both operands stream through LDS in chunks of 4 K blocks.
constexpr int kGRows = 128;   // rows per workgroup
constexpr int kGCols = 128;   // columns per block
constexpr int kGKb = 4;       // K blocks (16 slots) per LDS stage
constexpr int kGRow = kGKb * 2 * 16 + 16;  // LDS bytes per record per stage (both halves + pad)

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
// record, 4 x 16 bytes in each half: record bytes [h*NKB*16 + kc*64, +64).
__device__ __attribute__((always_inline)) inline void gemm_load(
    GemmRegs& g, const unsigned char* __restrict__ rows, const unsigned char* __restrict__ cols,
    int nkb, int nr, int r0, int c0, int kc) {
  const int64_t rsb = (int64_t)nkb * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = threadIdx.x + q * kThreads;  // 0..1023: record (ch >> 3), half ((ch >> 2) & 1), part (ch & 3)
    const int rec = ch >> 3, hh = (ch >> 2) & 1, part = ch & 3;
    const int64_t off = (int64_t)hh * nkb * 16 + (int64_t)kc * 64 + part * 16;
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

}  // namespace dev
}  // namespace sk
