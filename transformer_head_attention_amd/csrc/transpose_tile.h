// One 64 x 64 tile of a weight transpose, WT[n][k] = W[k][n], optionally with
// bf16 -> fp16 conversion, by a workgroup of 256 threads. Shared by the
// preparation kernel and the attention launch (whose first workgroups convert
// W_O while the attention runs).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace mha {

constexpr int kTransposeTile = 64;

__host__ __device__ inline int transpose_tiles(const TransposeJob& j) {
  return ((j.N + kTransposeTile - 1) / kTransposeTile) * ((j.K + kTransposeTile - 1) / kTransposeTile);
}

// Tile `blk` of job jb (tiles numbered along N first). tile: 64 x 72 16-bit
// LDS staging (rows padded by 16 bytes, so the 8 lanes gathering one column
// chunk hit different banks). Global traffic moves 16 bytes per lane both
// ways: rows of W are read as 8-element chunks, and each output chunk
// gathers 8 consecutive k of one column. Requires K and N multiples of 8.
__device__ __forceinline__ void transpose_tile64(const TransposeJob& jb, int blk,
                                                 uint16_t (*tile)[kTransposeTile + 8]) {
  constexpr int TT = kTransposeTile;
  const uint16_t* __restrict__ W = jb.W;
  uint16_t* __restrict__ WT = jb.WT;
  const int K = jb.K, N = jb.N;
  const int ntx = (N + TT - 1) / TT;
  const int n0 = (blk % ntx) * TT, k0 = (blk / ntx) * TT;
  const int t = threadIdx.x, r = t >> 3, c = t & 7;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int kr = r + 32 * pass, k = k0 + kr, n = n0 + 8 * c;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k < K && n < N) v = *reinterpret_cast<const u32x4*>(W + (size_t)k * N + n);
    *reinterpret_cast<u32x4*>(&tile[kr][8 * c]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int nr = r + 32 * pass, n = n0 + nr, k = k0 + 8 * c;
    if (n < N && k < K) {
      uint16_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t v = tile[8 * c + j][nr];
        if (jb.to_f16) {
          const float f = bf16_bits_to_float(v);
          v = float_to_f16_bits(f);
          flag_f16_overflow(jb.overflow, fabsf(f));
        }
        e[j] = v;
      }
      *reinterpret_cast<u32x4*>(WT + (size_t)n * K + k) =
          u32x4{e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16};
    }
  }
}

}  // namespace mha
