// Preparation kernels: W_O transposed and converted to fp16 for the output
// projection (both of its MFMA operands K-contiguous fp16), the gate weights'
// small transpose, and the scan of a padding mask (key extent and per-tile
// ignore bits of each batch element), in one launch; then the batch elements
// ranked by key extent.
#include "device_common.h"
#include "kernels.h"
#include "transpose_tile.h"

namespace mha {

namespace {

constexpr int TT = kTransposeTile;

// One launch: workgroups [0, tiles_t) transpose weights, WT[n][k] = W[k][n]
// for up to two matrices (the first `tiles0` workgroups take the first), one
// 64 x 64 tile each; workgroups [tiles_t, small_end) transpose a small matrix
// (the gate weights) one element per thread; workgroups past them scan the
// padding mask of one batch element each (the transpose tile itself:
// transpose_tile64).
//
// Mask scan: each wave takes 64-key tiles in turn, one key per lane; the
// wave's ballot of "ignored" (masked or past T_k) is the tile's 64-bit ignore
// mask, and its highest clear bit the tile's last unmasked key. kend[b] = 1 +
// the last unmasked key, 0 if every key is masked.
__global__ void __launch_bounds__(256)
prep_kernel(TransposeJob j0, TransposeJob j1, int tiles0, int tiles_t, SmallTranspose st,
            int small_end, MaskScan ms) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TT][TT + 8];
  __shared__ int red[4];
  if ((int)blockIdx.x >= tiles_t && (int)blockIdx.x < small_end) {
    // small transpose: one element per thread, the reads along W's rows
    const long long i = (long long)((int)blockIdx.x - tiles_t) * 256 + threadIdx.x;
    if (i < (long long)st.K * st.N) {
      const int k = (int)(i / st.N), n = (int)(i - (long long)k * st.N);
      st.WT[(size_t)n * st.K + k] = st.W[i];
    }
    return;
  }
  if ((int)blockIdx.x >= small_end) {
    const int b = (int)blockIdx.x - small_end;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int T_k = ms.T_k, ntk = (T_k + 63) / 64;
    const uint8_t* mrow = ms.mask + (size_t)b * T_k;
    int last = -1;
    for (int t = wave; t < ntk; t += 4) {
      const int key = t * 64 + lane;
      const bool ign = key >= T_k || mrow[key] != 0;
      const uint64_t ib = __ballot(ign);
      if (lane == 0) {
        ms.bits[((size_t)b * ntk + t) * 2] = (uint32_t)ib;
        ms.bits[((size_t)b * ntk + t) * 2 + 1] = (uint32_t)(ib >> 32);
      }
      const uint64_t keep = ~ib;
      if (keep) last = t * 64 + 63 - __builtin_clzll(keep);   // tiles rise per wave
    }
    if (lane == 0) red[wave] = last;
    __syncthreads();
    if (threadIdx.x == 0) ms.kend[b] = max(max(red[0], red[1]), max(red[2], red[3])) + 1;
    return;
  }
  const bool second = (int)blockIdx.x >= tiles0;
  transpose_tile64(second ? j1 : j0, second ? (int)blockIdx.x - tiles0 : (int)blockIdx.x, tile);
}

// One workgroup per batch element: largest unmasked key index + 1.
// Rank of each batch element by key extent (descending, ties by index); every
// workgroup stages all B extents in LDS and ranks 256 of them. B <= 1024.
__global__ void __launch_bounds__(256)
mask_order_kernel(const int* __restrict__ kend, int B, int* __restrict__ order) {
  __shared__ int ke[kMaskOrderMaxB];
  for (int i = threadIdx.x; i < B; i += 256) ke[i] = kend[i];
  __syncthreads();
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int mine = ke[b];
  int rank = 0;
  for (int i = 0; i < B; ++i) rank += (ke[i] > mine || (ke[i] == mine && i < b)) ? 1 : 0;
  order[rank] = b;
}

}  // namespace

hipError_t launch_prep(const TransposeJob& j0, const TransposeJob* j1, const SmallTranspose& st,
                       const MaskScan& ms, hipStream_t s) {
  const long long t0 = j0.W ? transpose_tiles(j0) : 0, t1 = j1 && j1->W ? transpose_tiles(*j1) : 0;
  const long long ns = st.W ? ((long long)st.K * st.N + 255) / 256 : 0;
  const long long nb = ms.mask ? ms.B : 0;
  if ((j1 && j1->W && !j0.W) || t0 + t1 + ns + nb < 1 || t0 + t1 + ns + nb > 0x7fffffffLL ||
      (ms.mask && ms.T_k < 1) || (st.W && (st.K < 1 || st.N < 1)))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(t0 + t1 + ns + nb)), dim3(256), 0, s, j0,
                     j1 ? *j1 : j0, (int)t0, (int)(t0 + t1), st, (int)(t0 + t1 + ns), ms);
  return hipGetLastError();
}

hipError_t launch_mask_order(const int* kend, int B, int* order, hipStream_t s) {
  if (B < 1 || B > kMaskOrderMaxB) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mask_order_kernel, dim3((B + 255) / 256), dim3(256), 0, s, kend, B, order);
  return hipGetLastError();
}


}  // namespace mha
