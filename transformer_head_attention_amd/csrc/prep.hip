// Preparation kernels: weight transpose (+ bf16 -> fp16 conversion) so that
// both MFMA operands of the projections are K-contiguous, and the key extent
// of a padding mask.
#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int TT = 64;   // transpose tile edge

// WT[n][k] = W[k][n]; one 64 x 64 tile per workgroup, 256 threads.
template <bool TO_F16>
__global__ void __launch_bounds__(256)
transpose_bf16_kernel(const uint16_t* __restrict__ W, int K, int N, uint16_t* __restrict__ WT) {
  __shared__ uint16_t tile[TT][TT + 2];
  const int n0 = blockIdx.x * TT, k0 = blockIdx.y * TT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < TT / 4; ++i) {
    const int kr = ty + 4 * i;
    const int k = k0 + kr, n = n0 + tx;
    tile[kr][tx] = (k < K && n < N) ? W[(size_t)k * N + n] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TT / 4; ++i) {
    const int nr = ty + 4 * i;
    const int n = n0 + nr, k = k0 + tx;
    if (n < N && k < K) {
      uint16_t v = tile[tx][nr];
      if (TO_F16) v = float_to_f16_bits(bf16_bits_to_float(v));
      WT[(size_t)n * K + k] = v;
    }
  }
}

// One workgroup per batch element: largest unmasked key index + 1.
__global__ void __launch_bounds__(256)
mask_extent_kernel(const uint8_t* __restrict__ mask, int T_k, int* __restrict__ kend) {
  __shared__ int red[4];
  const int b = blockIdx.x;
  int last = -1;
  for (int j = threadIdx.x; j < T_k; j += 256)
    if (mask[(size_t)b * T_k + j] == 0) last = j;
  for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = last;
  __syncthreads();
  if (threadIdx.x == 0) kend[b] = max(max(red[0], red[1]), max(red[2], red[3])) + 1;
}

}  // namespace

hipError_t launch_transpose_bf16(const uint16_t* W, int K, int N, uint16_t* WT, bool to_f16,
                                 hipStream_t s) {
  dim3 grid((N + TT - 1) / TT, (K + TT - 1) / TT);
  if (to_f16)
    hipLaunchKernelGGL(transpose_bf16_kernel<true>, grid, dim3(256), 0, s, W, K, N, WT);
  else
    hipLaunchKernelGGL(transpose_bf16_kernel<false>, grid, dim3(256), 0, s, W, K, N, WT);
  return hipGetLastError();
}

hipError_t launch_mask_extent(const uint8_t* mask, int B, int T_k, int* kend, hipStream_t s) {
  hipLaunchKernelGGL(mask_extent_kernel, dim3(B), dim3(256), 0, s, mask, T_k, kend);
  return hipGetLastError();
}

}  // namespace mha
