// Gate pre-activations of gated attention (itwiki "멀티 헤드 어텐션",
// 추론 비용과 변형, last paragraph: each head's scaled dot-product attention
// output is multiplied by a sigmoid gate of its own). One gate per row of the
// query-side input and head:
//   g[m][n] = x[m] . W_G[:, n] + b_G[n],   m < M rows, n < h heads,
// stored in fp32; the attention kernels multiply head n's output row m by
// 1 / (1 + exp(-g[m][n])) when they store it.
#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int GATE_UNROLL = 8;   // 16-deep k-steps per batch of loads (D % 128 == 0)

// bf16: one wave per 32 rows and 32 gates, v_mfma_f32_32x32x16_bf16 with the
// rows as the A operand and the gates (rows of W_G^T, K-contiguous) as B:
// lane l supplies row / gate l % 32 and the 8 k-values (l / 32) * 8 .. + 7 of
// each 16-deep step, 16 bytes straight from global memory, all loads of 8
// steps in flight before their MFMAs. The result holds gate n0 + l % 32 of
// rows 8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15.
__global__ void __launch_bounds__(256)
gate_bf16_kernel(const uint16_t* __restrict__ x, int M, int D, const uint16_t* __restrict__ wgT,
                 const uint16_t* __restrict__ bias, int h, float* __restrict__ g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r0 = ((int)blockIdx.x * 4 + wave) * 32;
  if (r0 >= M) return;
  const int lq = lane & 31, kh = (lane >> 5) * 8;
  const uint16_t* xr = x + (size_t)min(r0 + lq, M - 1) * D + kh;   // rows past M: never stored
  for (int n0 = 0; n0 < h; n0 += 32) {
    const int n = n0 + lq;
    const bool live = n < h;
    const uint16_t* wr = wgT + (size_t)(live ? n : 0) * D + kh;
    f32x16_t acc = {};
    for (int k0 = 0; k0 < D; k0 += 16 * GATE_UNROLL) {
      u32x4 a[GATE_UNROLL], b[GATE_UNROLL];
#pragma unroll
      for (int u = 0; u < GATE_UNROLL; ++u) {
        a[u] = *reinterpret_cast<const u32x4*>(xr + k0 + 16 * u);
        b[u] = *reinterpret_cast<const u32x4*>(wr + k0 + 16 * u);
      }
#pragma unroll
      for (int u = 0; u < GATE_UNROLL; ++u) {
        if (!live) b[u] = u32x4{0u, 0u, 0u, 0u};
        acc = mfma32x32x16<BF16>(a[u], b[u], acc);
      }
    }
    if (live) {
      const float bn = load_bias_bf16(bias, n);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M) g[(size_t)m * h + n] = acc[r] + bn;
      }
    }
  }
}

// fp32: one thread per (row, gate), the dot product in fp32 in k order.
__global__ void __launch_bounds__(256)
gate_f32_kernel(const float* __restrict__ x, int M, int D, const float* __restrict__ wg,
                const float* __restrict__ bias, int h, float* __restrict__ g) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * h) return;
  const int m = (int)(i / h), n = (int)(i - (long long)m * h);
  const float* xr = x + (size_t)m * D;
  float acc = 0.0f;
  for (int k = 0; k < D; ++k) acc = __builtin_fmaf(xr[k], wg[(size_t)k * h + n], acc);
  g[i] = acc + (bias ? bias[n] : 0.0f);
}

}  // namespace

hipError_t launch_gate_bf16(const uint16_t* x, int M, int D, const uint16_t* wgT,
                            const uint16_t* bias, int h, float* g, hipStream_t s) {
  if (M < 1 || h < 1 || D < 16 * GATE_UNROLL || D % (16 * GATE_UNROLL) != 0)
    return hipErrorInvalidValue;
  const long long blocks = ((long long)M + 127) / 128;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gate_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, M, D, wgT, bias,
                     h, g);
  return hipGetLastError();
}

hipError_t launch_gate_f32(const float* x, int M, int D, const float* wg, const float* bias, int h,
                           float* g, hipStream_t s) {
  if (M < 1 || h < 1 || D < 1) return hipErrorInvalidValue;
  const long long blocks = ((long long)M * h + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, M, D, wg, bias, h,
                     g);
  return hipGetLastError();
}

}  // namespace mha
