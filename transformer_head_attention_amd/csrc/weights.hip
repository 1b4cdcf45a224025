// Inspection outputs of the forward pass.
//
// attn_weights_kernel: the attention weights themselves, per head (B, h, T_q,
// T_k) or averaged over heads (B, T_q, T_k), the two forms nn.MultiheadAttention
// returns (molayo1419.me, return values: head-averaged by default, per head
// with average_attn_weights=False). The weights are
// softmax(QK^T/sqrt(d_k) + M) of itwiki "멀티 헤드 어텐션", 수식, recomputed
// from the Q and K the forward pass already holds, one score row at a time:
// a pass for the scores and their maximum, one for the sum of exponentials,
// one for the normalised row. Meant for small problems (T_k <= 4096: the
// row lives in LDS).
//
// add_residual_f32_kernel: y += x (the residual output of the fp32 path;
// iamjaehka13.blog "[Deep Learning 5]", §14).
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float load_elem(const void* p, size_t i, bool f16) {
  return f16 ? f16_bits_to_float(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// One wave per (query row t, batch element b); heads in turn. Lane j-strided
// over the keys.
__global__ void __launch_bounds__(64)
attn_weights_kernel(WeightsArgs a) {
  extern __shared__ float row[];   // T_k scores, then weights
  __shared__ float qv[128];
  const int lane = threadIdx.x, t = blockIdx.x, b = blockIdx.y;
  const bool f16 = a.f16 != 0;
  float* avg = row + a.T_k;        // running head average (average mode)
  if (a.average)
    for (int j = lane; j < a.T_k; j += 64) avg[j] = 0.0f;
  for (int head = 0; head < a.h; ++head) {
    const size_t qo = (size_t)b * a.q_bs + (size_t)head * a.q_hs + (size_t)t * a.q_ld;
    for (int c = lane; c < a.d_k; c += 64) qv[c] = load_elem(a.q, qo + c, f16);
    __syncthreads();
    const size_t ko = (size_t)b * a.k_bs + (size_t)(head / a.group) * a.k_hs;
    float mx = -INFINITY;
    for (int j = lane; j < a.T_k; j += 64) {
      bool ign = (a.causal && j > t) || (a.mask && a.mask[(size_t)b * a.T_k + j] != 0);
      float s = -INFINITY;
      if (!ign) {
        float d = 0.0f;
        const size_t kr = ko + (size_t)j * a.k_ld;
        for (int c = 0; c < a.d_k; ++c) d += qv[c] * load_elem(a.k, kr + c, f16);
        s = d * a.score_scale;
      }
      row[j] = s;
      mx = fmaxf(mx, s);
    }
    mx = wmax(mx);
    float sum = 0.0f;
    for (int j = lane; j < a.T_k; j += 64) {
      const float e = mx == -INFINITY ? 0.0f : exp2f(row[j] - mx);
      row[j] = e;
      sum += e;
    }
    sum = wsum(sum);
    const float inv = 1.0f / sum;   // all keys masked: 0 * inf = NaN, as 0/0
    float* out = a.out + (((size_t)b * a.h + head) * a.T_q + t) * a.T_k;
    for (int j = lane; j < a.T_k; j += 64) {
      const float w = row[j] * inv;
      if (a.average)
        avg[j] += w;
      else
        out[j] = w;
    }
    __syncthreads();
  }
  if (a.average) {
    float* out = a.out + ((size_t)b * a.T_q + t) * a.T_k;
    for (int j = lane; j < a.T_k; j += 64) out[j] = avg[j] / (float)a.h;
  }
}

__global__ void __launch_bounds__(256)
add_residual_f32_kernel(float* __restrict__ y, const float* __restrict__ x, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] += x[i];
}

}  // namespace

hipError_t launch_attn_weights(const WeightsArgs& a, hipStream_t s) {
  if (a.T_k < 1 || a.T_k > kWeightsMaxKeys || a.d_k > 128 || a.group < 1 || a.h % a.group != 0 ||
      a.B > 65535)
    return hipErrorInvalidValue;
  const size_t lds = (size_t)a.T_k * sizeof(float) * (a.average ? 2 : 1);
  hipLaunchKernelGGL(attn_weights_kernel, dim3(a.T_q, a.B), dim3(64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_add_residual_f32(float* y, const float* x, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_residual_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, x,
                     n);
  return hipGetLastError();
}

}  // namespace mha
