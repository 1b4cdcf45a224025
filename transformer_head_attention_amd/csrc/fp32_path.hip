// fp32 kernels: the whole path for fp32 inputs.
//
//  * gemm_f32: C = A . B + bias with v_mfma_f32_16x16x4_f32 (full fp32
//    products and sums); B and bias may be stored as bf16 (converted exactly).
//    Used for X . W_QKV and O . W_O (itwiki "멀티 헤드 어텐션",
//    텐서 모양으로 본 계산, 투영 and 출력 투영 rows).
//  * attn_f32: softmax(q . k / sqrt(d_k) + M) v row by row in fp32
//    (same page, 수식; iamjaehka13.blog "[Deep Learning 5]", §7-§13). Each
//    query row is shared by d_k/16 lanes that each own 16 of its dimensions;
//    keys are staged through LDS in chunks of 64 and folded into a running
//    max / running sum.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool B_BF16>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, int lda, int M, int K, const void* __restrict__ Bv,
                int ldb, int N, const void* __restrict__ biasv, float* __restrict__ C, int ldc,
                int rows_in, int rows_out) {
  __shared__ float As[FBM][FBK + 1];
  __shared__ float Bs[FBK][FBN + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * FBM, n0 = blockIdx.x * FBN;

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += FBK) {
    {
      const int row = tid >> 2, c = (tid & 3) * 4;
      const int m = min(m0 + row, M - 1);
      const float4 v = *reinterpret_cast<const float4*>(A + (size_t)m * lda + k0 + c);
      As[row][c] = v.x; As[row][c + 1] = v.y; As[row][c + 2] = v.z; As[row][c + 3] = v.w;
    }
    if (!B_BF16) {
      const float* Bf = static_cast<const float*>(Bv);
      const int row = tid >> 4, c = (tid & 15) * 4;
      const float4 v = *reinterpret_cast<const float4*>(Bf + (size_t)(k0 + row) * ldb + n0 + c);
      Bs[row][c] = v.x; Bs[row][c + 1] = v.y; Bs[row][c + 2] = v.z; Bs[row][c + 3] = v.w;
    } else if (tid < 128) {
      const uint16_t* Bb = static_cast<const uint16_t*>(Bv);
      const int row = tid >> 3, c = (tid & 7) * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(Bb + (size_t)(k0 + row) * ldb + n0 + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Bs[row][c + 2 * e] = __uint_as_float(w[e] << 16);
        Bs[row][c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK / 4; ++kk) {
      float av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = As[wm * 32 + i * 16 + (lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = Bs[kk * 4 + (lane >> 4)][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x4f32(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 32 + j * 16 + (lane & 15);
    if (n >= N) continue;
    float bias = 0.0f;
    if (biasv) {
      bias = B_BF16 ? bf16_bits_to_float(static_cast<const uint16_t*>(biasv)[n])
                    : static_cast<const float*>(biasv)[n];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
        if (m < M) {
          const int g = m / rows_in;
          const size_t out_row = (size_t)g * rows_out + (m - g * rows_in);
          C[out_row * ldc + n] = acc[i][j][r] + bias;
        }
      }
  }
}

constexpr int KC = 64;           // keys per LDS chunk
constexpr int ATTN32_NT = 256;   // threads per workgroup

template <int DK>
__global__ void __launch_bounds__(ATTN32_NT)
attn_f32_kernel(AttnF32Args a) {
  constexpr int TPR = DK / 16;           // lanes per query row
  constexpr int RPB = ATTN32_NT / TPR;   // query rows per workgroup
  __shared__ __attribute__((aligned(16))) float Ks[KC][DK];
  __shared__ __attribute__((aligned(16))) float Vs[KC][DK];

  const int tid = threadIdx.x, r = tid / TPR, p = tid % TPR;
  const int head = blockIdx.y, b = blockIdx.z;
  const int t = blockIdx.x * RPB + r;
  const bool valid = t < a.rows;
  const float scale = 1.0f / sqrtf((float)DK);

  float q[16], acc[16];
  const float* qp = a.q + (size_t)b * a.q_bstride + (size_t)t * a.q_ld + head * DK + p * 16;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    q[c] = valid ? qp[c] : 0.0f;
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  int kend = a.T_k;
  if (a.causal) kend = min(kend, blockIdx.x * RPB + RPB);
  const float* kb = a.k + (size_t)b * a.kv_bstride + (head / a.group) * DK;
  const float* vb = a.v + (size_t)b * a.kv_bstride + (head / a.group) * DK;
  const uint8_t* mb = a.mask ? a.mask + (size_t)b * a.mask_ld : nullptr;

  for (int j0 = 0; j0 < kend; j0 += KC) {
    __syncthreads();
    for (int idx = tid; idx < KC * DK / 4; idx += ATTN32_NT) {
      const int key = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4, j = j0 + key;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (j < a.T_k) {
        kv = *reinterpret_cast<const float4*>(kb + (size_t)j * a.kv_ld + c4);
        vv = *reinterpret_cast<const float4*>(vb + (size_t)j * a.kv_ld + c4);
      }
      *reinterpret_cast<float4*>(&Ks[key][c4]) = kv;
      *reinterpret_cast<float4*>(&Vs[key][c4]) = vv;
    }
    __syncthreads();

    float s[KC];
    float cmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < KC; ++jj) {
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) part = __builtin_fmaf(q[c], Ks[jj][p * 16 + c], part);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) part += __shfl_xor(part, off);
      const int j = j0 + jj;
      const bool ign = j >= a.T_k || (a.causal && j > t) || (mb && mb[j] != 0);
      s[jj] = ign ? -INFINITY : part * scale;
      cmax = fmaxf(cmax, s[jj]);
    }
    const float m_new = fmaxf(m, cmax);
    const float base = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = expf(m - base);
    l *= corr;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] *= corr;
#pragma unroll
    for (int jj = 0; jj < KC; ++jj) {
      const float pj = expf(s[jj] - base);
      l += pj;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = __builtin_fmaf(pj, Vs[jj][p * 16 + c], acc[c]);
    }
    m = m_new;
  }

  if (valid) {
    float* op = a.o + (size_t)b * a.o_bstride + (size_t)t * a.o_ld + head * DK + p * 16;
#pragma unroll
    for (int c = 0; c < 16; ++c) op[c] = acc[c] / l;
  }
}

}  // namespace

hipError_t launch_gemm_f32(const float* A, int lda, int M, int K, const void* B, int ldb, int N,
                           bool b_bf16, const void* bias, float* C, int ldc, int rows_in,
                           int rows_out, hipStream_t s) {
  dim3 grid((N + FBN - 1) / FBN, (M + FBM - 1) / FBM);
  if (b_bf16)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, s, A, lda, M, K, B, ldb, N, bias,
                       C, ldc, rows_in, rows_out);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, s, A, lda, M, K, B, ldb, N,
                       bias, C, ldc, rows_in, rows_out);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnF32Args& a, int d_k, hipStream_t s) {
  if (a.group < 1 || a.h % a.group != 0) return hipErrorInvalidValue;
  if (d_k == 64) {
    dim3 grid((a.rows + 63) / 64, a.h, a.B);
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(ATTN32_NT), 0, s, a);
  } else if (d_k == 128) {
    dim3 grid((a.rows + 31) / 32, a.h, a.B);
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(ATTN32_NT), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mha
