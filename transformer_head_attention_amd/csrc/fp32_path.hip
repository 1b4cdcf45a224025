// fp32 kernels: the whole path for fp32 inputs.
//
//  * gemm_f32: C = A . B + bias with v_mfma_f32_16x16x4_f32 (full fp32
//    products and sums); B and bias may be stored as bf16 (converted exactly).
//    64- or 128-deep K slices, the next one loaded into registers under the
//    current one's MFMAs; 32 x 32 tiles when 64 x 64 ones would not fill the
//    CUs.
//    Used for X . W_QKV and O . W_O (itwiki "멀티 헤드 어텐션",
//    텐서 모양으로 본 계산, 투영 and 출력 투영 rows).
//  * attn_f32: softmax(q . k / sqrt(d_k) + M) v row by row in fp32
//    (same page, 수식; iamjaehka13.blog "[Deep Learning 5]", §7-§13). Each
//    query row is shared by d_k/16 lanes that each own 16 of its dimensions;
//    keys are staged through LDS in chunks of 64, split over the four waves
//    of a workgroup, folded into running max / sum states that are merged at
//    the end.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

// TBM x TBN tile per workgroup (4 waves, 2 x 2, of TBM/2 x TBN/2), K in
// TBK-deep slices; the next slice is loaded into registers while the current
// one is multiplied from LDS, so each slice costs one global latency at most
// once. Small problems take 32 x 32 tiles (more workgroups) and deep K takes
// 128-deep slices (half the latency-bound steps).
template <bool B_BF16, int TBM, int TBN, int TBK>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, int lda, int M, int K, const void* __restrict__ Bv,
                int ldb, int N, const void* __restrict__ biasv, float* __restrict__ C, int ldc,
                int rows_in, int rows_out) {
  static_assert(TBM % 32 == 0 && TBN % 32 == 0 && TBK % 64 == 0, "tile shape");
  constexpr int WI = TBM / 32, WJ = TBN / 32;     // 16 x 16 blocks per wave
  constexpr int ACH = TBK / 4, BCH = TBN / 4, BCH8 = TBN / 8;
  constexpr int A_V4 = TBM * TBK / 4 / 256;       // float4 loads per thread
  constexpr int B_V4 = TBK * TBN / 4 / 256;
  constexpr int B_H8 = TBK * TBN / 8 / 256;       // 8 x bf16 loads per thread
  static_assert(A_V4 * 1024 == TBM * TBK && B_H8 * 2048 == TBK * TBN, "loads per thread");
  __shared__ float As[TBM][TBK + 1];
  __shared__ float Bs[TBK][TBN + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * TBM, n0 = blockIdx.x * TBN;

  f32x4_t acc[WI][WJ];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A slice: TBM rows x TBK k; B slice: TBK k x TBN n, as float4 (fp32) or
  // 8 x bf16 per load. Rows past M are clamped (never stored); N is a
  // multiple of TBN here.
  f32x4_t ra[A_V4], rb[B_BF16 ? 1 : B_V4];
  u32x4 rbh[B_BF16 ? B_H8 : 1];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_V4; ++i) {
      const int p = i * 256 + tid, row = p / ACH, c = (p % ACH) * 4;
      ra[i] = *reinterpret_cast<const f32x4_t*>(A + (size_t)min(m0 + row, M - 1) * lda + k0 + c);
    }
    if constexpr (!B_BF16) {
      const float* Bf = static_cast<const float*>(Bv);
#pragma unroll
      for (int i = 0; i < B_V4; ++i) {
        const int p = i * 256 + tid, row = p / BCH, c = (p % BCH) * 4;
        rb[i] = *reinterpret_cast<const f32x4_t*>(Bf + (size_t)(k0 + row) * ldb + n0 + c);
      }
    } else {
      const uint16_t* Bb = static_cast<const uint16_t*>(Bv);
#pragma unroll
      for (int i = 0; i < B_H8; ++i) {
        const int p = i * 256 + tid, row = p / BCH8, c = (p % BCH8) * 8;
        rbh[i] = *reinterpret_cast<const u32x4*>(Bb + (size_t)(k0 + row) * ldb + n0 + c);
      }
    }
  };
  auto stash = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_V4; ++i) {
      const int p = i * 256 + tid, row = p / ACH, c = (p % ACH) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) As[row][c + e] = ra[i][e];
    }
    if constexpr (!B_BF16) {
#pragma unroll
      for (int i = 0; i < B_V4; ++i) {
        const int p = i * 256 + tid, row = p / BCH, c = (p % BCH) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[row][c + e] = rb[i][e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_H8; ++i) {
        const int p = i * 256 + tid, row = p / BCH8, c = (p % BCH8) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Bs[row][c + 2 * e] = __uint_as_float(rbh[i][e] << 16);
          Bs[row][c + 2 * e + 1] = __uint_as_float(rbh[i][e] & 0xffff0000u);
        }
      }
    }
  };

  load(0);
  for (int k0 = 0; k0 < K; k0 += TBK) {
    stash();
    __syncthreads();
    if (k0 + TBK < K) load(k0 + TBK);
#pragma unroll
    for (int kk = 0; kk < TBK / 4; ++kk) {
      float av[WI], bv[WJ];
#pragma unroll
      for (int i = 0; i < WI; ++i)
        av[i] = As[wm * (TBM / 2) + i * 16 + (lane & 15)][kk * 4 + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < WJ; ++j)
        bv[j] = Bs[kk * 4 + (lane >> 4)][wn * (TBN / 2) + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j) acc[i][j] = mfma16x16x4f32(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int n = n0 + wn * (TBN / 2) + j * 16 + (lane & 15);
    if (n >= N) continue;
    float bias = 0.0f;
    if (biasv) {
      bias = B_BF16 ? bf16_bits_to_float(static_cast<const uint16_t*>(biasv)[n])
                    : static_cast<const float*>(biasv)[n];
    }
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (TBM / 2) + i * 16 + 4 * (lane >> 4) + r;
        if (m < M) {
          const int g = m / rows_in;
          const size_t out_row = (size_t)g * rows_out + (m - g * rows_in);
          C[out_row * ldc + n] = acc[i][j][r] + bias;
        }
      }
  }
}

constexpr int KC = 64;           // keys per LDS chunk
constexpr int ATTN32_NT = 256;   // threads per workgroup (4 waves)
constexpr int KW = KC / 4;       // keys of a chunk per wave

// A workgroup takes 64 / (d_k/16) query rows (16 at d_k = 64, 8 at 128);
// each wave holds all of them and takes a quarter of every 64-key chunk
// (keys 16 w .. 16 w + 15), with its own running max, sum and accumulator;
// the four partial states are merged through LDS at the end. Scores in log2
// units (q . k times log2(e)/sqrt(d_k)), exponentials exp2.
template <int DK>
__global__ void __launch_bounds__(ATTN32_NT)
attn_f32_kernel(AttnF32Args a) {
  constexpr int TPR = DK / 16;    // lanes per query row
  constexpr int RPB = 64 / TPR;   // query rows per workgroup
  __shared__ __attribute__((aligned(16))) float Ks[KC][DK];
  __shared__ __attribute__((aligned(16))) float Vs[KC][DK];
  __shared__ uint8_t Ms[KC];
  __shared__ float m_s[4][RPB], l_s[4][RPB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane / TPR, p = lane % TPR;
  const int head = blockIdx.y, b = blockIdx.z;
  const int t = blockIdx.x * RPB + r;
  const bool valid = t < a.rows;
  const float scale = 1.4426950408889634f / sqrtf((float)DK);

  float q[16], acc[16];
  const float* qp = a.q + (size_t)b * a.q_bstride + (size_t)(valid ? t : 0) * a.q_ld + head * DK +
                    p * 16;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    q[c] = valid ? qp[c] * scale : 0.0f;
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  int kend = a.T_k;
  if (a.causal) kend = min(kend, blockIdx.x * RPB + RPB);
  const float* kb = a.k + (size_t)b * a.kv_bstride + (head / a.group) * DK;
  const float* vb = a.v + (size_t)b * a.kv_bstride + (head / a.group) * DK;
  const uint8_t* mb = a.mask ? a.mask + (size_t)b * a.mask_ld : nullptr;

  // Chunk loads go to registers first: the next chunk's are in flight while
  // the current one is used from LDS.
  constexpr int LD = KC * DK / 4 / ATTN32_NT;   // float4 of K (and of V) per thread
  static_assert(LD * ATTN32_NT * 4 == KC * DK, "chunk / thread mismatch");
  float4 kr[LD], vr[LD];
  uint8_t mr = 0;
  auto load_chunk = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int idx = it * ATTN32_NT + tid, key = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
      const int j = j0 + key;
      kr[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      vr[it] = kr[it];
      if (j < a.T_k) {
        kr[it] = *reinterpret_cast<const float4*>(kb + (size_t)j * a.kv_ld + c4);
        vr[it] = *reinterpret_cast<const float4*>(vb + (size_t)j * a.kv_ld + c4);
      }
    }
    if (tid < KC) mr = (mb && j0 + tid < a.T_k) ? mb[j0 + tid] : 0;
  };
  if (kend > 0) load_chunk(0);
  for (int j0 = 0; j0 < kend; j0 += KC) {
    __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int idx = it * ATTN32_NT + tid, key = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
      *reinterpret_cast<float4*>(&Ks[key][c4]) = kr[it];
      *reinterpret_cast<float4*>(&Vs[key][c4]) = vr[it];
    }
    if (tid < KC) Ms[tid] = mr;
    __syncthreads();
    if (j0 + KC < kend) load_chunk(j0 + KC);

    float s[KW];
    float cmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < KW; ++jj) {
      const int kk = wave * KW + jj, j = j0 + kk;
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) part = __builtin_fmaf(q[c], Ks[kk][p * 16 + c], part);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) part += __shfl_xor(part, off);
      const bool ign = j >= a.T_k || (a.causal && j > t) || Ms[kk] != 0;
      s[jj] = ign ? -INFINITY : part;
      cmax = fmaxf(cmax, s[jj]);
    }
    const float m_new = fmaxf(m, cmax);
    const float base = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = exp2f(m - base);
    l *= corr;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] *= corr;
#pragma unroll
    for (int jj = 0; jj < KW; ++jj) {
      const float pj = exp2f(s[jj] - base);
      l += pj;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = __builtin_fmaf(pj, Vs[wave * KW + jj][p * 16 + c], acc[c]);
    }
    m = m_new;
  }

  // Merge the four waves' states (wave order, fixed): Ks holds the
  // accumulators once every wave is past the last chunk.
  __syncthreads();
  float (*accs)[RPB][DK] = reinterpret_cast<float (*)[RPB][DK]>(&Ks[0][0]);
  static_assert(4 * RPB * DK <= KC * DK, "merge buffer");
#pragma unroll
  for (int c = 0; c < 16; ++c) accs[wave][r][p * 16 + c] = acc[c];
  if (p == 0) {
    m_s[wave][r] = m;
    l_s[wave][r] = l;
  }
  __syncthreads();
  if (wave != 0 || !valid) return;
  float mx = m_s[0][r];
#pragma unroll
  for (int w = 1; w < 4; ++w) mx = fmaxf(mx, m_s[w][r]);
  const float base = mx == -INFINITY ? 0.0f : mx;
  float lt = 0.0f, o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float f = exp2f(m_s[w][r] - base);   // 0 for a wave that saw no key
    lt += l_s[w][r] * f;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] = __builtin_fmaf(accs[w][r][p * 16 + c], f, o[c]);
  }
  // gated attention: the head's output row times its gate
  const float gt = a.gate ? gate_sigmoid(a.gate[(size_t)b * a.gate_bstride + (size_t)t * a.h + head])
                          : 1.0f;
  float* op = a.o + (size_t)b * a.o_bstride + (size_t)t * a.o_ld + head * DK + p * 16;
#pragma unroll
  for (int c = 0; c < 16; ++c) op[c] = o[c] / lt * gt;   // all keys masked: 0 / 0 = NaN
}

}  // namespace

namespace {
template <int TBM, int TBN, int TBK>
void launch_gemm_f32_tiles(const float* A, int lda, int M, int K, const void* B, int ldb, int N,
                           bool b_bf16, const void* bias, float* C, int ldc, int rows_in,
                           int rows_out, hipStream_t s) {
  dim3 grid(N / TBN, (M + TBM - 1) / TBM);
  if (b_bf16)
    hipLaunchKernelGGL((gemm_f32_kernel<true, TBM, TBN, TBK>), grid, dim3(256), 0, s, A, lda, M, K,
                       B, ldb, N, bias, C, ldc, rows_in, rows_out);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<false, TBM, TBN, TBK>), grid, dim3(256), 0, s, A, lda, M,
                       K, B, ldb, N, bias, C, ldc, rows_in, rows_out);
}
}  // namespace

hipError_t launch_gemm_f32(const float* A, int lda, int M, int K, const void* B, int ldb, int N,
                           bool b_bf16, const void* bias, float* C, int ldc, int rows_in,
                           int rows_out, hipStream_t s) {
  if (K % 64 != 0 || N % 64 != 0 || M < 1) return hipErrorInvalidValue;
  // 64 x 64 tiles once they fill the 256 CUs, else 32 x 32 (four times the
  // workgroups); 128-deep K slices when K allows.
  const bool big = (long long)(N / 64) * ((M + 63) / 64) >= 256, deep = K % 128 == 0;
  if (big && deep)
    launch_gemm_f32_tiles<64, 64, 128>(A, lda, M, K, B, ldb, N, b_bf16, bias, C, ldc, rows_in,
                                       rows_out, s);
  else if (big)
    launch_gemm_f32_tiles<64, 64, 64>(A, lda, M, K, B, ldb, N, b_bf16, bias, C, ldc, rows_in,
                                      rows_out, s);
  else if (deep)
    launch_gemm_f32_tiles<32, 32, 128>(A, lda, M, K, B, ldb, N, b_bf16, bias, C, ldc, rows_in,
                                       rows_out, s);
  else
    launch_gemm_f32_tiles<32, 32, 64>(A, lda, M, K, B, ldb, N, b_bf16, bias, C, ldc, rows_in,
                                      rows_out, s);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnF32Args& a, int d_k, hipStream_t s) {
  if (a.group < 1 || a.h % a.group != 0) return hipErrorInvalidValue;
  if (d_k == 64) {
    constexpr int rpb = 64 / 4;
    dim3 grid((a.rows + rpb - 1) / rpb, a.h, a.B);
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(ATTN32_NT), 0, s, a);
  } else if (d_k == 128) {
    constexpr int rpb = 64 / 8;
    dim3 grid((a.rows + rpb - 1) / rpb, a.h, a.B);
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(ATTN32_NT), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mha
