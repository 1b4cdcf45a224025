// One generation step against a KV cache (itwiki "멀티 헤드 어텐션", section
// 추론 비용과 변형: each step reads every cached key and value, so the step is
// bound by memory bandwidth; iamjaehka13.blog "[Deep Learning 5]", §21: the
// cache keeps the earlier tokens' keys and values so that they are not
// recomputed).
//
// Kernels, in launch order:
//   rows_gemm_kernel      partial products of a few rows X (M = B*T_new) with a
//                         row-major weight matrix, split over K; MFMA with the
//                         weight tile transposed through LDS.
//   decode_route_kernel   sums the K split, adds the bias and routes the
//                         columns: Q (fp32 and fp16, pre-scaled), K and V
//                         (fp32 copies for this step; bf16 rows appended to the
//                         caches).
//   decode_split_kernel   attention of the new query rows over one chunk of
//                         cached keys: partial (max, sum, unnormalised output)
//                         per query row. One wave per (chunk, key/value set,
//                         32-row query block, batch element).
//   decode_merge_kernel   merges the chunks, adds the new tokens' own keys
//                         (causal among the new tokens) in fp32, normalises.
//   rows_gemm_kernel + decode_out_kernel   Y = O . W_O + b_O.
#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Eight bf16 values -> eight fp16 values (exact for normal-range values).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4& r) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_f16x2(__uint_as_float(r[i] << 16), __uint_as_float(r[i] & 0xffff0000u));
  return o;
}

// Position of key k (0..63) of a tile inside a transposed V row: bits 2 and 3
// swapped, so that the 8 keys one lane half feeds to a P.V MFMA step are
// contiguous (same order as the score accumulator rows of that lane half).
__device__ __forceinline__ int vt_slot(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// ---------------------------------------------------------------------------
// Skinny GEMM: part[ks][m][n] = sum over k in slice ks of X[m][k] * W[k][n].
// X (M x K) row-major, bf16 or fp32 (fp32 rows are split into bf16 hi + lo
// parts, two MFMAs); W (K x N) bf16 row-major. Workgroup: 4 waves, 32 rows x
// 128 columns (32 per wave); the weight slab is staged in LDS row-major and
// each lane gathers its 8 k-values of one column for the MFMA B operand.
constexpr int RG_N = 128;
constexpr int RG_K = 64;

template <bool X_F32>
__global__ void __launch_bounds__(256)
rows_gemm_kernel(const void* __restrict__ Xv, int M, int K, const uint16_t* __restrict__ W, int N,
                 int KR, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[RG_K][RG_N + 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * RG_N, ks = blockIdx.y, m0 = blockIdx.z * 32;
  const int k0 = ks * KR, kn = min(KR, K - k0);
  const int lq = lane & 31, kg = lane >> 5;
  const int m = m0 + lq;
  f32x16_t acc = {};
  for (int kk = 0; kk < kn; kk += RG_K) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RG_K * RG_N / 8 / 256; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n0 + col < N) v = *reinterpret_cast<const u32x4*>(W + (size_t)(k0 + kk + row) * N + n0 + col);
      *reinterpret_cast<u32x4*>(&ws[row][col]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < RG_K / 16; ++s) {
      const int kx = k0 + kk + 16 * s + 8 * kg;
      u32x4 a = {0u, 0u, 0u, 0u}, alo = {0u, 0u, 0u, 0u};
      if (m < M) {
        if constexpr (X_F32) {
          const float* xr = static_cast<const float*>(Xv) + (size_t)m * K + kx;
          const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(xr);
          const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(xr + 4);
          float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t h0 = float_to_bf16_bits(xv[2 * e]), h1 = float_to_bf16_bits(xv[2 * e + 1]);
            const uint16_t l0 = float_to_bf16_bits(xv[2 * e] - bf16_bits_to_float(h0));
            const uint16_t l1 = float_to_bf16_bits(xv[2 * e + 1] - bf16_bits_to_float(h1));
            a[e] = h0 | (uint32_t)h1 << 16;
            alo[e] = l0 | (uint32_t)l1 << 16;
          }
        } else {
          a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Xv) + (size_t)m * K + kx);
        }
      }
      u32x4 b;
      const int col = wave * 32 + lq, r0 = 16 * s + 8 * kg;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        b[e] = ws[r0 + 2 * e][col] | (uint32_t)ws[r0 + 2 * e + 1][col] << 16;
      acc = mfma32x32x16<BF16>(a, b, acc);
      if constexpr (X_F32) acc = mfma32x32x16<BF16>(alo, b, acc);
    }
  }
  const int n = n0 + wave * 32 + lq;
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mr = m0 + 8 * (i >> 2) + 4 * kg + (i & 3);
      if (mr < M) part[((size_t)ks * M + mr) * N + n] = acc[i];
    }
  }
}

__device__ __forceinline__ int clamp_len(const int* len, int b, int T_max, int T_new) {
  return min(max(len[b], 0), T_max - T_new);
}

// Sum of the K split plus bias, routed by column of [Q | K | V].
__global__ void __launch_bounds__(256)
decode_route_kernel(DecodeArgs a, const float* __restrict__ part, int KS) {
  const int N = a.D + 2 * a.Dkv;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const int M = a.B * a.T_new;
  if (idx >= (long long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx - (long long)m * N);
  float v = 0.0f;
  for (int s = 0; s < KS; ++s) v += part[((size_t)s * M + m) * N + n];
  if (a.b_qkv) v += bf16_bits_to_float(a.b_qkv[n]);
  const int b = m / a.T_new, t = m - b * a.T_new, DK = a.d_k;
  if (n < a.D) {
    const float qv = v * a.q_scale;
    a.q32[(size_t)m * a.D + n] = qv;
    const int head = n / DK, c = n - head * DK;
    a.q16[(((size_t)b * a.h + head) * a.T_new + t) * DK + c] = float_to_f16_bits(qv);
    return;
  }
  const bool is_k = n < a.D + a.Dkv;
  const int nc = n - a.D - (is_k ? 0 : a.Dkv);
  const int g = nc / DK, c = nc - g * DK;
  (is_k ? a.k32 : a.v32)[(size_t)m * a.Dkv + nc] = v;
  const int L = clamp_len(a.cache_len, b, a.T_max, a.T_new);
  uint16_t* cache = is_k ? a.k_cache : a.v_cache;
  cache[(((size_t)b * a.h_kv + g) * a.T_max + L + t) * DK + c] = float_to_bf16_bits(v);
}

// ---------------------------------------------------------------------------
// Attention of up to 32 query rows (the query heads of one key/value set times
// the new tokens) over cached keys [p*CW, min((p+1)*CW, L)). S^T = K Q^T with
// the K rows read from the cache straight into the MFMA A operand (bf16 ->
// fp16, exact); each lane owns one query row's scores. V is staged transposed
// in LDS (fp16), in the slot order of the P operand. Output: the running max,
// sum and unnormalised O of every row, in log2 units (Q carries log2(e)/sqrt(d_k)).
template <int DK>
__global__ void __launch_bounds__(64)
decode_split_kernel(DecodeArgs a) {
  constexpr int KSTEP = DK / 16, DB = DK / 32;
  __shared__ __attribute__((aligned(16))) uint16_t vts[DK][64 + 8];
  const int lane = threadIdx.x, lq = lane & 31, kg = lane >> 5;
  const int p = blockIdx.x, b = blockIdx.z;
  const int g = blockIdx.y / a.nqb, qb = blockIdx.y - g * a.nqb;
  const int L = clamp_len(a.cache_len, b, a.T_max, a.T_new);
  const int kbeg = p * a.CW;
  if (kbeg >= L) return;
  const int kend = min(kbeg + a.CW, L);
  const int G = (a.h / a.h_kv) * a.T_new;

  // Q^T operand: lane supplies query row qb*32 + lq (zero past G).
  u32x4 qf[KSTEP];
  const int row = qb * 32 + lq;
  const uint16_t* qrow = a.q16 + (((size_t)b * a.h_kv + g) * G + row) * DK;
#pragma unroll
  for (int s = 0; s < KSTEP; ++s) {
    qf[s] = u32x4{0u, 0u, 0u, 0u};
    if (row < G) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * kg);
  }
  const uint16_t* Kc = a.k_cache + ((size_t)b * a.h_kv + g) * a.T_max * DK;
  const uint16_t* Vc = a.v_cache + ((size_t)b * a.h_kv + g) * a.T_max * DK;

  f32x16_t o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int t0 = kbeg; t0 < kend; t0 += 64) {
    u32x4 kr[2][KSTEP], vr[2][KSTEP];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(t0 + kb * 32 + lq, kend - 1);
#pragma unroll
      for (int s = 0; s < KSTEP; ++s)
        kr[kb][s] = *reinterpret_cast<const u32x4*>(Kc + (size_t)key * DK + 16 * s + 8 * kg);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(t0 + kb * 32 + lq, kend - 1);
#pragma unroll
      for (int s = 0; s < KSTEP; ++s)
        vr[kb][s] = *reinterpret_cast<const u32x4*>(Vc + (size_t)key * DK + 16 * s + 8 * kg);
    }
    // scores
    f32x16_t sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KSTEP; ++s) sc[kb] = mfma32x32x16<F16>(bf16x8_to_f16x8(kr[kb][s]), qf[s], sc[kb]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + kb * 32 + 8 * (i >> 2) + 4 * kg + (i & 3);
        if (key >= kend) sc[kb][i] = -INFINITY;
        mx = fmaxf(mx, sc[kb][i]);
      }
    mx = pair32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.0f;
    u32x4 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = exp2f(sc[kb][8 * hlf + i] - m_new);
          rs += e[i];
        }
        pf[2 * kb + hlf] = u32x4{pack_f16x2(e[0], e[1]), pack_f16x2(e[2], e[3]),
                                 pack_f16x2(e[4], e[5]), pack_f16x2(e[6], e[7])};
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[d][i] *= alpha;

    // V -> LDS, transposed (dim-major), keys in slot order. (One-wave
    // workgroup: the barriers only order this wave's LDS writes and reads.)
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int slot = vt_slot(kb * 32 + lq);
#pragma unroll
      for (int s = 0; s < KSTEP; ++s) {
        const u32x4 h = bf16x8_to_f16x8(vr[kb][s]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vts[16 * s + 8 * kg + 2 * e][slot] = static_cast<uint16_t>(h[e] & 0xffffu);
          vts[16 * s + 8 * kg + 2 * e + 1][slot] = static_cast<uint16_t>(h[e] >> 16);
        }
      }
    }
    __syncthreads();
    // O^T += V^T P^T
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(&vts[d * 32 + lq][16 * st + 8 * kg]);
        o[d] = mfma32x32x16<F16>(va, pf[st], o[d]);
      }
  }
  l_run = pair32_sum(l_run);

  const size_t unit = (((size_t)b * a.h_kv + g) * a.nqb + qb) * a.nparts + p;
  if (kg == 0) {
    a.part_m[unit * 32 + lq] = m_run;
    a.part_l[unit * 32 + lq] = l_run;
  }
  float* po = a.part_o + (unit * 32 + lq) * DK;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<f32x4_t*>(po + d * 32 + 8 * r + 4 * kg) =
          f32x4_t{o[d][4 * r], o[d][4 * r + 1], o[d][4 * r + 2], o[d][4 * r + 3]};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per (new token t, query head, batch element): merge the cached
// chunks' partial states, then attend to new tokens 0..t in fp32, normalise.
template <int DK>
__global__ void __launch_bounds__(64)
decode_merge_kernel(DecodeArgs a) {
  constexpr int PL = DK / 64;   // dims per lane
  const int lane = threadIdx.x, t = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int grp = a.h / a.h_kv, g = head / grp;
  const int rr = (head - g * grp) * a.T_new + t, qb = rr >> 5, j = rr & 31;
  const int L = clamp_len(a.cache_len, b, a.T_max, a.T_new);
  const int np = (L + a.CW - 1) / a.CW;
  const size_t unit0 = (((size_t)b * a.h_kv + g) * a.nqb + qb) * a.nparts;

  float mstar = -INFINITY;
  for (int p = lane; p < np; p += 64) mstar = fmaxf(mstar, a.part_m[(unit0 + p) * 32 + j]);
  mstar = wave_max(mstar);
  float l = 0.0f, acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.0f;
  for (int p = 0; p < np; ++p) {
    const size_t u = (unit0 + p) * 32 + j;
    const float w = exp2f(a.part_m[u] - mstar);
    l += a.part_l[u] * w;
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] += a.part_o[u * DK + lane + 64 * e] * w;
  }
  // New tokens 0..t (fp32 Q, K, V of this step).
  const int m = b * a.T_new + t;
  float q[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) q[e] = a.q32[(size_t)m * a.D + head * DK + lane + 64 * e];
  float mrun = mstar;
  for (int jj = 0; jj <= t; ++jj) {
    const size_t kv = (size_t)(b * a.T_new + jj) * a.Dkv + g * DK;
    float d = 0.0f;
#pragma unroll
    for (int e = 0; e < PL; ++e) d += q[e] * a.k32[kv + lane + 64 * e];
    const float s = wave_sum(d);
    const float mn = fmaxf(mrun, s);
    const float sc = exp2f(mrun - mn), pe = exp2f(s - mn);
    l = l * sc + pe;
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] = acc[e] * sc + pe * a.v32[kv + lane + 64 * e];
    mrun = mn;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < PL; ++e) a.o32[(size_t)m * a.D + head * DK + lane + 64 * e] = acc[e] * inv;
}

// Y = sum of the K split + b_O.
__global__ void __launch_bounds__(256)
decode_out_kernel(const float* __restrict__ part, int KS, int M, int N,
                  const uint16_t* __restrict__ bias, float* __restrict__ y) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx - (long long)m * N);
  float v = 0.0f;
  for (int s = 0; s < KS; ++s) v += part[((size_t)s * M + m) * N + n];
  if (bias) v += bf16_bits_to_float(bias[n]);
  y[idx] = v;
}

}  // namespace

static int k_rows(int K, int KS) {
  const int slabs = K / RG_K;
  return ((slabs + KS - 1) / KS) * RG_K;
}

int decode_k_split(int M, int K, int N) {
  // Enough workgroups to spread the weight read over the chip, while the
  // fp32 partial sums (KS * M * N * 4 bytes) stay below the weight bytes.
  const int col_tiles = (N + RG_N - 1) / RG_N, row_tiles = (M + 31) / 32;
  int ks = (512 + col_tiles * row_tiles - 1) / (col_tiles * row_tiles);
  const int max_parts = max(1, K / (2 * max(M, 1)));
  ks = min(ks, max_parts);
  ks = max(1, min(ks, K / RG_K));
  // number of non-empty slices of RG_K-aligned rows
  const int KR = k_rows(K, ks);
  return (K + KR - 1) / KR;
}

hipError_t launch_rows_gemm(const void* X, bool x_f32, int M, int K, const uint16_t* W, int N,
                            int KS, float* part, hipStream_t s) {
  if (K % RG_K != 0 || N % 8 != 0 || KS < 1) return hipErrorInvalidValue;
  const int KR = k_rows(K, KS);
  // every slice non-empty and together covering K
  if ((KS - 1) * KR >= K || (long long)KS * KR < K) return hipErrorInvalidValue;
  dim3 grid((N + RG_N - 1) / RG_N, KS, (M + 31) / 32);
  if (x_f32)
    hipLaunchKernelGGL(rows_gemm_kernel<true>, grid, dim3(256), 0, s, X, M, K, W, N, KR, part);
  else
    hipLaunchKernelGGL(rows_gemm_kernel<false>, grid, dim3(256), 0, s, X, M, K, W, N, KR, part);
  return hipGetLastError();
}

hipError_t launch_decode_route(const DecodeArgs& a, const float* part, int KS, hipStream_t s) {
  const long long total = (long long)a.B * a.T_new * (a.D + 2 * a.Dkv);
  hipLaunchKernelGGL(decode_route_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                     part, KS);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const DecodeArgs& a, hipStream_t s) {
  if (a.h_kv < 1 || a.h % a.h_kv != 0 || a.CW % 64 != 0 || a.CW < 64) return hipErrorInvalidValue;
  dim3 g1(a.nparts, a.h_kv * a.nqb, a.B);
  dim3 g2(a.T_new, a.h, a.B);
  if (a.d_k == 64) {
    hipLaunchKernelGGL(decode_split_kernel<64>, g1, dim3(64), 0, s, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g2, dim3(64), 0, s, a);
  } else if (a.d_k == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, g1, dim3(64), 0, s, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g2, dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_out(const float* part, int KS, int M, int N, const uint16_t* bias, float* y,
                             hipStream_t s) {
  const long long total = (long long)M * N;
  hipLaunchKernelGGL(decode_out_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     KS, M, N, bias, y);
  return hipGetLastError();
}

}  // namespace mha
