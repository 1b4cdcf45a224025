// 16-bit MFMA GEMMs for the two projections.
//
//  * QKV projection (itwiki "멀티 헤드 어텐션", 텐서 모양으로 본 계산: one D x 3D
//    matrix; the head split is a view of its output): C = X . W_QKV + b with
//    bf16 operands and fp32 accumulation. The epilogue performs the head split
//    in its stores: Q and K go to (B, h, T, d_k), V to (B, h, d_k, T)
//    (transposed, so the attention kernel's P.V operand is key-contiguous),
//    all rounded to fp16; rows t < early_rows are also kept in fp32.
//  * Output projection (same table, 출력 투영 row): Y = O . W_O + b_O with
//    fp16 operands, fp32 accumulation and an fp32 result.
//
// Both operands are K-contiguous (A row-major M x K, B given transposed as
// N x K). Tiles are staged through LDS, double-buffered with a register
// prefetch of the next K slice; each wave owns a WM x WN sub-tile computed
// with v_mfma_f32_32x32x16.
#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int BK = 64;          // K slice per stage (16-bit elements)
constexpr int LDS_STRIDE = BK + 8;   // padded LDS row, in 16-bit elements

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int NWAVES = (BM / WM) * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_PER_T = BM * BK / 8 / NT;   // 16-byte chunks per thread
  static constexpr int B_PER_T = BN * BK / 8 / NT;
  static constexpr int STAGE = (BM + BN) * LDS_STRIDE;
  static_assert(BM * BK / 8 % NT == 0 && BN * BK / 8 % NT == 0, "tile / thread mismatch");
};

// Map a linear workgroup id so that consecutive logical tiles land on the same
// XCD (workgroups are dispatched round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / 8;
  if (L >= per * 8) return L;
  return (L % 8) * per + L / 8;
}

template <typename C, typename Tag, typename Epi>
__global__ void __launch_bounds__(C::NT)
gemm16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, int M, int N,
              int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // Tile order: column tiles of one row band are consecutive, and a group of
  // row bands shares an XCD so that its A rows and all of B stay in that L2.
  const int ntn = (N + C::BN - 1) / C::BN, ntm = (M + C::BM - 1) / C::BM;
  const int logical = xcd_remap(blockIdx.x, ntn * ntm);
  const int bm = logical / ntn, bn = logical % ntn;
  const int m0 = bm * C::BM, n0 = bn * C::BN;

  u32x4 ra[C::A_PER_T], rb[C::B_PER_T];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int c = tid + i * C::NT, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      const int m = min(m0 + row, M - 1);
      ra[i] = *reinterpret_cast<const u32x4*>(A + (size_t)m * K + k0 + col);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int c = tid + i * C::NT, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      const int n = min(n0 + row, N - 1);
      rb[i] = *reinterpret_cast<const u32x4*>(Bt + (size_t)n * K + k0 + col);
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
    uint16_t* As = smem + buf * C::STAGE;
    uint16_t* Bs = As + C::BM * LDS_STRIDE;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int c = tid + i * C::NT, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      *reinterpret_cast<u32x4*>(As + row * LDS_STRIDE + col) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int c = tid + i * C::NT, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      *reinterpret_cast<u32x4*>(Bs + row * LDS_STRIDE + col) = rb[i];
    }
  };

  f32x16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int arow = wm * C::WM + (lane & 31), brow = wn * C::WN + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint16_t* As = smem + (kt & 1) * C::STAGE;
    const uint16_t* Bs = As + C::BM * LDS_STRIDE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 a[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(As + (arow + i * 32) * LDS_STRIDE + ks * 16 + kofs);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(Bs + (brow + j * 32) * LDS_STRIDE + ks * 16 + kofs);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32x32x16<Tag>(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }
  epi.template apply<C::TM, C::TN>(acc, m0 + wm * C::WM, n0 + wn * C::WN, lane, M, N);
}

// Head-split epilogue of the QKV projection.
struct QkvEpi {
  QkvEpilogue e;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x16_t (&acc)[TM][TN], int mbase, int nbase, int lane,
                                        int M, int N) const {
    const int D = e.D, d_k = e.d_k;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nbase + j * 32 + (lane & 31);
      if (n >= N) continue;
      const int ng = e.n_base + n;
      const int which = ng / D, hc = ng - which * D;
      const int head = hc / d_k, c = hc - head * d_k;
      const float bias = load_bias_bf16(e.bias, ng);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int mf = mbase + i * 32 + 8 * rg + 4 * (lane >> 5);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][rg * 4 + r] + bias;
          const int b0 = mf / e.T, t0 = mf - b0 * e.T;
          if (e.early && (t0 < e.early_rows || t0 + 4 > e.T)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = mf + r;
              if (m >= M) break;
              const int b = m / e.T, t = m - b * e.T;
              if (t < e.early_rows)
                e.early[((size_t)b * e.early_rows + t) * (3 * D) + ng] = v[r];
            }
          }
          if (which == 2) {
            // V^T: four consecutive t of one column -> one 8-byte store when aligned.
            if ((e.T & 3) == 0 && mf + 3 < M) {
              uint16_t* dst = e.vt + (((size_t)b0 * e.h + head) * d_k + c) * e.Tpad_kv + t0;
              u32x2 pk;
              pk.x = pack_f16x2(v[0], v[1]);
              pk.y = pack_f16x2(v[2], v[3]);
              *reinterpret_cast<u32x2*>(dst) = pk;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int m = mf + r;
                if (m >= M) break;
                const int b = m / e.T, t = m - b * e.T;
                e.vt[(((size_t)b * e.h + head) * d_k + c) * e.Tpad_kv + t] = float_to_f16_bits(v[r]);
              }
            }
          } else {
            uint16_t* base = which == 0 ? e.q : e.k;
            const int tpad = which == 0 ? e.Tpad_q : e.Tpad_kv;
            const float sc = which == 0 ? e.q_scale : 1.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = mf + r;
              if (m >= M) break;
              const int b = m / e.T, t = m - b * e.T;
              base[(((size_t)b * e.h + head) * tpad + t) * d_k + c] = float_to_f16_bits(v[r] * sc);
            }
          }
        }
      }
    }
  }
};

// fp32 result epilogue of the output projection.
struct OutEpi {
  const uint16_t* bias;
  float* Y;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x16_t (&acc)[TM][TN], int mbase, int nbase, int lane,
                                        int M, int N) const {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nbase + j * 32 + (lane & 31);
      if (n >= N) continue;
      const float b = load_bias_bf16(bias, n);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mbase + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < M) Y[(size_t)m * N + n] = acc[i][j][r] + b;
        }
    }
  }
};

// Output projection of the first rows of each causal sequence, from their
// fp32 attention output: Y[b*T_q + t] = O32[b*R + t] . W_O + b_O for t < R.
// Each fp32 value x is split into fp16 hi = fp16(x) and lo = fp16(x - hi), and
// hi . W + lo . W is accumulated in fp32 on the fp16 MFMA, which keeps about
// 22 significant bits of x. A workgroup owns a 32 x 32 tile of Y; its four
// waves take a quarter of K each and are summed through LDS in a fixed order.
__global__ void __launch_bounds__(256)
early_out_kernel(const float* __restrict__ O32, int M, int K, const uint16_t* __restrict__ WoT,
                 int N, const uint16_t* __restrict__ bias, float* __restrict__ Y, int R, int T_q) {
  __shared__ f32x16_t red[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int kw = K / 4, kbeg = wave * kw;
  const int row = min(m0 + (lane & 31), M - 1);
  const float* ap = O32 + (size_t)row * K + (lane >> 5) * 8;
  const uint16_t* bp = WoT + (size_t)(n0 + (lane & 31)) * K + (lane >> 5) * 8;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll 4
  for (int k = kbeg; k < kbeg + kw; k += 16) {
    const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(ap + k);
    const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(ap + k + 4);
    const u32x4 bf = *reinterpret_cast<const u32x4*>(bp + k);
    const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 h0 = static_cast<_Float16>(av[2 * e]);
      const _Float16 h1 = static_cast<_Float16>(av[2 * e + 1]);
      hi[e] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
      lo[e] = pack_f16x2(av[2 * e] - static_cast<float>(h0), av[2 * e + 1] - static_cast<float>(h1));
    }
    acc = mfma32x32x16<F16>(u32x4{hi[0], hi[1], hi[2], hi[3]}, bf, acc);
    acc = mfma32x32x16<F16>(u32x4{lo[0], lo[1], lo[2], lo[3]}, bf, acc);
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += red[w][lane];
  const int n = n0 + (lane & 31);
  const float bv = load_bias_bf16(bias, n);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (m < M) {
      const int bb = m / R, t = m - bb * R;
      Y[((size_t)bb * T_q + t) * N + n] = acc[r] + bv;
    }
  }
}

using QkvCfg = Cfg<128, 128, 64, 64>;
using OutCfg = Cfg<128, 128, 64, 64>;

}  // namespace

hipError_t launch_gemm_qkv(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const QkvEpilogue& e, hipStream_t s) {
  using C = QkvCfg;
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  QkvEpi epi{e};
  hipLaunchKernelGGL((gemm16_kernel<C, BF16, QkvEpi>), dim3(tiles), dim3(C::NT), 0, s, A, Bt, M,
                     N, K, epi);
  return hipGetLastError();
}

hipError_t launch_early_out(const float* O32, int M, int K, const uint16_t* WoT, int N,
                            const uint16_t* bias, float* Y, int R, int T_q, hipStream_t s) {
  dim3 grid(N / 32, (M + 31) / 32);
  hipLaunchKernelGGL(early_out_kernel, grid, dim3(256), 0, s, O32, M, K, WoT, N, bias, Y, R, T_q);
  return hipGetLastError();
}

hipError_t launch_gemm_out(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const uint16_t* bias, float* Y, hipStream_t s) {
  using C = OutCfg;
  const int tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  OutEpi epi{bias, Y};
  hipLaunchKernelGGL((gemm16_kernel<C, F16, OutEpi>), dim3(tiles), dim3(C::NT), 0, s, A, Bt, M, N,
                     K, epi);
  return hipGetLastError();
}

}  // namespace mha
