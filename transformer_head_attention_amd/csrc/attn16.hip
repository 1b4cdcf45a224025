// Fused scaled dot-product attention, fp16 MFMA operands, fp32 softmax state.
//
// Computes, per (batch, head) and query row i,
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k) + M_ij) v_j
// (itwiki "멀티 헤드 어텐션", 수식, eq. Attention; iamjaehka13.blog
// "[Deep Learning 5] Attention의 내부 계산", §7-§13) without forming the
// T_q x T_k score matrix. Keys are visited in tiles of 64; the softmax is
// accumulated online: a running row maximum m and row sum l, with the partial
// output rescaled by exp(m_old - m_new) whenever m grows. This is the same
// softmax in exact arithmetic (the exp(-m) factor cancels between numerator
// and denominator).
//
// Masks: key j > query i under the causal mask and keys flagged in the
// padding mask (nonzero = ignore) get -inf, so their weight is exactly 0
// (iamjaehka13.blog §9; molayo1419.me "MHA란 무엇인가?", trap 2). Key tiles
// entirely in a wave's future are skipped; key tiles beyond the last unmasked
// key of a batch element are never visited. A row with no unmasked key ends
// with l = 0 and writes 0 * (1/0) = NaN (molayo1419.me, trap 3).
//
// Layout of one wave's work: 32 query rows x one 64-key tile.
//   S^T = K . Q^T with v_mfma_f32_32x32x16_f16: the K tile is the A operand
//   (from LDS), Q^T the B operand (held in registers for the whole kernel).
//   The result puts one query per lane column, so the row max and row sum
//   over keys are reductions inside a lane plus one exchange with lane l^32.
//   O^T += V^T . P^T: P^T is repacked from the S^T accumulators in registers
//   (fp16, round to nearest even) and used directly as the B operand; V^T
//   comes from LDS in the same key order.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int BLOCK_N = 64;   // keys per tile
constexpr int NWAVES = 4;

__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / 8;
  if (L >= per * 8) return L;
  return (L % 8) * per + L / 8;
}

template <int DK>
struct Lds {
  static constexpr int KS = DK + 8;        // K tile row stride (16-bit elements)
  static constexpr int VS = BLOCK_N + 8;   // V^T tile row stride
  static constexpr int K_ELEMS = BLOCK_N * KS;
  static constexpr int V_ELEMS = DK * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
};

// Clear the fp16 elements of an 8-element chunk whose key index is >= limit.
__device__ __forceinline__ u32x4 zero_from(u32x4 v, int first_key, int limit) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int k0 = first_key + 2 * e;
    if (k0 >= limit) w[e] = 0u;
    else if (k0 + 1 >= limit) w[e] &= 0xffffu;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

template <int DK, int NQ>
__global__ void __launch_bounds__(NWAVES * 64)
attn_f16_kernel(AttnF16Args a) {
  constexpr int BLOCK_M = NWAVES * 32 * NQ;
  constexpr int NT = NWAVES * 64;
  constexpr int K_PER_T = BLOCK_N * DK / 8 / NT;   // 16-byte chunks per thread
  constexpr int V_PER_T = DK * BLOCK_N / 8 / NT;
  constexpr int KSTEPS = DK / 16;
  constexpr int DT = DK / 32;
  using L = Lds<DK>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];
  __shared__ uint64_t mbits[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lh = lane >> 5;

  // Workgroup -> (batch, head, query block). All query blocks of one
  // (batch, head) run on one XCD and share its L2 copy of K and V; under the
  // causal mask the longest blocks are dispatched first.
  const int nqb = a.Tqp / BLOCK_M;
  const int logical = xcd_remap(blockIdx.x, nqb * a.h * a.B);
  const int bh = logical / nqb;
  int qblk = logical - bh * nqb;
  if (a.causal) qblk = nqb - 1 - qblk;
  const int b = bh / a.h, head = bh - b * a.h;

  const uint16_t* Qg = a.q + (size_t)bh * a.Tqp * DK;
  const uint16_t* Kg = a.k + (size_t)bh * a.Tkp * DK;
  const uint16_t* Vg = a.vt + (size_t)bh * DK * a.Tkp;
  const int qw0 = qblk * BLOCK_M + wave * 32 * NQ;

  u32x4 qreg[NQ][KSTEPS];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const int row = qw0 + qi * 32 + lq;
    const uint16_t* p = Qg + (size_t)row * DK + lh * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qreg[qi][ks] = row < a.T_q ? *reinterpret_cast<const u32x4*>(p + ks * 16)
                                 : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16_t o[NQ][DT];
  float m_run[NQ], l_run[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    m_run[qi] = -INFINITY;
    l_run[qi] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qi][dt][r] = 0.0f;
  }

  int kv_end = a.T_k;
  if (a.kend) kv_end = min(kv_end, a.kend[b]);
  if (a.causal) kv_end = min(kv_end, qblk * BLOCK_M + BLOCK_M);
  const int ntiles = kv_end > 0 ? (kv_end + BLOCK_N - 1) / BLOCK_N : 0;
  const bool has_mask = a.mask != nullptr;
  const uint8_t* maskb = has_mask ? a.mask + (size_t)b * a.T_k : nullptr;
  // log2(e) / sqrt(d_k): scores are exponentiated with exp2.
  const float sl2 = 1.4426950408889634f / sqrtf((float)DK);

  u32x4 rk[K_PER_T], rv[V_PER_T];
  uint64_t rbits = 0;
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT, row = c / (DK / 8), col = (c % (DK / 8)) * 8;
      rk[i] = *reinterpret_cast<const u32x4*>(Kg + (size_t)(k0 + row) * DK + col);
    }
    const bool tail = k0 + BLOCK_N > a.T_k;
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int c = tid + i * NT, row = c / (BLOCK_N / 8), col = (c % (BLOCK_N / 8)) * 8;
      rv[i] = *reinterpret_cast<const u32x4*>(Vg + (size_t)row * a.Tkp + k0 + col);
      if (tail) rv[i] = zero_from(rv[i], k0 + col, a.T_k);
    }
    if (wave == 0) {
      const int key = k0 + lane;
      const bool ignore = key >= a.T_k || (has_mask && maskb[key] != 0);
      rbits = __ballot(ignore);
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
    uint16_t* Ks = smem + buf * L::STAGE;
    uint16_t* Vs = Ks + L::K_ELEMS;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int c = tid + i * NT, row = c / (DK / 8), col = (c % (DK / 8)) * 8;
      *reinterpret_cast<u32x4*>(Ks + row * L::KS + col) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int c = tid + i * NT, row = c / (BLOCK_N / 8), col = (c % (BLOCK_N / 8)) * 8;
      *reinterpret_cast<u32x4*>(Vs + row * L::VS + col) = rv[i];
    }
    if (tid == 0) mbits[buf] = rbits;
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * BLOCK_N;
    const int buf = it & 1;
    if (it + 1 < ntiles) gload(k0 + BLOCK_N);
    const uint16_t* Ks = smem + buf * L::STAGE;
    const uint16_t* Vs = Ks + L::K_ELEMS;
    const uint64_t bits = mbits[buf] >> (4 * lh);
    const bool tile_masked = has_mask || (k0 + BLOCK_N > a.T_k);

#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int q_lo = qw0 + qi * 32;
      if (a.causal && k0 > q_lo + 31) continue;   // whole tile in this wave's future

      f32x16_t s[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kh][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const u32x4 kf =
              *reinterpret_cast<const u32x4*>(Ks + (kh * 32 + lq) * L::KS + ks * 16 + lh * 8);
          s[kh] = mfma32x32x16<F16>(kf, qreg[qi][ks], s[kh]);
        }
      }

      // Key of accumulator element (kh, r): k0 + kh*32 + 8*(r/4) + 4*lh + r%4.
      const bool diag = a.causal && (k0 + BLOCK_N - 1 > q_lo);
      if (diag || tile_masked) {
        const int lim = q_lo + lq - k0 - 4 * lh;   // causal: masked iff rel > lim
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = kh * 32 + 8 * (r >> 2) + (r & 3);
            const bool ign = (tile_masked && ((bits >> rel) & 1ull)) || (a.causal && rel > lim);
            if (ign) s[kh][r] = -INFINITY;
          }
      }

      float mx = s[0][0];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qi], mx);
      const float base = (m_new == -INFINITY) ? 0.0f : m_new * sl2;
      const float alpha = __builtin_amdgcn_exp2f(__builtin_fmaf(m_run[qi], sl2, -base));
      m_run[qi] = m_new;

      float rs = 0.0f;
      u32x4 pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c >> 1][(c & 1) * 8 + e], sl2, -base));
          rs += p[e];
        }
        pf[c] = u32x4{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]),
                      pack_f16x2(p[4], p[5]), pack_f16x2(p[6], p[7])};
      }
      l_run[qi] = __builtin_fmaf(l_run[qi], alpha, rs);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qi][dt][r] *= alpha;

      // P^T fragment c covers keys c*16 + {4*lh + 0..3, 8 + 4*lh + 0..3}; V^T
      // supplies the same keys for its row d.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint16_t* vp = Vs + (dt * 32 + lq) * L::VS + c * 16 + lh * 4;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
          o[qi][dt] = mfma32x32x16<F16>(u32x4{lo.x, lo.y, hi.x, hi.y}, pf[c], o[qi][dt]);
        }
    }

    if (it + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // O = acc / l; head `head` occupies columns [head*DK, (head+1)*DK) of (B, T_q, D).
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const float lt = l_run[qi] + __shfl_xor(l_run[qi], 32);
    const float inv = 1.0f / lt;
    const int row = qw0 + qi * 32 + lq;
    if (row < a.T_q) {
      uint16_t* op = a.o + ((size_t)b * a.T_q + row) * a.D + head * DK;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = dt * 32 + 8 * rg + 4 * lh;
          u32x2 pk;
          pk.x = pack_f16x2(o[qi][dt][rg * 4 + 0] * inv, o[qi][dt][rg * 4 + 1] * inv);
          pk.y = pack_f16x2(o[qi][dt][rg * 4 + 2] * inv, o[qi][dt][rg * 4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d0) = pk;
        }
    }
  }
}

constexpr int kNQ = 1;

}  // namespace

int attn_f16_block_m(int /*d_k*/) { return NWAVES * 32 * kNQ; }

hipError_t launch_attn_f16(const AttnF16Args& a, int d_k, hipStream_t s) {
  const int bm = attn_f16_block_m(d_k);
  const int total = (a.Tqp / bm) * a.h * a.B;
  if (d_k == 64)
    hipLaunchKernelGGL((attn_f16_kernel<64, kNQ>), dim3(total), dim3(NWAVES * 64), 0, s, a);
  else if (d_k == 128)
    hipLaunchKernelGGL((attn_f16_kernel<128, kNQ>), dim3(total), dim3(NWAVES * 64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mha
