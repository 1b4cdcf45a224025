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

// Kernel templates are instantiated directly in the non-template launch
// functions below (instantiating them from inside another template left their
// host stubs undefined).
namespace gemm_impl {

// BM x BN output tile, WM x WN per wave, BK-deep K slices (32 or 64 16-bit
// elements: 64- or 128-byte LDS rows), NS slices in flight.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_;
  static constexpr int CH = BK / 8;                 // 16-byte chunks per LDS row
  static constexpr int WAVES_N = BN / WN;
  static constexpr int NWAVES = (BM / WM) * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LPT = A_BYTES / 16 / NT;   // DMA loads per thread per K slice
  static constexpr int B_LPT = B_BYTES / 16 / NT;
  static constexpr int LPT = A_LPT + B_LPT;
  static_assert(A_BYTES % (16 * NT) == 0 && B_BYTES % (16 * NT) == 0, "tile / thread mismatch");
  static_assert(NS >= 2 && NS <= 4, "pipeline depth");
  static_assert(BK == 32 || BK == 64, "K slice");
};

// Map a linear workgroup id so that consecutive logical tiles land on the same
// XCD (workgroups are dispatched round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / 8;
  if (L >= per * 8) return L;
  return (L % 8) * per + L / 8;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte chunk c of LDS row `row` is stored at a row-dependent XOR of c, so
// that the 16 rows one quarter-wave reads for an MFMA operand cover all 64
// banks: 128-byte rows (8 chunks) pair up per 256-byte bank window, 64-byte
// rows (4 chunks) group by four.
template <int CH>
__device__ __forceinline__ int swz(int row, int c) {
  return CH == 8 ? (c ^ ((row >> 1) & 7)) : (c ^ ((row >> 2) & 3));
}

// TRANS computes each 32 x 32 tile as (B^T A^T)^T: the MFMA result then holds,
// per lane, one row m and four consecutive columns n (instead of one column
// and four consecutive rows).
template <typename C, typename Tag, bool TRANS, typename Epi>
__global__ void __launch_bounds__(C::NT)
gemm16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, int M, int N,
              int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NS * C::STAGE];
  // wave index in a scalar register: the DMA LDS bases below stay scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // Tile order: each XCD takes a contiguous range of logical tiles, walked in
  // groups of GM row bands so that the concurrently resident workgroups of
  // an XCD share A rows and B columns in its L2.
#ifndef MHA_GEMM_GM
#define MHA_GEMM_GM 4
#endif
  constexpr int GM = MHA_GEMM_GM;
  const int ntn = (N + C::BN - 1) / C::BN, ntm = (M + C::BM - 1) / C::BM;
  const int logical = xcd_remap(blockIdx.x, ntn * ntm);
  const int group = logical / (GM * ntn);
  const int gm0 = group * GM, gsz = min(GM, ntm - gm0);
  const int in_group = logical - group * GM * ntn;
  const int bm = gm0 + in_group % gsz, bn = in_group / gsz;
  const int m0 = bm * C::BM, n0 = bn * C::BN;

  // DMA of K slice kt into stage `stage`: lane chunk p of a wave-wide load
  // lands at byte 16*p of the wave's 1 KiB window and fetches the global
  // chunk the swizzled layout places there. Rows past M or N are clamped
  // (their results are never stored).
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    uint8_t* as = smem + stage * C::STAGE;
    uint8_t* bs = as + C::A_BYTES;
    const int k0 = kt * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_LPT; ++i) {
      const int p = i * C::NT + tid, row = p / C::CH, c = swz<C::CH>(row, p % C::CH);
      const int m = min(m0 + row, M - 1);
      lds_dma16(A + (size_t)m * K + k0 + c * 8,
                as + (i * C::NT + wave * 64) * 16);
    }
#pragma unroll
    for (int i = 0; i < C::B_LPT; ++i) {
      const int p = i * C::NT + tid, row = p / C::CH, c = swz<C::CH>(row, p % C::CH);
      const int n = min(n0 + row, N - 1);
      lds_dma16(Bt + (size_t)n * K + k0 + c * 8,
                bs + (i * C::NT + wave * 64) * 16);
    }
  };

  f32x16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = K / C::BK;
#pragma unroll
  for (int t = 0; t < C::NS - 1; ++t)
    if (t < nk) issue(t, t);

  const int arow0 = wm * C::WM + (lane & 31), brow0 = wn * C::WN + (lane & 31);
  const int lh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    // Slice kt is complete once at most the younger slices' loads are
    // outstanding (up to NS-2 of them).
    const int younger = min(C::NS - 2, nk - 1 - kt);
    if (younger >= 2) wait_vmcnt<2 * C::LPT>();
    else if (younger == 1) wait_vmcnt<C::LPT>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();   // slice kt has landed; the stage read last is free
    const uint8_t* as = smem + (kt % C::NS) * C::STAGE;
    const uint8_t* bs = as + C::A_BYTES;
    // Operand fragments are double-buffered in registers: the LDS reads of
    // k-step ks+1 are issued before the MFMAs of k-step ks, so their latency
    // hides behind 16 MFMAs of this wave.
    u32x4 a[2][C::TM], b[2][C::TN];
    auto frags = [&](int ks, u32x4 (&fa)[C::TM], u32x4 (&fb)[C::TN]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int row = arow0 + i * 32;
        fa[i] = *reinterpret_cast<const u32x4*>(as + (row * C::CH + swz<C::CH>(row, 2 * ks + lh)) * 16);
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int row = brow0 + j * 32;
        fb[j] = *reinterpret_cast<const u32x4*>(bs + (row * C::CH + swz<C::CH>(row, 2 * ks + lh)) * 16);
      }
    };
    frags(0, a[0], b[0]);
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < C::BK / 16) frags(ks + 1, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = TRANS ? mfma32x32x16<Tag>(b[cur][j], a[cur][i], acc[i][j])
                            : mfma32x32x16<Tag>(a[cur][i], b[cur][j], acc[i][j]);
    }
    // Slice kt+NS-1 goes into the stage read in the previous iteration. The
    // load is issued every iteration (past the last slice it re-reads the
    // last slice into a stage nobody reads again), which keeps it in the same
    // basic block as the MFMAs so the two can interleave.
    issue(min(kt + C::NS - 1, nk - 1), (kt + C::NS - 1) % C::NS);
    // Issue order for the scheduler (0x100 = LDS read, 0x008 = MFMA,
    // 0x020 = global load): the fragments of k-step 0; in each k-step but the
    // last, the next step's reads go out one per MFMA over its first MFMAs so
    // the rest cover their latency; in the last k-step the next slices'
    // global->LDS loads go out between MFMAs.
    constexpr int KS = C::BK / 16, NR = C::TM + C::TN, NMF = C::TM * C::TN;
    constexpr int VPER = (C::LPT + NMF - 1) / NMF, NV = (C::LPT + VPER - 1) / VPER;
    static_assert(NR <= NMF && NV <= NMF, "schedule shape");
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF - NR, 0);
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, VPER, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - NV, 0);
  }
  wait_vmcnt<0>();   // no global->LDS copy may outlive the workgroup
  // Every wave has finished reading the stages: each wave may now use its
  // share of the LDS to stage its output tile.
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  static_assert(C::WM * C::WN * 2 <= C::NS * C::STAGE / C::NWAVES, "staging window");
  epi.template apply<C::TM, C::TN>(acc, m0 + wm * C::WM, n0 + wn * C::WN, lane, M, N,
                                   smem + wave * (C::NS * C::STAGE / C::NWAVES));
}

// Output staging: 16-byte chunk c of LDS row `row` (RB bytes per row) sits at
// a row-dependent XOR of c so that the 8-byte writes of 32 lanes to 32
// consecutive rows spread over the banks.
template <int RB>
__device__ __forceinline__ int stage_chunk(int row, int c) {
  return RB == 128 ? (c ^ ((row >> 1) & 7)) : (c ^ (row & 15));
}

// Head-split epilogues of the QKV projection. Column n of [Q|K|V] is head
// (n mod D) / d_k, channel (n mod D) mod d_k; row m is batch m / T, position
// m mod T. A wave's tile is staged in LDS and written back 16 bytes per lane,
// so each store instruction covers whole contiguous lines; tiles that cross a
// batch boundary or the matrix edge are stored directly from registers.

// Position of key t in a V^T row: bits 2 and 3 of t swapped, so each 16-key
// group is stored as keys {0-3, 8-11, 4-7, 12-15}. One 16-byte chunk then
// holds exactly the 8 keys one lane half of the P.V MFMA consumes.
__device__ __forceinline__ int vt_pos(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

// Q and K columns (transposed tiles): a lane holds row m and channels
// n..n+3. Q is scaled by q_scale; rows t < early_rows are also written in fp32.
struct QkEpi {
  QkvEpilogue e;

  __device__ __forceinline__ void bias4(int ng, const f32x16_t& a, int r0, float (&v)[4]) const {
    if (e.bias) {
      const u32x2 bb = *reinterpret_cast<const u32x2*>(e.bias + ng);
      v[0] = a[r0 + 0] + __uint_as_float(bb.x << 16);
      v[1] = a[r0 + 1] + __uint_as_float(bb.x & 0xffff0000u);
      v[2] = a[r0 + 2] + __uint_as_float(bb.y << 16);
      v[3] = a[r0 + 3] + __uint_as_float(bb.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = a[r0 + r];
    }
  }

  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x16_t (&acc)[TM][TN], int mbase, int nbase, int lane,
                                        int M, int N, uint8_t* lds) const {
    constexpr int WM = TM * 32, WN = TN * 32, RB = WN * 2, CPR = WN / 8;
    const int D = e.D, d_k = e.d_k, T = e.T, lq = lane & 31, lh = lane >> 5;
    const int bw = mbase / T, tw = mbase - bw * T;
    const bool staged = tw + WM <= T && mbase + WM <= M && nbase + WN <= N;
    const bool early = e.early && tw < e.early_rows;
    if (staged) {
      // The wave's WN columns lie in one of Q or K (WN divides D).
      const int ng0 = e.n_base + nbase, which = ng0 / D, hc0 = ng0 - which * D;
      const float sc = which == 0 ? e.q_scale : 1.0f;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = i * 32 + lq;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int c = j * 32 + 8 * rg + 4 * lh;
            float v[4];
            bias4(ng0 + c, acc[i][j], rg * 4, v);
            if (early && tw + r < e.early_rows)
              *reinterpret_cast<f32x4_t*>(e.early + ((size_t)bw * e.early_rows + tw + r) * (3 * D) +
                                          ng0 + c) = f32x4_t{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<u32x2*>(lds + r * RB + stage_chunk<RB>(r, c >> 3) * 16 + lh * 8) =
                u32x2{pack_f16x2(v[0] * sc, v[1] * sc), pack_f16x2(v[2] * sc, v[3] * sc)};
          }
      }
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
      // Write-back: chunk runs of one head are contiguous in (B, h, T, d_k).
      const int hseg = min(WN, d_k), lg_cph = hseg == 128 ? 4 : 3;   // chunks per head segment
      const int tpad = which == 0 ? e.Tpad_q : e.Tpad_kv;
      uint16_t* base = (which == 0 ? e.q : e.k) + (size_t)bw * e.h * tpad * d_k;
#pragma unroll 4
      for (int k = 0; k < WM * CPR / 64; ++k) {
        const int idx = k * 64 + lane;
        const int cb = idx >> (lg_cph + __builtin_ctz(WM)), rem = idx & ((WM << lg_cph) - 1);
        const int r = rem >> lg_cph, c8 = (cb << lg_cph) + (rem & ((1 << lg_cph) - 1));
        const u32x4 val = *reinterpret_cast<const u32x4*>(lds + r * RB + stage_chunk<RB>(r, c8) * 16);
        const int col = hc0 + c8 * 8, head = col / d_k, ch = col - head * d_k;
        *reinterpret_cast<u32x4*>(base + ((size_t)head * tpad + tw + r) * d_k + ch) = val;
      }
      return;
    }
    // Direct path: 8-byte stores of four channels.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mbase + i * 32 + lq;
      if (m >= M) continue;
      const int b = m / T, t = m - b * T;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = nbase + j * 32 + 8 * rg + 4 * lh;   // four columns n..n+3
          if (n >= N) continue;
          const int ng = e.n_base + n;
          const int which = ng / D, hc = ng - which * D, head = hc / d_k, c = hc - head * d_k;
          float v[4];
          bias4(ng, acc[i][j], rg * 4, v);
          if (e.early && t < e.early_rows)
            *reinterpret_cast<f32x4_t*>(e.early + ((size_t)b * e.early_rows + t) * (3 * D) + ng) =
                f32x4_t{v[0], v[1], v[2], v[3]};
          const float sc = which == 0 ? e.q_scale : 1.0f;
          const int tpad = which == 0 ? e.Tpad_q : e.Tpad_kv;
          uint16_t* dst = (which == 0 ? e.q : e.k) +
                          (((size_t)b * e.h + head) * tpad + t) * d_k + c;
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{pack_f16x2(v[0] * sc, v[1] * sc), pack_f16x2(v[2] * sc, v[3] * sc)};
        }
      }
    }
  }
};

// V columns (normal tiles): a lane holds column n and rows m..m+3, i.e. four
// consecutive positions of one V^T row.
struct VEpi {
  QkvEpilogue e;
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x16_t (&acc)[TM][TN], int mbase, int nbase, int lane,
                                        int M, int N, uint8_t* lds) const {
    constexpr int WM = TM * 32, WN = TN * 32, RB = WM * 2, CPR = WM / 8;
    const int D = e.D, d_k = e.d_k, T = e.T, lq = lane & 31, lh = lane >> 5;
    const int bw = mbase / T, tw = mbase - bw * T;
    // One batch element, a full tile, and a start on a 16-position group so
    // the position permutation stays inside the tile.
    const bool staged = (tw & 15) == 0 && tw + WM <= T && mbase + WM <= M && nbase + WN <= N;
    if (staged) {
      const int hc0 = e.n_base + nbase - 2 * D;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = j * 32 + lq;
        const int ng = e.n_base + nbase + c;
        const float bias = load_bias_bf16(e.bias, ng);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int r0 = i * 32 + 8 * rg + 4 * lh;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[i][j][rg * 4 + r] + bias;
            if (e.early && tw + r0 < e.early_rows) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (tw + r0 + r < e.early_rows)
                  e.early[((size_t)bw * e.early_rows + tw + r0 + r) * (3 * D) + ng] = v[r];
            }
            const int pos = vt_pos(r0);
            *reinterpret_cast<u32x2*>(lds + c * RB + stage_chunk<RB>(c, pos >> 3) * 16 +
                                      (pos & 7) * 2) =
                u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
          }
      }
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
      // Write-back: each V^T row segment of WM positions is contiguous.
#pragma unroll 4
      for (int k = 0; k < WN * CPR / 64; ++k) {
        const int idx = k * 64 + lane;
        const int c = idx / CPR, p8 = idx - c * CPR;
        const u32x4 val = *reinterpret_cast<const u32x4*>(lds + c * RB + stage_chunk<RB>(c, p8) * 16);
        const int col = hc0 + c, head = col / d_k, ch = col - head * d_k;
        *reinterpret_cast<u32x4*>(e.vt + (((size_t)bw * e.h + head) * d_k + ch) * e.Tpad_kv + tw +
                                  p8 * 8) = val;
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nbase + j * 32 + lq;
      if (n >= N) continue;
      const int ng = e.n_base + n;
      const int hc = ng - 2 * D, head = hc / d_k, c = hc - head * d_k;
      const float bias = load_bias_bf16(e.bias, ng);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int mf = mbase + i * 32 + 8 * rg + 4 * lh;
          if (mf >= M) continue;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][rg * 4 + r] + bias;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = mf + r;
            if (m >= M) break;
            const int b = m / T, t = m - b * T;
            if (e.early && t < e.early_rows)
              e.early[((size_t)b * e.early_rows + t) * (3 * D) + ng] = v[r];
            e.vt[(((size_t)b * e.h + head) * d_k + c) * e.Tpad_kv + vt_pos(t)] =
                float_to_f16_bits(v[r]);
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
                                        int M, int N, uint8_t* /*lds*/) const {
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

// Large problems: 256 x 256 tiles, four waves of 128 x 128 (accumulators in
// AGPRs, one wave per SIMD). Problems with too few such tiles to fill the
// 256 CUs use 128 x 128 tiles, four waves of 64 x 64.
#ifndef MHA_BIG_BK
#define MHA_BIG_BK 32
#endif
#ifndef MHA_BIG_NS
#define MHA_BIG_NS 4
#endif
#ifndef MHA_SMALL_BK
#define MHA_SMALL_BK 32
#endif
#ifndef MHA_SMALL_NS
#define MHA_SMALL_NS 4
#endif
using BigCfg = Cfg<256, 256, 128, 128, MHA_BIG_BK, MHA_BIG_NS>;
using SmallCfg = Cfg<128, 128, 64, 64, MHA_SMALL_BK, MHA_SMALL_NS>;

int tiles_of(int M, int N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }
#ifndef MHA_GEMM_BIG_MIN_TILES
#define MHA_GEMM_BIG_MIN_TILES 384
#endif
bool use_big(int M, int N) { return tiles_of(M, N, 256, 256) >= MHA_GEMM_BIG_MIN_TILES; }

}  // namespace gemm_impl

using namespace gemm_impl;

namespace {
template <bool TRANS, typename Epi>
hipError_t launch_qkv_part(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const Epi& epi, hipStream_t s) {
  // The V epilogue holds too many live values next to 256 accumulators per
  // lane: V columns always use the 128 x 128 tiles.
  bool big = false;
  if constexpr (TRANS) big = use_big(M, N);
  if constexpr (TRANS) {
    if (big) {
      hipLaunchKernelGGL((gemm16_kernel<BigCfg, BF16, TRANS, Epi>), dim3(tiles_of(M, N, 256, 256)),
                         dim3(BigCfg::NT), 0, s, A, Bt, M, N, K, epi);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm16_kernel<SmallCfg, BF16, TRANS, Epi>), dim3(tiles_of(M, N, 128, 128)),
                     dim3(SmallCfg::NT), 0, s, A, Bt, M, N, K, epi);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_qkv(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const QkvEpilogue& e, hipStream_t s) {
  // Columns [n_base, n_base + N) of [Q|K|V]: the Q and K part runs with
  // transposed tiles, the V part with normal tiles.
  const int n_lo = e.n_base, n_hi = e.n_base + N, split = 2 * e.D;
  if (n_lo < split) {
    QkEpi epi{e};
    const hipError_t err = launch_qkv_part<true>(A, M, K, Bt, min(n_hi, split) - n_lo, epi, s);
    if (err != hipSuccess) return err;
  }
  if (n_hi > split) {
    const int v_lo = max(n_lo, split);
    VEpi epi{e};
    epi.e.n_base = v_lo;
    return launch_qkv_part<false>(A, M, K, Bt + (size_t)(v_lo - n_lo) * K, n_hi - v_lo, epi, s);
  }
  return hipSuccess;
}

hipError_t launch_early_out(const float* O32, int M, int K, const uint16_t* WoT, int N,
                            const uint16_t* bias, float* Y, int R, int T_q, hipStream_t s) {
  dim3 grid(N / 32, (M + 31) / 32);
  hipLaunchKernelGGL(early_out_kernel, grid, dim3(256), 0, s, O32, M, K, WoT, N, bias, Y, R, T_q);
  return hipGetLastError();
}

hipError_t launch_gemm_out(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const uint16_t* bias, float* Y, hipStream_t s) {
  OutEpi epi{bias, Y};
  if (use_big(M, N))
    hipLaunchKernelGGL((gemm16_kernel<BigCfg, F16, false, OutEpi>), dim3(tiles_of(M, N, 256, 256)),
                       dim3(BigCfg::NT), 0, s, A, Bt, M, N, K, epi);
  else
    hipLaunchKernelGGL((gemm16_kernel<SmallCfg, F16, false, OutEpi>), dim3(tiles_of(M, N, 128, 128)),
                       dim3(SmallCfg::NT), 0, s, A, Bt, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace mha
