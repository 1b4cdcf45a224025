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
// A is row-major M x K. The QKV projection reads W_QKV as it is given (K x N
// row-major, through transposing LDS reads); the output projection reads
// W_O^T (N x K, converted to fp16 by the preparation kernel). Tiles are staged
// through LDS by asynchronous global->LDS copies, two K slices in flight;
// each wave owns a WM x WN sub-tile computed with v_mfma_f32_32x32x16.
#include <utility>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mha {

// Kernel templates are instantiated directly in the non-template launch
// functions below (instantiating them from inside another template left their
// host stubs undefined).
namespace gemm_impl {

// BM x BN output tile, WM x WN per wave, BK-deep K slices (32 or 64 16-bit
// elements: 64- or 128-byte LDS rows), NS slices in flight, OCC waves per
// SIMD (the register budget: 512 / OCC per lane, accumulators included).
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_, int OCC_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_, OCC = OCC_;
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
  static_assert(NS >= 2 && NS <= 5, "pipeline depth");
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

// Scheduling hints for one run of MFMAs (0x008 = MFMA, 0x100 = LDS read,
// 0x020 = global load): SLOTS slots of one MFMA each, the NR LDS reads spread
// over the first slots, then the NV global loads over the slots after them.
constexpr int clamp_count(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

template <int D, int V>
__device__ __forceinline__ void sched_slot() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
  if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
}

template <int SLOTS, int NR, int NV, int... S>
__device__ __forceinline__ void sched_run(std::integer_sequence<int, S...>) {
  constexpr int DPER = (NR + SLOTS - 1) / SLOTS;
  constexpr int ND = DPER ? (NR + DPER - 1) / DPER : 0;
  constexpr int VSL = SLOTS - ND > 0 ? SLOTS - ND : SLOTS;   // slots that take loads
  constexpr int V0 = SLOTS - ND > 0 ? ND : 0;                 // first of them
  constexpr int VPER = (NV + VSL - 1) / VSL;
  (sched_slot<clamp_count(NR - S * DPER, DPER),
              S < V0 ? 0 : clamp_count(NV - (S - V0) * VPER, VPER)>(), ...);
}

template <int SLOTS, int NR, int NV>
__device__ __forceinline__ void sched_run() {
  sched_run<SLOTS, NR, NV>(std::make_integer_sequence<int, SLOTS>{});
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order.
template <typename F, int... S>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// TRANS computes each 32 x 32 tile as (B^T A^T)^T: the MFMA result then holds,
// per lane, one row m and four consecutive columns n (instead of one column
// and four consecutive rows).
// BROW: the second operand is given row-major, B (K x N, row stride ldb), as
// the projection weights are, instead of N x K: its K slices are copied as
// BK rows of BN columns and the MFMA fragments (8 consecutive k of one
// column per lane) are read with the transposing LDS read.
// Tile order: each XCD takes a contiguous range of logical tiles, walked in
// groups of GM row bands so that the concurrently resident workgroups of an
// XCD share A rows and B columns in its L2. (m0, n0): this workgroup's tile.
#ifndef MHA_GEMM_GM
#define MHA_GEMM_GM 8
#endif
template <typename C>
__device__ __forceinline__ void tile_origin(int M, int N, int& m0, int& n0) {
  constexpr int GM = MHA_GEMM_GM;
  const int ntn = (N + C::BN - 1) / C::BN, ntm = (M + C::BM - 1) / C::BM;
  const int logical = xcd_remap(blockIdx.x, ntn * ntm);
  const int group = logical / (GM * ntn);
  const int gm0 = group * GM, gsz = min(GM, ntm - gm0);
  const int in_group = logical - group * GM * ntn;
  const int bm = gm0 + in_group % gsz, bn = in_group / gsz;
  m0 = bm * C::BM;
  n0 = bn * C::BN;
}

// One output tile at (m0, n0), with the workgroup's LDS `smem` (NS * STAGE bytes).
template <typename C, typename Tag, bool TRANS, typename Epi, bool BUF, bool BROW>
__device__ __forceinline__ void gemm16_tile(const uint16_t* __restrict__ A,
                                            const uint16_t* __restrict__ Bt, int M, int N, int K,
                                            int ldb, const Epi& epi, int m0, int n0,
                                            uint8_t* smem) {
  // wave index in a scalar register: the DMA LDS bases below stay scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // DMA of K slice kt into stage `stage`: lane chunk p of a wave-wide load
  // lands at byte 16*p of the wave's 1 KiB window and fetches the global
  // chunk the swizzled layout places there. Rows past M or N are clamped
  // (their results are never stored).
  // BUF: the operands are under 2 GiB each, so every copy is a buffer load
  // with a loop-invariant per-lane byte offset and the slice's scalar offset.
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A, BUF ? (uint32_t)M * K * 2 : 0u);
  const __amdgpu_buffer_rsrc_t rb =
      buffer_rsrc(Bt, BUF ? (uint32_t)(BROW ? K * ldb : N * K) * 2 : 0u);
  // BROW stage layout: BK rows of BCH 16-byte chunks; chunk c of row r sits
  // at c ^ 4 (r & 3), so the four rows one transposing read takes land on
  // four different 64-byte bank groups.
  constexpr int BCH = C::BN / 8;
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    uint8_t* as = smem + stage * C::STAGE;
    uint8_t* bs = as + C::A_BYTES;
    const int k0 = kt * C::BK;
    if constexpr (BUF) {
#pragma unroll
      for (int i = 0; i < C::A_LPT; ++i) {
        const int p = i * C::NT + tid, row = p / C::CH, c = swz<C::CH>(row, p % C::CH);
        const int m = min(m0 + row, M - 1);
        lds_dma16_buf(ra, (uint32_t)(m * K + c * 8) * 2u, (uint32_t)k0 * 2u,
                      as + (i * C::NT + wave * 64) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::B_LPT; ++i) {
        if constexpr (BROW) {
          const int p = i * C::NT + tid, r = p / BCH, c = (p % BCH) ^ ((r & 3) << 2);
          const int n = min(n0 + c * 8, N - 8);
          lds_dma16_buf(rb, (uint32_t)(r * ldb + n) * 2u, (uint32_t)k0 * (uint32_t)ldb * 2u,
                        bs + (i * C::NT + wave * 64) * 16);
        } else {
          const int p = i * C::NT + tid, row = p / C::CH, c = swz<C::CH>(row, p % C::CH);
          const int n = min(n0 + row, N - 1);
          lds_dma16_buf(rb, (uint32_t)(n * K + c * 8) * 2u, (uint32_t)k0 * 2u,
                        bs + (i * C::NT + wave * 64) * 16);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::A_LPT; ++i) {
      const int p = i * C::NT + tid, row = p / C::CH, c = swz<C::CH>(row, p % C::CH);
      const int m = min(m0 + row, M - 1);
      lds_dma16(A + (size_t)m * K + k0 + c * 8,
                as + (i * C::NT + wave * 64) * 16);
    }
#pragma unroll
    for (int i = 0; i < C::B_LPT; ++i) {
      if constexpr (BROW) {
        const int p = i * C::NT + tid, r = p / BCH, c = (p % BCH) ^ ((r & 3) << 2);
        const int n = min(n0 + c * 8, N - 8);
        lds_dma16(Bt + (size_t)(k0 + r) * ldb + n, bs + (i * C::NT + wave * 64) * 16);
      } else {
        const int p = i * C::NT + tid, row = p / C::CH, c = swz<C::CH>(row, p % C::CH);
        const int n = min(n0 + row, N - 1);
        lds_dma16(Bt + (size_t)n * K + k0 + c * 8,
                  bs + (i * C::NT + wave * 64) * 16);
      }
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
  const int arow0 = wm * C::WM + (lane & 31), brow0 = wn * C::WN + (lane & 31);
  const int lh = lane >> 5;
  // BROW fragment reads: lane 16 g + 4 e + q of a transposing read names row
  // 16 ks + 8 (g / 2) + 4 h + e (h = 0, 1: the two reads of a fragment) and
  // columns 32 j + 16 (g % 2) + 4 q .. +3 of the wave's tile; lane l then
  // holds column l % 32 at k = 16 ks + 8 (l / 32) + 4 h + 0..3, the same k as
  // the A fragment's 16-byte chunk. Row 16 ks + ... has (row & 3) = e.
  int trb[C::TN];
  if constexpr (BROW) {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      trb[j] = (8 * (g >> 1) + e) * BCH * 16 +
               ((((wn * C::WN + 32 * j) >> 3) ^ (e << 2)) + 2 * (g & 1) + (q >> 1)) * 16 +
               (q & 1) * 8;
  }
  // Operand fragments of one 16-deep k-step, read from a stage (the step is a
  // compile-time constant: the transposing reads take their offsets as
  // immediates).
  auto frags_a = [&](const uint8_t* as, auto ksc, u32x4 (&fa)[C::TM])
      __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int row = arow0 + i * 32;
      fa[i] = *reinterpret_cast<const u32x4*>(as + (row * C::CH + swz<C::CH>(row, 2 * ks + lh)) * 16);
    }
  };
  auto frags_b = [&](const uint8_t* as, auto ksc, u32x4 (&fb)[C::TN])
      __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value;
    const uint8_t* bs = as + C::A_BYTES;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      if constexpr (BROW) {
        const uint32_t ad = lds_addr(as) + trb[j];
        const u32x2 lo = lds_read_tr16<C::A_BYTES + 16 * ks * BCH * 16>(ad);
        const u32x2 hi = lds_read_tr16<C::A_BYTES + (16 * ks + 4) * BCH * 16>(ad);
        fb[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        const int row = brow0 + j * 32;
        fb[j] = *reinterpret_cast<const u32x4*>(bs + (row * C::CH + swz<C::CH>(row, 2 * ks + lh)) * 16);
      }
    }
  };
  auto frags = [&](const uint8_t* as, auto ksc, u32x4 (&fa)[C::TM], u32x4 (&fb)[C::TN])
      __attribute__((always_inline)) {
    frags_a(as, ksc, fa);
    frags_b(as, ksc, fb);
  };
  auto frag_a_at = [&](const uint8_t* as, auto ksc, int i) __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value;
    const int row = arow0 + i * 32;
    return *reinterpret_cast<const u32x4*>(as + (row * C::CH + swz<C::CH>(row, 2 * ks + lh)) * 16);
  };
  auto frag_b_tr_at = [&](const uint8_t* as, auto ksc, int j) __attribute__((always_inline)) {
    constexpr int ks = decltype(ksc)::value;
    const uint32_t ad = lds_addr(as) + trb[j];
    const u32x2 lo = lds_read_tr16<C::A_BYTES + 16 * ks * BCH * 16>(ad);
    const u32x2 hi = lds_read_tr16<C::A_BYTES + (16 * ks + 4) * BCH * 16>(ad);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  auto mfma_one = [&](int idx, const u32x4 (&fa)[C::TM], const u32x4 (&fb)[C::TN])
      __attribute__((always_inline)) {
    const int i = idx / C::TN, j = idx % C::TN;
    acc[i][j] = TRANS ? mfma32x32x16<Tag>(fb[j], fa[i], acc[i][j])
                      : mfma32x32x16<Tag>(fa[i], fb[j], acc[i][j]);
  };

  // Pipeline. Load group g carries K slice min(g, nk-1) into stage g % NS;
  // groups 0..NS-1 go out first, then one more group per slice boundary. In
  // the last k-step of slice kt, after a few MFMAs are queued, every wave
  // waits for slice kt+1 (NS-2 younger groups may stay in flight) and meets
  // at a barrier: slice kt+1 is then visible to all waves and the stage of
  // slice kt is no longer read, so group kt+NS is issued into it and the
  // first fragments of slice kt+1 are read under the remaining MFMAs of slice
  // kt. Groups past the last slice re-read it into a stage nobody reads again
  // (which keeps the group count, and so every vmcnt wait, uniform).
#pragma unroll
  for (int t = 0; t < C::NS; ++t) issue(min(t, nk - 1), t);
  wait_vmcnt<(C::NS - 1) * C::LPT>();
  __builtin_amdgcn_s_barrier();

  // (NR counts the reads the scheduler sees: not the assembly ones)
  constexpr int KS = C::BK / 16, NR = C::TM + (BROW ? 0 : C::TN), NMF = C::TM * C::TN;
#ifndef MHA_GEMM_PRE
#define MHA_GEMM_PRE 2
#endif
  // MFMAs of the last k-step queued before the barrier
  constexpr int PRE = MHA_GEMM_PRE < NMF ? MHA_GEMM_PRE : NMF / 2;
  static_assert(PRE >= 1 && PRE < NMF, "schedule shape");
  constexpr int LB = (KS - 1) & 1;   // fragment buffer of the last k-step
  u32x4 a[2][C::TM], b[2][C::TN];
  // All k-steps of slice kt but the last, and the first PRE MFMAs of the last.
  // BROW: each k-step first waits for its fragments (read during the
  // previous k-step), then issues the next k-step's transposing reads ahead of
  // everything else (the scheduler does not count them as LDS reads and would
  // otherwise leave them to the end of the step), then its A reads spread
  // over its MFMAs.
  auto slice_head = [&](int kt) __attribute__((always_inline)) {
    const uint8_t* as = smem + (kt % C::NS) * C::STAGE;
    if constexpr (BROW) {
      static_for<KS - 1>([&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value, cur = ks & 1, nxt = cur ^ 1;
        lds_tr_wait(b[cur], a[cur]);
        // MFMA q, then read group q of the next k-step: the TN transposed B
        // fragments first (two reads each), then the TM A fragments; the
        // order is fixed with scheduling barriers.
        static_for<NMF>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          mfma_one(q, a[cur], b[cur]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (q < C::TN) {
            b[nxt][q] = frag_b_tr_at(as, std::integral_constant<int, ks + 1>{}, q);
          } else if constexpr (q < C::TN + C::TM) {
            a[nxt][q - C::TN] = frag_a_at(as, std::integral_constant<int, ks + 1>{}, q - C::TN);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        static_for<(C::TN + C::TM > NMF ? C::TN + C::TM - NMF : 0)>([&](auto rc)
            __attribute__((always_inline)) {
          constexpr int r = decltype(rc)::value + NMF;
          if constexpr (r < C::TN) b[nxt][r] = frag_b_tr_at(as, std::integral_constant<int, ks + 1>{}, r);
          else a[nxt][r - C::TN] = frag_a_at(as, std::integral_constant<int, ks + 1>{}, r - C::TN);
        });
      });
      lds_tr_wait(b[LB], a[LB]);
#pragma unroll
      for (int q = 0; q < PRE; ++q) mfma_one(q, a[LB], b[LB]);
    } else {
      static_for<KS - 1>([&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value;
        frags(as, std::integral_constant<int, ks + 1>{}, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
        for (int q = 0; q < NMF; ++q) mfma_one(q, a[ks & 1], b[ks & 1]);
      });
#pragma unroll
      for (int q = 0; q < PRE; ++q) mfma_one(q, a[LB], b[LB]);
      // Issue order: the next k-step's reads go out one per MFMA over the
      // first MFMAs, so the remaining ones cover their latency.
#pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) sched_run<NMF, NR, 0>();
    }
  };
  frags(smem, std::integral_constant<int, 0>{}, a[0], b[0]);
  for (int kt = 0; kt < nk - 1; ++kt) {
    slice_head(kt);
    // (sched_barrier: nothing may be moved across the wait and the barrier,
    // MFMAs included, so exactly the MFMAs above are queued while waiting.)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(C::NS - 2) * C::LPT>();
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (BROW) {
      const uint8_t* nx = smem + ((kt + 1) % C::NS) * C::STAGE;
      frags_b(nx, std::integral_constant<int, 0>{}, b[0]);
      __builtin_amdgcn_sched_barrier(0);
      issue(min(kt + C::NS, nk - 1), kt % C::NS);
      frags_a(nx, std::integral_constant<int, 0>{}, a[0]);
    } else {
      issue(min(kt + C::NS, nk - 1), kt % C::NS);
      frags(smem + ((kt + 1) % C::NS) * C::STAGE, std::integral_constant<int, 0>{}, a[0], b[0]);
    }
#pragma unroll
    for (int q = PRE; q < NMF; ++q) mfma_one(q, a[LB], b[LB]);
    // Reads of the next slice's first k-step first, then the new group's
    // global->LDS loads, spread over the remaining MFMAs.
    sched_run<NMF - PRE, NR, C::LPT>();
  }
  slice_head(nk - 1);
#pragma unroll
  for (int q = PRE; q < NMF; ++q) mfma_one(q, a[LB], b[LB]);
  wait_vmcnt<0>();   // no global->LDS copy may outlive the workgroup
  // Every wave has finished reading the stages: each wave may now use its
  // share of the LDS to stage its output tile.
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  static_assert(C::WM * C::WN * 2 <= C::NS * C::STAGE / C::NWAVES, "staging window");
  epi.template apply<C::TM, C::TN>(acc, m0 + wm * C::WM, n0 + wn * C::WN, lane, M, N,
                                   smem + wave * (C::NS * C::STAGE / C::NWAVES));
}

template <typename C, typename Tag, bool TRANS, typename Epi, bool BUF, bool BROW>
__global__ void __launch_bounds__(C::NT, C::OCC)
gemm16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, int M, int N,
              int K, int ldb, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NS * C::STAGE];
  int m0, n0;
  tile_origin<C>(M, N, m0, n0);
  gemm16_tile<C, Tag, TRANS, Epi, BUF, BROW>(A, Bt, M, N, K, ldb, epi, m0, n0, smem);
}

// Output staging: 16-byte chunk c of LDS row `row` (RB bytes per row) sits at
// a row-dependent XOR of c so that the 8-byte writes of 32 lanes to 32
// consecutive rows spread over the banks.
template <int RB>
__device__ __forceinline__ int stage_chunk(int row, int c) {
  return RB == 128 ? (c ^ ((row >> 1) & 7)) : (c ^ (row & 15));
}

// Head-split epilogues of the QKV projection. [Q|K|V] has a D-wide Q block
// (h heads) and Dkv-wide K and V blocks (h_kv key/value sets); inside a block,
// column c is head c / d_k, channel c mod d_k. Row m is batch m / T, position
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
// Every tile goes through LDS: the wave's fp16 tile is staged row by row, then
// written back 16 bytes per lane. Each 16-byte chunk is 8 channels of one
// head at one position; runs of a head are contiguous in (B, h, T, d_k).
struct QkEpi {
  QkvEpilogue e;

  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x16_t (&acc)[TM][TN], int mbase, int nbase, int lane,
                                        int M, int N, uint8_t* lds) const {
    constexpr int WM = TM * 32, WN = TN * 32, RB = WN * 2, CPR = WN / 8;
    const int D = e.D, d_k = e.d_k, T = e.T, lq = lane & 31, lh = lane >> 5;
    const int bw = mbase / T, tw = mbase - bw * T;
    // The wave's WN columns lie in one of Q or K (WN divides D; the K block
    // ends at N).
    const int NQKV = D + 2 * e.Dkv;
    const int ng0 = e.n_base + nbase, which = ng0 >= D ? 1 : 0, hc0 = ng0 - which * D;
    const float sc = which == 0 ? e.q_scale : 1.0f;
    // The wave's bias values, fetched together (one latency, not one per
    // fragment): lane columns ng0 + 32 j + 8 rg + 4 lh + 0..3 (clamped to the
    // last column; values past N are never stored).
    u32x2 bb[TN][4];
    if (e.bias) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          bb[j][rg] = *reinterpret_cast<const u32x2*>(
              e.bias + e.n_base + min(nbase + j * 32 + 8 * rg + 4 * lh, N - 4));
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) bb[j][rg] = u32x2{0u, 0u};
    }
    auto biased = [&](int i, int j, int rg, float (&v)[4]) __attribute__((always_inline)) {
      const f32x16_t& a = acc[i][j];
      const u32x2 b2 = bb[j][rg];
      v[0] = a[rg * 4 + 0] + __uint_as_float(b2.x << 16);
      v[1] = a[rg * 4 + 1] + __uint_as_float(b2.x & 0xffff0000u);
      v[2] = a[rg * 4 + 2] + __uint_as_float(b2.y << 16);
      v[3] = a[rg * 4 + 3] + __uint_as_float(b2.y & 0xffff0000u);
    };
    // Rows t < early_rows also go out in fp32 (tiles holding such rows only).
    if (e.early && (tw < e.early_rows || tw + WM > T)) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = mbase + i * 32 + lq;
        const int b = m / T, t = m - b * T;
        if (m < M && t < e.early_rows) {
          float* er = e.early + ((size_t)b * e.early_rows + t) * NQKV + ng0;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int c = j * 32 + 8 * rg + 4 * lh;
              if (nbase + c < N) {
                float v[4];
                biased(i, j, rg, v);
                *reinterpret_cast<f32x4_t*>(er + c) = f32x4_t{v[0], v[1], v[2], v[3]};
              }
            }
        }
      }
    }
    // fp16 tile into LDS, one 32-row block at a time (the scheduling fence
    // keeps the compiler from hoisting every block's accumulator reads).
    // amax: the largest magnitude stored (NaN if a value is NaN).
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = i * 32 + lq;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int c = j * 32 + 8 * rg + 4 * lh;
          float v[4];
          biased(i, j, rg, v);
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] *= sc;
          amax = vmax3(amax, fabsf(v[0]), fabsf(v[1]));
          amax = vmax3(amax, fabsf(v[2]), fabsf(v[3]));
          *reinterpret_cast<u32x2*>(lds + r * RB + stage_chunk<RB>(r, c >> 3) * 16 + lh * 8) =
              u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    flag_f16_overflow(e.overflow, amax);
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
    // Write-back. Chunk order: head segment, row, chunk within the segment,
    // so consecutive lanes cover contiguous memory.
    const int hseg = min(WN, d_k), lg_cph = hseg == 128 ? 4 : 3;   // chunks per head segment
    const int tpad = which == 0 ? e.Tpad_q : e.Tpad_kv;
    const int nheads = which == 0 ? e.h : e.h_kv;
    uint16_t* const dst = which == 0 ? e.q : e.k;
    const bool simple = tw + WM <= T && mbase + WM <= M && nbase + WN <= N;
#pragma unroll 4
    for (int k = 0; k < WM * CPR / 64; ++k) {
      const int idx = k * 64 + lane;
      const int cb = idx >> (lg_cph + __builtin_ctz(WM)), rem = idx & ((WM << lg_cph) - 1);
      const int r = rem >> lg_cph, c8 = (cb << lg_cph) + (rem & ((1 << lg_cph) - 1));
      const u32x4 val = *reinterpret_cast<const u32x4*>(lds + r * RB + stage_chunk<RB>(r, c8) * 16);
      const int col = hc0 + c8 * 8, head = col / d_k, ch = col - head * d_k;
      int b = bw, t = tw + r;
      if (!simple) {   // tile crosses a sequence end or the matrix edge
        const int m = mbase + r;
        if (m >= M || nbase + c8 * 8 >= N) continue;
        b = m / T;
        t = m - b * T;
      }
      __builtin_nontemporal_store(
          val, reinterpret_cast<u32x4*>(dst + (((size_t)b * nheads + head) * tpad + t) * d_k + ch));
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
    const int NQKV = D + 2 * e.Dkv, v0 = D + e.Dkv;   // V block starts at column v0
    const int bw = mbase / T, tw = mbase - bw * T;
    // One batch element, a full tile, and a start on a 16-position group so
    // the position permutation stays inside the tile.
    const bool staged = (tw & 15) == 0 && tw + WM <= T && mbase + WM <= M && nbase + WN <= N;
    if (staged) {
      const int hc0 = e.n_base + nbase - v0;
      float amax = 0.0f;   // the largest magnitude stored (NaN if a value is NaN)
      float bj[TN];   // the wave's bias values, fetched together
      if (e.bias) {
#pragma unroll
        for (int j = 0; j < TN; ++j) bj[j] = bf16_bits_to_float(e.bias[e.n_base + nbase + j * 32 + lq]);
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) bj[j] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = j * 32 + lq;
        const int ng = e.n_base + nbase + c;
        const float bias = bj[j];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int r0 = i * 32 + 8 * rg + 4 * lh;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[i][j][rg * 4 + r] + bias;
            amax = vmax3(amax, fabsf(v[0]), fabsf(v[1]));
            amax = vmax3(amax, fabsf(v[2]), fabsf(v[3]));
            if (e.early && tw + r0 < e.early_rows) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (tw + r0 + r < e.early_rows)
                  e.early[((size_t)bw * e.early_rows + tw + r0 + r) * NQKV + ng] = v[r];
            }
            const int pos = vt_pos(r0);
            *reinterpret_cast<u32x2*>(lds + c * RB + stage_chunk<RB>(c, pos >> 3) * 16 +
                                      (pos & 7) * 2) =
                u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
          }
      }
      flag_f16_overflow(e.overflow, amax);
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
      // Write-back: each V^T row segment of WM positions is contiguous.
#pragma unroll 4
      for (int k = 0; k < WN * CPR / 64; ++k) {
        const int idx = k * 64 + lane;
        const int c = idx / CPR, p8 = idx - c * CPR;
        const u32x4 val = *reinterpret_cast<const u32x4*>(lds + c * RB + stage_chunk<RB>(c, p8) * 16);
        const int col = hc0 + c, head = col / d_k, ch = col - head * d_k;
        __builtin_nontemporal_store(
            val, reinterpret_cast<u32x4*>(e.vt + (((size_t)bw * e.h_kv + head) * d_k + ch) * e.Tpad_kv +
                                          tw + p8 * 8));
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = nbase + j * 32 + lq;
      if (n >= N) continue;
      const int ng = e.n_base + n;
      const int hc = ng - v0, head = hc / d_k, c = hc - head * d_k;
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
              e.early[((size_t)b * e.early_rows + t) * NQKV + ng] = v[r];
            e.vt[(((size_t)b * e.h_kv + head) * d_k + c) * e.Tpad_kv + vt_pos(t)] =
                float_to_f16_bits(v[r]);
            flag_f16_overflow(e.overflow, fabsf(v[r]));
          }
        }
      }
    }
  }
};

// Result epilogue of the output projection, on transposed tiles: a lane holds
// row m and four consecutive columns n..n+3 per fragment group. The bias is
// added in registers; each 32-row block of the wave's tile then goes through
// the wave's LDS window (fp32, 16-byte chunks XOR-swizzled by row so that
// both the fragment writes and the row reads are free of bank conflicts) and
// out row by row: one store instruction covers two whole row segments of the
// tile (WN * 4 bytes each), the residual (bf16) is read in the same order and
// the bf16 result, if asked for, converted there.
template <bool RESID, bool YBF16>
struct OutEpi {
  const uint16_t* bias;
  void* Y;               // fp32, or bf16 with YBF16
  const uint16_t* resid; // (M x N) bf16 added to the result with RESID
  template <int TM, int TN>
  __device__ __forceinline__ void apply(f32x16_t (&acc)[TM][TN], int mbase, int nbase, int lane,
                                        int M, int N, uint8_t* lds) const {
    constexpr int WN = TN * 32, CPR = WN / 4;   // 16-byte chunks per staged row
    static_assert(CPR == 16 || CPR == 32, "staged row width");
    const int lq = lane & 31, lh = lane >> 5;
    // The wave's bias values, fetched together (clamped to the last columns;
    // values past N are never stored).
    u32x2 bb[TN][4];
    if (bias) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          bb[j][rg] = *reinterpret_cast<const u32x2*>(bias + min(nbase + j * 32 + 8 * rg + 4 * lh, N - 4));
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) bb[j][rg] = u32x2{0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // fragments of rows i*32 .. i*32+31 into LDS (row lq, chunk 8 j + 2 rg + lh)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x16_t& a = acc[i][j];
          const u32x2 b2 = bb[j][rg];
          const f32x4_t v = {a[rg * 4 + 0] + __uint_as_float(b2.x << 16),
                             a[rg * 4 + 1] + __uint_as_float(b2.x & 0xffff0000u),
                             a[rg * 4 + 2] + __uint_as_float(b2.y << 16),
                             a[rg * 4 + 3] + __uint_as_float(b2.y & 0xffff0000u)};
          const int c = 8 * j + 2 * rg + lh;
          *reinterpret_cast<f32x4_t*>(lds + lq * (CPR * 16) + ((c ^ (lq & 15)) << 4)) = v;
        }
      // rows out: 64 / CPR rows per instruction, each row segment contiguous;
      // the block's residual values are fetched together first (one latency)
      constexpr int KO = 32 * CPR / 64;
      u32x2 rr[RESID ? KO : 1];
      if constexpr (RESID) {
#pragma unroll
        for (int k = 0; k < KO; ++k) {
          const int idx = k * 64 + lane, r = idx / CPR, c = idx % CPR;
          const int m = min(mbase + i * 32 + r, M - 1), n = min(nbase + 4 * c, N - 4);
          rr[k] = *reinterpret_cast<const u32x2*>(resid + (size_t)m * N + n);
        }
      }
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
      // The block's staged rows, read back together (one LDS latency), then
      // stored: a block wholly inside Y by buffer stores (its rows as the
      // resource, one lane offset, the row group as a scalar offset), a block
      // at the edge of Y element-checked.
      f32x4_t vv[KO];
#pragma unroll
      for (int k = 0; k < KO; ++k) {
        const int idx = k * 64 + lane, r = idx / CPR, c = idx % CPR;
        vv[k] = *reinterpret_cast<const f32x4_t*>(lds + r * (CPR * 16) + ((c ^ (r & 15)) << 4));
        if constexpr (RESID) {
          const u32x2 r2 = rr[k];
          vv[k][0] += __uint_as_float(r2.x << 16);
          vv[k][1] += __uint_as_float(r2.x & 0xffff0000u);
          vv[k][2] += __uint_as_float(r2.y << 16);
          vv[k][3] += __uint_as_float(r2.y & 0xffff0000u);
        }
      }
      constexpr int ES = YBF16 ? 2 : 4;   // bytes per element of Y
      if (mbase + i * 32 + 32 <= M && nbase + WN <= N) {
        const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(
            static_cast<uint8_t*>(Y) + ((size_t)(mbase + i * 32) * N + nbase) * ES,
            (uint32_t)(32 * N * ES));
        const uint32_t voff = (uint32_t)((lane / CPR) * N + 4 * (lane % CPR)) * ES;
#pragma unroll
        for (int k = 0; k < KO; ++k) {
          const uint32_t soff = (uint32_t)(k * (64 / CPR) * N * ES);
          if constexpr (YBF16)
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{pack_bf16x2(vv[k][0], vv[k][1]), pack_bf16x2(vv[k][2], vv[k][3])}, ry,
                voff, soff, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, vv[k]), ry, voff,
                                                   soff, 0);
        }
      } else {
#pragma unroll
        for (int k = 0; k < KO; ++k) {
          const int idx = k * 64 + lane, r = idx / CPR, c = idx % CPR;
          const int m = mbase + i * 32 + r, n = nbase + 4 * c;
          if (m >= M || n >= N) continue;
          const size_t yi = (size_t)m * N + n;
          if constexpr (YBF16)
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Y) + yi) =
                u32x2{pack_bf16x2(vv[k][0], vv[k][1]), pack_bf16x2(vv[k][2], vv[k][3])};
          else
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(Y) + yi) = vv[k];
        }
      }
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // reads done before the next block
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Output projection of the first rows of each causal sequence, from their
// fp32 attention output: Y[b*T_q + t] = O32[b*R + t] . W_O + b_O for t < R.
// Each fp32 value x is split into fp16 hi = fp16(x) and lo = fp16(x - hi), and
// hi . W + lo . W is accumulated in fp32 on the fp16 MFMA, which keeps about
// 22 significant bits of x. A workgroup owns a 32 x 64 tile of Y. K is cut
// into 64-deep chunks dealt round-robin to the four waves; each wave copies
// its chunks of O (32 rows, fp32) and of W_O^T (64 columns, fp16) global ->
// LDS itself (1 KiB contiguous per instruction, two chunks in flight, no
// workgroup barrier), reads its MFMA fragments from there, and the four
// partial tiles are summed through LDS in a fixed order, each wave finishing
// and storing a quarter of the tile.
constexpr int EO_WAVES = 4;
constexpr int EO_TN = 2;                          // 32-column blocks per tile
constexpr int EO_KC = 64;                         // K per chunk
constexpr int EO_A_BYTES = 32 * EO_KC * 4;        // 8 KiB: 32 rows x 64 fp32
constexpr int EO_B_BYTES = 32 * EO_TN * EO_KC * 2;   // 8 KiB: 64 columns x 64 fp16
constexpr int EO_STAGE = EO_A_BYTES + EO_B_BYTES;

__global__ void __launch_bounds__(EO_WAVES * 64)
early_out_kernel(const float* __restrict__ O32, int M, int K, const uint16_t* __restrict__ WoT,
                 int N, const uint16_t* __restrict__ bias, OutOptions opt, int R, int T_q,
                 const float* __restrict__ gate, int h, int d_k) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[EO_WAVES * 2 * EO_STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32 * EO_TN;
  const int lq = lane & 31, lh = lane >> 5;
  uint8_t* const wbase = smem + wave * 2 * EO_STAGE;

  // Chunk `c` into stage `st`. LDS rows: A 256 bytes (16 chunks of 16 B,
  // chunk index XOR row & 15), B 128 bytes (8 chunks, XOR (row >> 1) & 7), so
  // the fragment reads below are free of bank conflicts; lane p of each
  // instruction lands at byte 16 p of a 1 KiB window and fetches the global
  // chunk that the swizzle places there. Rows past M are clamped (never
  // stored).
  auto issue = [&](int c, int st) __attribute__((always_inline)) {
    const int k0 = c * EO_KC;
    uint8_t* as = wbase + st * EO_STAGE;
    uint8_t* bs = as + EO_A_BYTES;
#pragma unroll
    for (int i = 0; i < EO_A_BYTES / 1024; ++i) {
      const int slot = i * 64 + lane, row = slot >> 4, ch = (slot & 15) ^ (row & 15);
      lds_dma16(O32 + (size_t)min(m0 + row, M - 1) * K + k0 + ch * 4, as + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < EO_B_BYTES / 1024; ++i) {
      const int slot = i * 64 + lane, row = slot >> 3, ch = (slot & 7) ^ ((row >> 1) & 7);
      lds_dma16(WoT + (size_t)(n0 + row) * K + k0 + ch * 8, bs + i * 1024);
    }
  };
  constexpr int LPC = (EO_A_BYTES + EO_B_BYTES) / 1024;   // DMA instructions per chunk

  f32x16_t acc[EO_TN];
#pragma unroll
  for (int j = 0; j < EO_TN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  const int nch = K / EO_KC;
  // this wave's chunks: wave, wave + 4, ...
  const int mine = nch > wave ? (nch - wave + EO_WAVES - 1) / EO_WAVES : 0;
  if (mine > 0) issue(wave, 0);
  if (mine > 1) issue(wave + EO_WAVES, 1);
  // gated attention: this lane's row (b, t) of O32; a 64-deep chunk lies in
  // one head (d_k % 64 == 0), so one gate per lane and chunk
  const int gm = min(m0 + lq, M - 1), gb = gm / R;
  const float* grow = gate ? gate + ((size_t)gb * T_q + (gm - gb * R)) * h : nullptr;
  for (int i = 0; i < mine; ++i) {
    const float gt = grow ? gate_sigmoid(grow[(wave + i * EO_WAVES) * EO_KC / d_k]) : 1.0f;
    if (i + 1 < mine) wait_vmcnt<LPC>();
    else wait_vmcnt<0>();
    const uint8_t* as = wbase + (i & 1) * EO_STAGE;
    const uint8_t* bs = as + EO_A_BYTES;
#pragma unroll
    for (int ks = 0; ks < EO_KC / 16; ++ks) {
      // A: this lane's 8 k-values of row lq are logical chunks 4 ks + 2 lh, +1.
      const int c0 = 4 * ks + 2 * lh;
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(as + lq * 256 + ((c0 ^ (lq & 15)) << 4));
      const f32x4_t a1 =
          *reinterpret_cast<const f32x4_t*>(as + lq * 256 + (((c0 + 1) ^ (lq & 15)) << 4));
      u32x4 bf[EO_TN];
#pragma unroll
      for (int j = 0; j < EO_TN; ++j) {
        const int row = j * 32 + lq;
        bf[j] = *reinterpret_cast<const u32x4*>(bs + row * 128 +
                                                (((2 * ks + lh) ^ ((row >> 1) & 7)) << 4));
      }
      const float av[8] = {a0[0] * gt, a0[1] * gt, a0[2] * gt, a0[3] * gt,
                           a1[0] * gt, a1[1] * gt, a1[2] * gt, a1[3] * gt};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 h0 = static_cast<_Float16>(av[2 * e]);
        const _Float16 h1 = static_cast<_Float16>(av[2 * e + 1]);
        hi[e] = __builtin_bit_cast(uint32_t, half2_t{h0, h1});
        lo[e] = pack_f16x2(av[2 * e] - static_cast<float>(h0), av[2 * e + 1] - static_cast<float>(h1));
      }
      const u32x4 ah = u32x4{hi[0], hi[1], hi[2], hi[3]}, al = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
      for (int j = 0; j < EO_TN; ++j) {
        acc[j] = mfma32x32x16<F16>(ah, bf[j], acc[j]);
        acc[j] = mfma32x32x16<F16>(al, bf[j], acc[j]);
      }
    }
    // The stage is refilled only after this wave's reads of it completed.
    if (i + 2 < mine) {
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
      issue(wave + (i + 2) * EO_WAVES, i & 1);
    }
  }

  // The four partial tiles through LDS (the staging area is free once every
  // wave has passed the barrier). Wave w then finishes row group w of the
  // tile (accumulator elements 4w..4w+3: rows 8w + 4 lh + 0..3), summing the
  // partials in wave order, so the stores are spread over the four waves.
  __syncthreads();
  f32x16_t(*red)[EO_TN][64] = reinterpret_cast<f32x16_t(*)[EO_TN][64]>(smem);
#pragma unroll
  for (int j = 0; j < EO_TN; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  // this lane's four rows of Y (row m of O32 is position t < R of batch bb)
  size_t yrow[4];
  bool ok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = m0 + 8 * wave + 4 * lh + e;
    ok[e] = m < M;
    const int bb = m / R, t = m - bb * R;
    yrow[e] = ((size_t)bb * T_q + t) * N;
  }
#pragma unroll
  for (int j = 0; j < EO_TN; ++j) {
    f32x4_t v = reinterpret_cast<const f32x4_t*>(&red[0][j][lane])[wave];
#pragma unroll
    for (int w = 1; w < EO_WAVES; ++w) v += reinterpret_cast<const f32x4_t*>(&red[w][j][lane])[wave];
    const int n = n0 + 32 * j + lq;
    const float bv = load_bias_bf16(bias, n);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!ok[e]) continue;
      const size_t yi = yrow[e] + n;
      float y = v[e] + bv;
      if (opt.resid) y += bf16_bits_to_float(opt.resid[yi]);
      if (opt.y_bf16)
        static_cast<uint16_t*>(opt.y)[yi] = static_cast<uint16_t>(pack_bf16x2(y, 0.0f) & 0xffffu);
      else
        static_cast<float*>(opt.y)[yi] = y;
    }
  }
}

// The whole [Q|K|V] (or [K|V]) column range of the projection in one launch
// of 256 x 256 tiles: a workgroup whose tile lies in the V block (columns
// n >= vcol) runs the V path (normal tiles, V^T epilogue), the others the
// Q/K path (transposed tiles). One launch instead of two lets each row band's
// tiles of all three blocks run together, and saves a launch boundary.
template <typename C, bool BUF>
__global__ void __launch_bounds__(C::NT, C::OCC)
gemm16_qkv_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, int M, int N,
                  int K, int ldw, QkEpi qk, VEpi ve, int vcol) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NS * C::STAGE];
  int m0, n0;
  tile_origin<C>(M, N, m0, n0);
  if (n0 >= vcol)
    gemm16_tile<C, BF16, false, VEpi, BUF, true>(A, W, M, N, K, ldw, ve, m0, n0, smem);
  else
    gemm16_tile<C, BF16, true, QkEpi, BUF, true>(A, W, M, N, K, ldw, qk, m0, n0, smem);
}

// Key/value sets of 64 columns (d_k = 64) on their own, as one key/value set
// shared by every query head (MQA) gives: the K and V blocks are one wave
// column each of a 128 x 128 tile, so the waves of the K half take the K
// path (transposed tile, QkEpi) and those of the V half the V path (VEpi),
// over the same staged slices and through the same barriers, instead of two
// launches of half-empty tiles.
template <typename C>
__global__ void __launch_bounds__(C::NT, C::OCC)
gemm16_kv64_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, int M, int N,
                   int K, int ldw, QkEpi qk, VEpi ve) {
  static_assert(C::WN == 64 && C::BN == 2 * C::WN, "one wave column per block");
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NS * C::STAGE];
  int m0, n0;
  tile_origin<C>(M, N, m0, n0);
  const int wn = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) % C::WAVES_N);
  if (wn == 0)
    gemm16_tile<C, BF16, true, QkEpi, false, true>(A, W, M, N, K, ldw, qk, m0, n0, smem);
  else
    gemm16_tile<C, BF16, false, VEpi, false, true>(A, W, M, N, K, ldw, ve, m0, n0, smem);
}

// Large problems: 256 x 256 tiles (below). Problems with too few such tiles
// to fill the 256 CUs use 128 x 128 tiles, four waves of 64 x 64 (two
// workgroups per CU).
#ifndef MHA_BIG_BK
#define MHA_BIG_BK 64
#endif
#ifndef MHA_BIG_NS
#define MHA_BIG_NS 2
#endif
#ifndef MHA_SMALL_BK
#define MHA_SMALL_BK 64
#endif
#ifndef MHA_SMALL_NS
#define MHA_SMALL_NS 2
#endif
// 256 x 256 tiles over 8 waves of 128 x 64 (two waves per SIMD, 128
// accumulators per lane): while one wave of a SIMD waits on its LDS reads or
// issues its share of the global->LDS copies, the other keeps the matrix core
// busy. (Four waves of 128 x 128 read a third less from LDS but leave each
// SIMD with a single wave: the QKV stage took 0.240 instead of 0.205 ms at
// D = 1024.)
using BigCfg = Cfg<256, 256, 128, 64, MHA_BIG_BK, MHA_BIG_NS, 2>;
using SmallCfg = Cfg<128, 128, 64, 64, MHA_SMALL_BK, MHA_SMALL_NS>;
// 256 x 128 tiles over 8 waves of 64 x 64, 32-deep slices, 3 stages (72 KiB):
// two workgroups per CU. For the single QKV launch when 256 x 256 tiles would
// leave a last round at most half full (the D = 512 workload: 384 big tiles,
// 1.5 rounds): its 768 tiles finish in about 1.2 big-tile rounds.
using MidCfg = Cfg<256, 128, 64, 64, 32, 3, 2>;

int tiles_of(int M, int N, int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); }
// Big tiles once they fill at least one round of the 256 CUs (one workgroup
// per CU): a launch of 256 big tiles (the Q|K columns at D = 512, measured
// when they ran as a launch of their own) took 41 instead of 44 us that way;
// half a round (128 tiles) is slower than the small tiles.
#ifndef MHA_GEMM_BIG_MIN_TILES
#define MHA_GEMM_BIG_MIN_TILES 256
#endif
// Operands small enough for buffer-addressed copies (32-bit byte offsets):
// A is M x K, the second operand `b_elems` 16-bit values (N x K, or K rows of
// stride ldb).
bool buf_ok(int M, int K, long long b_elems) {
  return (long long)M * K * 2 <= 0x7fffffffLL && b_elems * 2 <= 0x7fffffffLL;
}
bool use_big(int M, int N) {
  return tiles_of(M, N, BigCfg::BM, BigCfg::BN) >= MHA_GEMM_BIG_MIN_TILES;
}

}  // namespace gemm_impl

using namespace gemm_impl;

namespace {
// The projection weights are read as they are given, row-major (K x N, row
// stride ldw), through the transposing fragment reads.
template <bool TRANS, typename Epi>
hipError_t launch_qkv_part(const uint16_t* A, int M, int K, const uint16_t* W, int ldw, int N,
                           const Epi& epi, hipStream_t s) {
  if (use_big(M, N)) {
    if (buf_ok(M, K, (long long)K * ldw)) {
      hipLaunchKernelGGL((gemm16_kernel<BigCfg, BF16, TRANS, Epi, true, true>),
                         dim3(tiles_of(M, N, BigCfg::BM, BigCfg::BN)), dim3(BigCfg::NT), 0, s, A,
                         W, M, N, K, ldw, epi);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm16_kernel<BigCfg, BF16, TRANS, Epi, false, true>),
                       dim3(tiles_of(M, N, BigCfg::BM, BigCfg::BN)), dim3(BigCfg::NT), 0, s, A,
                       W, M, N, K, ldw, epi);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm16_kernel<SmallCfg, BF16, TRANS, Epi, false, true>),
                     dim3(tiles_of(M, N, SmallCfg::BM, SmallCfg::BN)), dim3(SmallCfg::NT), 0, s, A,
                     W, M, N, K, ldw, epi);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_qkv(const uint16_t* A, int M, int K, const uint16_t* W, int ldw, int N,
                           const QkvEpilogue& e, hipStream_t s) {
  // Columns [n_base, n_base + N) of [Q|K|V] (W points at column n_base): the
  // Q and K part runs with transposed tiles, the V part with normal tiles.
  if (N % 8 != 0 || ldw % 8 != 0 || K % 64 != 0) return hipErrorInvalidValue;
  const int n_lo = e.n_base, n_hi = e.n_base + N, split = e.D + e.Dkv;
  // With grouped key/value heads the K block is narrower than Q: Q runs as a
  // launch of its own, so that Q and the rest each pick their tile size (one
  // launch over D + Dkv columns would leave a mostly empty last round of
  // large tiles).
  int lo = n_lo;
  if (e.Dkv < e.D && n_lo < e.D && n_hi > e.D) {
    QkEpi epi{e};
    const hipError_t err = launch_qkv_part<true>(A, M, K, W, ldw, e.D - n_lo, epi, s);
    if (err != hipSuccess) return err;
    lo = e.D;
  }
  const uint16_t* Wl = W + (lo - n_lo);
  const int Nl = n_hi - lo;
  // One launch for both parts when the V block starts on a tile boundary and
  // the launch fills the CUs with 256 x 256 tiles.
  if (lo < split && n_hi > split && (split - lo) % BigCfg::BN == 0 && use_big(M, Nl)) {
    QkEpi qk{e};
    qk.e.n_base = lo;
    VEpi ve{e};
    ve.e.n_base = lo;
    const int tb = tiles_of(M, Nl, BigCfg::BM, BigCfg::BN);
    if (tb % 256 != 0 && tb % 256 <= 128 && tb < 4 * 256) {   // a ragged last round
      const dim3 gm(tiles_of(M, Nl, MidCfg::BM, MidCfg::BN));
      if (buf_ok(M, K, (long long)K * ldw))
        hipLaunchKernelGGL((gemm16_qkv_kernel<MidCfg, true>), gm, dim3(MidCfg::NT), 0, s, A, Wl, M,
                           Nl, K, ldw, qk, ve, split - lo);
      else
        hipLaunchKernelGGL((gemm16_qkv_kernel<MidCfg, false>), gm, dim3(MidCfg::NT), 0, s, A, Wl,
                           M, Nl, K, ldw, qk, ve, split - lo);
      return hipGetLastError();
    }
    const dim3 grid(tiles_of(M, Nl, BigCfg::BM, BigCfg::BN));
    if (buf_ok(M, K, (long long)K * ldw))
      hipLaunchKernelGGL((gemm16_qkv_kernel<BigCfg, true>), grid, dim3(BigCfg::NT), 0, s, A, Wl, M,
                         Nl, K, ldw, qk, ve, split - lo);
    else
      hipLaunchKernelGGL((gemm16_qkv_kernel<BigCfg, false>), grid, dim3(BigCfg::NT), 0, s, A, Wl,
                         M, Nl, K, ldw, qk, ve, split - lo);
    return hipGetLastError();
  }
  // [K|V] of one 64-column key/value set each (MQA, d_k = 64): one launch
  if (split - lo == SmallCfg::WN && n_hi - lo == SmallCfg::BN && !use_big(M, Nl)) {
    QkEpi qk{e};
    qk.e.n_base = lo;
    VEpi ve{e};
    ve.e.n_base = lo;
    hipLaunchKernelGGL((gemm16_kv64_kernel<SmallCfg>),
                       dim3(tiles_of(M, Nl, SmallCfg::BM, SmallCfg::BN)), dim3(SmallCfg::NT), 0, s,
                       A, Wl, M, Nl, K, ldw, qk, ve);
    return hipGetLastError();
  }
  if (lo < split) {
    QkEpi epi{e};
    epi.e.n_base = lo;
    const hipError_t err = launch_qkv_part<true>(A, M, K, Wl, ldw, min(n_hi, split) - lo, epi, s);
    if (err != hipSuccess) return err;
  }
  if (n_hi > split) {
    const int v_lo = max(lo, split);
    VEpi epi{e};
    epi.e.n_base = v_lo;
    return launch_qkv_part<false>(A, M, K, W + (v_lo - n_lo), ldw, n_hi - v_lo, epi, s);
  }
  return hipSuccess;
}

hipError_t launch_early_out(const float* O32, int M, int K, const uint16_t* WoT, int N,
                            const uint16_t* bias, const OutOptions& opt, int R, int T_q,
                            const float* gate, int h, int d_k, hipStream_t s) {
  if (N % (32 * EO_TN) != 0 || K % EO_KC != 0 || M < 1) return hipErrorInvalidValue;
  if (gate && (d_k < EO_KC || d_k % EO_KC != 0 || h * d_k != K)) return hipErrorInvalidValue;
  dim3 grid(N / (32 * EO_TN), (M + 31) / 32);
  hipLaunchKernelGGL(early_out_kernel, grid, dim3(EO_WAVES * 64), 0, s, O32, M, K, WoT, N, bias, opt,
                     R, T_q, gate, h, d_k);
  return hipGetLastError();
}

namespace {
template <bool RESID, bool YBF16>
hipError_t launch_out_variant(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                              const uint16_t* bias, const OutOptions& opt, hipStream_t s) {
  OutEpi<RESID, YBF16> epi{bias, opt.y, opt.resid};
  if (use_big(M, N))
    if (buf_ok(M, K, (long long)N * K))
      hipLaunchKernelGGL((gemm16_kernel<BigCfg, F16, true, OutEpi<RESID, YBF16>, true, false>),
                         dim3(tiles_of(M, N, BigCfg::BM, BigCfg::BN)), dim3(BigCfg::NT), 0, s, A,
                         Bt, M, N, K, K, epi);
    else
    hipLaunchKernelGGL((gemm16_kernel<BigCfg, F16, true, OutEpi<RESID, YBF16>, false, false>),
                       dim3(tiles_of(M, N, BigCfg::BM, BigCfg::BN)), dim3(BigCfg::NT), 0, s, A,
                       Bt, M, N, K, K, epi);
  else
    hipLaunchKernelGGL((gemm16_kernel<SmallCfg, F16, true, OutEpi<RESID, YBF16>, false, false>),
                       dim3(tiles_of(M, N, SmallCfg::BM, SmallCfg::BN)), dim3(SmallCfg::NT), 0,
                       s, A, Bt, M, N, K, K, epi);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_out(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const uint16_t* bias, const OutOptions& opt, hipStream_t s) {
  if (opt.resid) {
    if (opt.y_bf16) return launch_out_variant<true, true>(A, M, K, Bt, N, bias, opt, s);
    return launch_out_variant<true, false>(A, M, K, Bt, N, bias, opt, s);
  }
  if (opt.y_bf16) return launch_out_variant<false, true>(A, M, K, Bt, N, bias, opt, s);
  return launch_out_variant<false, false>(A, M, K, Bt, N, bias, opt, s);
}

}  // namespace mha
