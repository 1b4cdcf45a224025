// Fused scaled dot-product attention, fp16 MFMA operands, fp32 softmax state.
//
// Computes, per (batch, head) and query row i,
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k) + M_ij) v_j
// (itwiki "멀티 헤드 어텐션", 수식, eq. Attention; iamjaehka13.blog
// "[Deep Learning 5] Attention의 내부 계산", §7-§13) without forming the
// T_q x T_k score matrix. Keys are visited in tiles of 64 and the softmax is
// accumulated online, against a per-row reference value `base`: the partial
// numerator sum_j exp2(s_j - base) v_j and denominator sum_j exp2(s_j - base)
// are carried across tiles, and both are multiplied by exp2(base_old -
// base_new) when the reference moves. Any reference gives the same softmax
// in exact arithmetic (the factor exp2(-base) cancels). The reference stays
// 0 if the first tile's row maximum lies in [0, 8] (log2 units), else it
// becomes that maximum; afterwards it moves only when a score exceeds it by
// more than 8. Either way the exponentials stay in [0, 256] and the largest
// weight seen is at least 1, and most tiles need no rescaling. Scores are
// produced in log2 units: Q is stored pre-multiplied by log2(e)/sqrt(d_k), and
// the S accumulator starts at -base, or at the MFMA's constant 0 (no register
// initialisation) while every row of the wave still has reference 0.
//
// Masks: key j > query i under the causal mask and keys flagged in the
// padding mask (nonzero = ignore) get -inf, so their weight is exactly 0
// (iamjaehka13.blog §9; molayo1419.me "MHA란 무엇인가?", trap 2). Key tiles
// entirely in a query tile's future are skipped; key tiles beyond the last
// unmasked key of a batch element are never visited. A row with no unmasked
// key ends with l = 0 and writes 0 * (1/0) = NaN (molayo1419.me, trap 3).
//
// One wave's work per key tile: NQ x 32 query rows x 64 keys.
//   S^T = K . Q^T with v_mfma_f32_32x32x16_f16: the K tile is the A operand
//   (from LDS), Q^T the B operand (held in registers for the whole kernel).
//   The result puts one query per lane column, so the row max over keys is a
//   reduction inside a lane plus one exchange with lane l^32.
//   O^T += V^T . P^T: P^T is repacked from the S^T accumulators in registers
//   (fp16, round to nearest even) and used directly as the B operand. V^T
//   rows are stored with each 16-key group ordered {0-3, 8-11, 4-7, 12-15},
//   so the keys a lane half needs for one k-step form one 16-byte chunk.
//   Row sums of P go to the matrix cores too (VALU issue, not MFMA, is the
//   scarcer resource here): ones . P^T with v_mfma_f32_16x16x32_f16, whose A
//   operand is a lane selector (below), sums exactly the fp16 weights that
//   the P . V product uses.
//
// Data movement: K and V^T tiles (and, with a padding mask, the tile's 64-bit
// ignore mask) go from global memory straight into LDS with
// global_load_lds_dwordx4, up to NS tiles in flight. Tiles are stored
// unpadded with their 16-byte chunks XOR-swizzled by row so the MFMA operand
// reads spread over the LDS banks. The waits are explicit (s_waitcnt vmcnt +
// s_barrier): a __syncthreads() would wait for every outstanding load.
#include <math.h>

#include "device_common.h"
#include "kernels.h"
#include "transpose_tile.h"

namespace mha {

namespace {

// K and V bytes a group of interleaved causal units may span: twice one
// XCD's 4 MiB L2. What no longer fits the L2 is refetched from the Infinity
// Cache; the longer groups balance the causal schedule better than that costs.
#ifndef MHA_ATTN_GROUP_BYTES
#define MHA_ATTN_GROUP_BYTES (8LL << 20)
#endif
constexpr int BLOCK_N = 64;   // keys per tile
constexpr int NWAVES = 4;
constexpr int NT = NWAVES * 64;

__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / 8;
  if (L >= per * 8) return L;
  return (L % 8) * per + L / 8;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only (LDS reads and writes of this wave complete).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Physical 16-byte chunk of logical chunk c in row `row` of a tile.
template <int CHUNKS>
__device__ __forceinline__ int swz(int row, int c) {
  // 8 chunks per row (128-byte rows): pairs of rows share a 256-byte bank
  // window, so rows 2r and 2r+1 rotate by the same amount.
  return CHUNKS == 8 ? (c ^ ((row >> 1) & 7)) : (c ^ (row & 15));
}

// ---------------------------------------------------------------------------
// Early causal rows in fp32. Query rows t < rows of every causal sequence see
// at most 64 keys, so their outputs are averages of few value rows and are
// the largest of the layer; they are evaluated a second time here from the
// fp32 Q/K/V the QKV epilogue saved, and their output projection
// (early_out_kernel, which also applies the gates of gated attention to
// them) later overwrites those rows of Y. The workgroups doing
// this come first in the attention grid (their count rounded up to a
// multiple of 8, so the attention blocks keep their XCD placement); being
// short, they leave room to the long causal blocks within microseconds,
// which is cheaper than a launch of their own. A workgroup takes 4 er_rpw
// query rows of one (batch, head); 64 / er_rpw lanes share a row, each owning
// as many dimensions; all (<= 64) keys of the row sit in LDS as fp32 (rows
// past the extent zeroed, so the key loops have no branches), the scores in
// registers: two plain passes (maximum, then exponentials and the weighted
// sum of V), in log2 units.
// Query rows per wave of an early-row workgroup (4 waves): 16 at d_k = 64 (one
// workgroup per (batch element, head) for the 64 early rows, so each loads
// that head's keys and values once: the D = 512 attention 37.0 -> 35.2 us), 4
// at d_k = 128 (more rows per wave there made the D = 4096 attention slower).
template <int DK>
constexpr int er_rpw() { return DK == 64 ? 16 : 4; }
template <int DK>
constexpr int er_rows() { return 4 * er_rpw<DK>(); }   // query rows per early-row workgroup

// Sum over the 16 lanes of a DPP row (every lane gets the total):
// quad_perm xor 1, quad_perm xor 2, row_half_mirror, row_mirror.
// Sum over LPR consecutive lanes (4, 8 or 16; every lane gets its group's
// total): quad_perm xor 1, quad_perm xor 2, row_half_mirror, row_mirror.
template <int LPR>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "lane group");
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (LPR >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if constexpr (LPR >= 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

__host__ __device__ inline long long early_blocks(const AttnF32Args& e, int er) {
  return (long long)((e.rows + er - 1) / er) * e.h * e.B;
}

// blk: (row block, head, batch element) of the early rows, NWV waves of 4
// rows each; lds: at least 2 * 64 * DK * 4 bytes.
template <int DK, int NWV>
__device__ __forceinline__ void early_rows_block(const AttnF32Args& a, int blk, uint8_t* lds) {
  constexpr int RPW = er_rpw<DK>();   // query rows per wave
  constexpr int LPR = 64 / RPW;       // lanes per query row
  constexpr int CPL = DK / LPR;       // dimensions per lane
  constexpr int ERW = NWV * RPW;      // query rows per workgroup
  constexpr int NTW = NWV * 64;
  float (*Ks)[DK] = reinterpret_cast<float (*)[DK]>(lds);
  float (*Vs)[DK] = reinterpret_cast<float (*)[DK]>(lds + 64 * DK * 4);
  const int nx = (a.rows + ERW - 1) / ERW;
  const int bx = blk % nx, head = (blk / nx) % a.h, b = blk / (nx * a.h);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = lane % LPR;
  const int t = bx * ERW + wave * RPW + lane / LPR;
  const bool valid = t < a.rows;
  const int kend = a.causal ? min(a.T_k, bx * ERW + ERW) : a.T_k;   // <= 64 (host-checked)

  const float* kb = a.k + (size_t)b * a.kv_bstride + (head / a.group) * DK;
  const float* vb = a.v + (size_t)b * a.kv_bstride + (head / a.group) * DK;
  for (int idx = tid; idx < 64 * (DK / 4); idx += NTW) {
    const int key = idx / (DK / 4), c4 = (idx % (DK / 4)) * 4;
    f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = kv;
    if (key < kend) {
      kv = *reinterpret_cast<const f32x4_t*>(kb + (size_t)key * a.kv_ld + c4);
      vv = *reinterpret_cast<const f32x4_t*>(vb + (size_t)key * a.kv_ld + c4);
    }
    *reinterpret_cast<f32x4_t*>(&Ks[key][c4]) = kv;
    *reinterpret_cast<f32x4_t*>(&Vs[key][c4]) = vv;
  }
  // Keys this row ignores: past the extent, in the future, or padded.
  const bool padded = a.mask && lane < kend && a.mask[(size_t)b * a.mask_ld + lane] != 0;
  const uint64_t padm = __ballot(padded);

  // q pre-multiplied by log2(e) / sqrt(d_k): the softmax is exp2(s - max).
  const float scale = 1.4426950408889634f / sqrtf((float)DK);
  float q[CPL];
  const float* qp = a.q + (size_t)b * a.q_bstride + (size_t)(valid ? t : 0) * a.q_ld + head * DK +
                    p * CPL;
#pragma unroll
  for (int c = 0; c < CPL; c += 4) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(qp + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[c + e] = v[e] * scale;
  }
  __syncthreads();
  const int seen_keys = a.causal ? min(kend, t + 1) : kend;
  const uint64_t live = (seen_keys >= 64 ? ~0ull : ((1ull << max(seen_keys, 0)) - 1)) & ~padm;

  float sc[64];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) part = __builtin_fmaf(q[c], Ks[j][p * CPL + c], part);
    part = lanes_sum<LPR>(part);
    sc[j] = ((live >> j) & 1ull) ? part : -INFINITY;
    mx = fmaxf(mx, sc[j]);
  }
  const float base = mx == -INFINITY ? 0.0f : mx;
  float l = 0.0f, o[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = 0.0f;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float pj = __builtin_amdgcn_exp2f(sc[j] - base);
    l += pj;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = __builtin_fmaf(pj, Vs[j][p * CPL + c], o[c]);
  }
  if (valid) {
    float* op = a.o + (size_t)b * a.o_bstride + (size_t)t * a.o_ld + head * DK + p * CPL;
#pragma unroll
    for (int c = 0; c < CPL; c += 4)
      *reinterpret_cast<f32x4_t*>(op + c) =
          f32x4_t{o[c] / l, o[c + 1] / l, o[c + 2] / l, o[c + 3] / l};
  }
}

// Workgroup L (after the early-row workgroups) -> (batch, head, query block)
// for nqb query blocks per (batch, head). All query blocks of the heads that
// share one key/value set run on one XCD and share its L2 copy of K and V;
// under the causal mask the longest blocks are dispatched first. With a
// padding mask the work of a batch element grows with its key extent: the
// units (batch element, key/value set) are taken in `order` (longest extent
// first) and dealt round-robin to the 8 XCDs (hardware block L runs on XCD
// L % 8), so every XCD gets a like share and starts with its longest units.
template <bool HAS_MASK>
__device__ __forceinline__ void map_block(const AttnF16Args& a, int L, int nqb, int& b, int& head,
                                          int& qblk) {
  if (HAS_MASK && a.order != nullptr) {
    const int gh = a.h / a.h_kv, WU = gh * nqb, U = a.B * a.h_kv;
    int us, w;
    if (U % 8 == 0) {
      const int idx = L >> 3, j = idx / WU;
      us = (L & 7) + 8 * j;
      w = idx - j * WU;
    } else {
      us = L / WU;
      w = L - us * WU;
    }
    const int r = us / a.h_kv;
    b = a.order[r];
    head = (us - r * a.h_kv) * gh + w / nqb;
    qblk = w % nqb;
  } else {
    const int logical = xcd_remap(L, nqb * a.h * a.B);
    int bh0;
    if (a.group_units > 1 && a.causal) {
      // Groups of G (batch, head) units: their query blocks interleaved
      // longest first, so the long blocks of the last units of an XCD do not
      // trail at the end of the launch (G is bounded by MHA_ATTN_GROUP_BYTES
      // of K and V per group, twice one XCD's L2).
      const int G = a.group_units, units = a.h * a.B;
      const int g0 = (logical / (G * nqb)) * G, gs = min(G, units - g0);
      const int pos = logical - g0 * nqb;
      bh0 = g0 + pos % gs;
      qblk = pos / gs;
    } else {
      bh0 = logical / nqb;
      qblk = logical - bh0 * nqb;
    }
    b = bh0 / a.h;
    head = bh0 - b * a.h;
  }
  if (a.causal) qblk = nqb - 1 - qblk;
}

// d_k = 128: the register budget is capped at two waves per SIMD (247 VGPRs,
// no spill); with two pipeline stages (64 KiB of LDS) two workgroups then
// share a CU. d_k = 64: capped at three waves per SIMD (168 VGPRs; the W_O
// conversion path alone would let the compiler take a few more).
template <int DK, int NQ, int NS, bool HAS_MASK>
__global__ void __launch_bounds__(NT, (DK == 128 ? 2 : 3))
attn_f16_kernel(AttnF16Args a, AttnF32Args early, int early_slots) {
  constexpr int BLOCK_M = NWAVES * 32 * NQ;
  constexpr int KCH = DK / 8;                       // 16-byte chunks per K row
  constexpr int K_BYTES = BLOCK_N * DK * 2;
  constexpr int V_BYTES = DK * BLOCK_N * 2;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int K_LPT = K_BYTES / 16 / NT;          // DMA loads per thread per tile
  constexpr int V_LPT = V_BYTES / 16 / NT;
  constexpr int LPT = K_LPT + V_LPT + (HAS_MASK ? 1 : 0);
  constexpr int KSTEPS = DK / 16;
  constexpr int DT = DK / 32;
  static_assert(NS >= 2 && NS <= 4, "pipeline depth");
  // One LDS array (the tiles' masks at its end): with a second LDS variable
  // the compiler attaches alias scopes to the accesses and then makes every
  // LDS read wait for all outstanding global->LDS copies into the array.
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * STAGE + 32];
  uint32_t (*mask_s)[2] = reinterpret_cast<uint32_t (*)[2]>(smem + NS * STAGE);

  // The first wo_slots workgroups convert W_O for the output projection (a
  // multiple of 8, so the XCD of every later workgroup is unchanged), the
  // next early_slots evaluate the early causal rows.
  if ((int)blockIdx.x < a.wo_slots) {
    static_assert(NS * STAGE >= kTransposeTile * (kTransposeTile + 8) * 2, "tile fits the stages");
    if ((int)blockIdx.x < transpose_tiles(a.wo))
      transpose_tile64(a.wo, (int)blockIdx.x,
                       reinterpret_cast<uint16_t(*)[kTransposeTile + 8]>(smem));
    return;
  }
  const int bid = (int)blockIdx.x - a.wo_slots;
  if (bid < early_slots) {
    static_assert(NS * STAGE >= 2 * 64 * DK * 4, "early-row staging fits the stages");
    if ((long long)bid < early_blocks(early, er_rows<DK>()))
      early_rows_block<DK, NWAVES>(early, bid, smem);
    return;
  }
  // wave index in a scalar register: the query rows of the wave, the DMA LDS
  // bases and the causal tests on them stay scalar
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, lh = lane >> 5;

  const int nqb = (a.T_q + BLOCK_M - 1) / BLOCK_M;
  int b, head, qblk;
  map_block<HAS_MASK>(a, bid - early_slots, nqb, b, head, qblk);
  const int bh = b * a.h + head;
  // Key/value set of this query head: consecutive heads share one set, and
  // their workgroups are consecutive in the XCD mappings above, so a set's K
  // and V are read by one XCD; what its L2 cannot hold of a group's K and V
  // is refetched from the Infinity Cache.
  const int kvh = b * a.h_kv + head / (a.h / a.h_kv);

  const uint16_t* Qg = a.q + (size_t)bh * a.Tqp * DK;
  const uint16_t* Kg = a.k + (size_t)kvh * a.Tkp * DK;
  const uint16_t* Vg = a.vt + (size_t)kvh * DK * a.Tkp;
  const int qw0 = qblk * BLOCK_M + wave * 32 * NQ;

  int kv_end = a.T_k;
  if (HAS_MASK) kv_end = min(kv_end, a.kend[b]);
  if (a.causal) kv_end = min(kv_end, qblk * BLOCK_M + BLOCK_M);
  const int ntiles = kv_end > 0 ? (kv_end + BLOCK_N - 1) / BLOCK_N : 0;
  if (a.prio_maxt > 0) {
    // the launch is bound by its longest causal blocks: their waves issue
    // first (priority 2 from two thirds of the longest, 1 from a third)
    const int pr = (3 * ntiles) / a.prio_maxt;
    if (pr >= 2) __builtin_amdgcn_s_setprio(2);
    else if (pr >= 1) __builtin_amdgcn_s_setprio(1);
  }
  const uint32_t* mbits_g = HAS_MASK ? a.mbits + (size_t)b * a.mbits_ld * 2 : nullptr;

  // Issue the DMA loads of key tile `tile` into LDS stage `stage`. Lane
  // chunk p of each wave-wide instruction lands at byte 16*p of the wave's
  // contiguous 1 KiB window; the lane fetches the global chunk that the
  // swizzled layout places there. Successive instructions of a tile move 32
  // (K, d_k = 64; V) or 16 (K, d_k = 128) rows on, which leaves the swizzle
  // unchanged, so one byte offset per lane serves all of them: each copy is
  // a buffer load over the key/value set's K (or V^T) block with that lane
  // offset and a scalar offset for the tile and the copy (no vector address
  // arithmetic; the host keeps a block below 2 GiB).
  static_assert((NT / KCH) % 16 == 0 && (NT / 8) % 16 == 0, "swizzle period");
  const int krow0 = tid / KCH, vrow0 = tid / 8;
  const uint32_t koff = (uint32_t)(krow0 * DK + swz<KCH>(krow0, tid % KCH) * 8) * 2u;
  const uint32_t voff = (uint32_t)(vrow0 * a.Tkp + swz<8>(vrow0, tid % 8) * 8) * 2u;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(Kg, (uint32_t)a.Tkp * DK * 2);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(Vg, (uint32_t)DK * a.Tkp * 2);
  auto issue = [&](int tile, int stage) __attribute__((always_inline)) {
    const int k0 = tile * BLOCK_N;
    uint8_t* kst = smem + stage * STAGE;
    uint8_t* vst = kst + K_BYTES;
#pragma unroll
    for (int i = 0; i < K_LPT; ++i)
      lds_dma16_buf(rk, koff, (uint32_t)(k0 * DK * 2 + i * (NT / KCH) * DK * 2),
                    kst + (i * NT + wave * 64) * 16);
#pragma unroll
    for (int i = 0; i < V_LPT; ++i)
      lds_dma16_buf(rv, voff, (uint32_t)(k0 * 2 + i * (NT / 8) * a.Tkp * 2),
                    vst + (i * NT + wave * 64) * 16);
    if (HAS_MASK) {
      // The tile's two mask dwords; every wave writes the same bytes.
      if (lane < 2)
        lds_dma4(mbits_g + tile * 2 + lane, &mask_s[stage][0]);
    }
  };

  // Q tile in registers (B operand of S^T = K . Q^T); rows past T_q are zero.
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
  float base[NQ];
  f32x4_t lacc[NQ];
  // Row sums by MFMA. Fed as the B operand of a 16x16x32 product, the P^T
  // fragment of lane l becomes column l % 16, k-group l / 16: lanes n and
  // n+32 carry query n, lanes n+16 and n+48 query n+16. The A operand is ones
  // at row 0 for k-groups 0 and 2 and at row 1 for k-groups 1 and 3, zero
  // elsewhere (the k map is the same for A and B), so D[0][n] accumulates the
  // row sum of query n and D[1][n] that of query n+16: lane n, elements 0, 1.
  const bool selr = ((lane & 15) == 0 && ((lane >> 4) & 1) == 0) ||
                    ((lane & 15) == 1 && ((lane >> 4) & 1) == 1);
  const uint32_t selw = selr ? 0x3c003c00u : 0u;
  const u32x4 sel = u32x4{selw, selw, selw, selw};
  bool seen[NQ];   // has this lane's query met an unmasked key yet
  bool moved[NQ];  // wave-uniform: has any lane's reference left 0
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    base[qi] = 0.0f;
    seen[qi] = false;
    moved[qi] = false;
    lacc[qi] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qi][dt][r] = 0.0f;
  }

#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < ntiles) issue(t, t);

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * BLOCK_N;
    const int stage = it % NS;
    // Tile `it` is complete once at most the loads of the younger tiles
    // already issued (up to NS-2 of them) are outstanding.
    const int younger = min(NS - 2, ntiles - 1 - it);
    if (younger >= 2) wait_vmcnt<2 * LPT>();
    else if (younger == 1) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();   // every wave's part of tile `it` has landed

    const uint8_t* Ks = smem + stage * STAGE;
    const uint8_t* Vs = Ks + K_BYTES;
    const bool tail = k0 + BLOCK_N > a.T_k;
    if (tail) {
      // Keys >= T_k of the last tile hold no data: clear their V^T columns
      // (their weights are exactly 0, and 0 * garbage could be NaN). Chunk c
      // holds keys 16*(c/2) + 4*(c%2) + {0..3, 8..11}.
      uint8_t* vw = smem + stage * STAGE + K_BYTES;
      for (int p = tid; p < DK * 8; p += NT) {
        const int row = p / 8, c = p % 8;
        u32x4* chunk = reinterpret_cast<u32x4*>(vw + (row * 8 + swz<8>(row, c)) * 16);
        const u32x4 v = *chunk;
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // elements 2e and 2e+1 of the chunk
          const int key = k0 + 16 * (c >> 1) + 4 * (c & 1) + (2 * e & 3) + 8 * (e >> 1);
          if (key >= a.T_k) w[e] = 0u;
          else if (key + 1 >= a.T_k) w[e] &= 0xffffu;
        }
        *chunk = u32x4{w[0], w[1], w[2], w[3]};
      }
      wait_lgkmcnt0();
      __builtin_amdgcn_s_barrier();
    }
    // The tile's padding-mask bits; every lane reads the same two words, so
    // whether any key of the tile is masked is a wave-uniform (scalar) test.
    uint64_t bits = 0;
    bool mbits = false;
    if (HAS_MASK) {
      const uint32_t lo = mask_s[stage][0], hi = mask_s[stage][1];
      mbits = __builtin_amdgcn_readfirstlane(lo | hi) != 0u;
      bits = (((uint64_t)hi << 32) | lo) >> (4 * lh);
    }

    // Phase 1: S'^T = K . Q^T - base for every live query tile. All K
    // fragments of the tile are read before the first MFMA (one LDS latency
    // per tile instead of one per MFMA), and all V^T fragments right after
    // the MFMAs, so they arrive while the softmax runs.
    u32x4 kf[2][KSTEPS];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int row = kh * 32 + lq;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        kf[kh][ks] = *reinterpret_cast<const u32x4*>(
            Ks + (row * KCH + swz<KCH>(row, 2 * ks + lh)) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t s[NQ][2];
    bool live[NQ];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int q_lo = qw0 + qi * 32;
      live[qi] = !(a.causal && k0 > q_lo + 31);
      if (!live[qi]) continue;
      if (moved[qi]) {
        const float init = -base[qi];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qi][kh][r] = init;
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks)
            s[qi][kh] = mfma32x32x16<F16>(kf[kh][ks], qreg[qi][ks], s[qi][kh]);
        }
      } else {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          s[qi][kh] = mfma32x32x16<F16>(kf[kh][0], qreg[qi][0], f32x16_t{});
#pragma unroll
          for (int ks = 1; ks < KSTEPS; ++ks)
            s[qi][kh] = mfma32x32x16<F16>(kf[kh][ks], qreg[qi][ks], s[qi][kh]);
        }
      }
    }
    // (The V^T reads stay behind the score MFMAs: they are part of the
    // distance between those MFMAs and the row maximum below.)
    __builtin_amdgcn_sched_barrier(0);
    u32x4 vf[DT][4];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int row = dt * 32 + lq;
      const uint8_t* vrow = Vs + row * 128;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        vf[dt][c] = *reinterpret_cast<const u32x4*>(vrow + swz<8>(row, 2 * c + lh) * 16);
    }
    // The stage read in the previous iteration is free again (every wave
    // passed the barrier above). Its refill goes out after this tile's
    // fragment reads and score MFMAs, which then start sooner after the
    // barrier.
    if (it + NS - 1 < ntiles) issue(it + NS - 1, (it + NS - 1) % NS);
    __builtin_amdgcn_sched_barrier(0);

    // Phase 2 (per query tile): mask, lazy reference update, P = exp2(S'),
    // then O^T += V^T . P^T.
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      if (!live[qi]) continue;
      const int q_lo = qw0 + qi * 32;
      // Key of accumulator element (kh, r): k0 + kh*32 + 8*(r/4) + 4*lh + r%4.
      const bool diag = a.causal && (k0 + BLOCK_N - 1 > q_lo);
      // Element rel (key k0 + 4 lh + rel) lies past the query (causal:
      // rel > q - k0 - 4 lh) or past T_k (rel >= T_k - k0 - 4 lh) iff
      // rel > thr; the padding mask adds its own bits where the tile has any.
      const int kmax = a.T_k - k0 - 4 * lh;
      const int thr = a.causal ? min(q_lo + lq - k0 - 4 * lh, kmax - 1) : kmax - 1;
      if constexpr (HAS_MASK) {
        if (diag || tail || mbits) {
          // one bit per element: the padding mask's, or above thr
          const int sh = max(thr + 1, 0);
          const uint64_t ign = bits | (sh >= 64 ? 0ull : (~0ull << sh));
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rel = kh * 32 + 8 * (r >> 2) + (r & 3);
              if ((ign >> rel) & 1ull) s[qi][kh][r] = -INFINITY;
            }
        }
      } else if (diag || tail) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = kh * 32 + 8 * (r >> 2) + (r & 3);
            if (rel > thr) s[qi][kh][r] = -INFINITY;
          }
      }

      // Row maximum: two chains of three-input maxima over the 32 scores.
      float m2[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x16_t& sv = s[qi][g];
        float m = vmax3(sv[0], sv[1], sv[2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) m = vmax3(m, sv[r], sv[r + 1]);
        m2[g] = vmax2(m, sv[15]);
      }
      float mx = pair32_max(vmax2(m2[0], m2[1]));
      const bool first = !seen[qi] && mx != -INFINITY;
      const float shift = first ? ((mx >= 0.0f && mx <= 8.0f) ? 0.0f : mx)
                                : (mx > 8.0f ? mx : 0.0f);
      if (__ballot(shift != 0.0f)) {
        const float alpha = seen[qi] ? __builtin_amdgcn_exp2f(-shift) : 1.0f;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qi][kh][r] -= shift;
        // lane n < 16 holds the sums of queries n and n + 16
        const float ahi = __shfl(alpha, (lane & 15) | 16);
        lacc[qi][0] *= alpha;
        lacc[qi][1] *= ahi;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qi][dt][r] *= alpha;
        base[qi] += shift;
        moved[qi] = true;
      }
      seen[qi] = seen[qi] || first;

      // P = exp2(S') rounded to fp16: the B operand of P . V and of the row sum.
      u32x4 pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(s[qi][c >> 1][(c & 1) * 8 + e]);
        pf[c] = u32x4{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]),
                      pack_f16x2(p[4], p[5]), pack_f16x2(p[6], p[7])};
      }

      // P^T fragment c covers keys c*16 + {4*lh + 0..3, 8 + 4*lh + 0..3}; V^T
      // row d supplies the same keys as its chunk 2c + lh.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[qi][dt] = mfma32x32x16<F16>(vf[dt][c], pf[c], o[qi][dt]);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        lacc[qi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, sel),
                                                          __builtin_bit_cast(half8_t, pf[c]),
                                                          lacc[qi], 0, 0, 0);
    }
  }

  // O = acc / l (times the head's gate under gated attention); head `head`
// occupies columns [head*DK, (head+1)*DK) of (B, T_q, D).
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const float l0 = __shfl(lacc[qi][0], lq & 15), l1 = __shfl(lacc[qi][1], lq & 15);
    const float lt = lq < 16 ? l0 : l1;
    float inv = 1.0f / lt;
    const int row = qw0 + qi * 32 + lq;
    if (row < a.T_q) {
      // gated attention: the head's output row times its gate
      if (a.gate) inv *= gate_sigmoid(a.gate[((size_t)b * a.T_q + row) * a.h + head]);
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


// Query tiles (of 32 rows) per wave and pipeline depth per head size.
#ifndef MHA_ATTN_NQ64
#define MHA_ATTN_NQ64 1
#endif
#ifndef MHA_ATTN_NS64
#define MHA_ATTN_NS64 3
#endif
#ifndef MHA_ATTN_NS128
#define MHA_ATTN_NS128 2
#endif
constexpr int nq_for(int d_k) { return d_k == 64 ? MHA_ATTN_NQ64 : 1; }

template <int DK, int NS>
hipError_t launch_dk(const AttnF16Args& a, int total, const AttnF32Args& e, int extra,
                     hipStream_t s) {
  const unsigned grid = (unsigned)(a.wo_slots + extra + total);
  if (a.mbits)
    hipLaunchKernelGGL((attn_f16_kernel<DK, nq_for(DK), NS, true>), dim3(grid), dim3(NT), 0, s, a,
                       e, extra);
  else
    hipLaunchKernelGGL((attn_f16_kernel<DK, nq_for(DK), NS, false>), dim3(grid), dim3(NT), 0, s,
                       a, e, extra);
  return hipGetLastError();
}

}  // namespace

int attn_f16_block_m(int d_k) { return NWAVES * 32 * nq_for(d_k); }

int attn_mask_tiles(int T_k) { return (T_k + BLOCK_N - 1) / BLOCK_N; }

hipError_t launch_attn_f16(const AttnF16Args& a, int d_k, const AttnF32Args* early,
                           hipStream_t s) {
  if (a.h_kv < 1 || a.h % a.h_kv != 0) return hipErrorInvalidValue;
  const int bm = attn_f16_block_m(d_k);
  // early rows per workgroup
  const int er = d_k == 64 ? er_rows<64>() : er_rows<128>();
  AttnF32Args e{};
  int extra = 0;
  if (early) {
    // rows <= T_k <= 64 (the early rows of causal sequences)
    if (early->T_k < 1 || early->T_k > 64 || early->rows > early->T_k || early->group < 1 ||
        early->h % early->group != 0)
      return hipErrorInvalidValue;
    e = *early;
    const long long n = (early_blocks(e, er) + 7) / 8 * 8;
    if (n > 0x7fffffffLL) return hipErrorInvalidValue;
    extra = (int)n;
  }
  if (a.Tqp % bm != 0 || a.Tkp % bm != 0 || a.Tqp < a.T_q || a.Tkp < a.T_k)
    return hipErrorInvalidValue;
  const int total = ((a.T_q + bm - 1) / bm) * a.h * a.B;
  // Causal, unpadded: query blocks of groups of G units are interleaved
  // longest first. G keeps the group's K and V (4 Tkp d_k bytes per key/value
  // set, shared by h / h_kv heads) within MHA_ATTN_GROUP_BYTES (twice that
  // at d_k = 128, whose two workgroups per CU leave each XCD fewer units in
  // flight: at D = 4096, T = 8192 G = 4 instead of 2 took the attention from
  // 0.541 to 0.535 ms), at most 16 and at most the units one XCD runs.
  AttnF16Args ag = a;
  ag.group_units = 1;
  if (a.causal && !a.mbits) {
    const long long unit_kv = 4LL * a.Tkp * d_k / (a.h / a.h_kv);
    const long long per_xcd = (long long)a.h * a.B / 8;
    const long long gbytes = d_k == 128 ? 2 * MHA_ATTN_GROUP_BYTES : MHA_ATTN_GROUP_BYTES;
    while (ag.group_units < 16 && 2LL * ag.group_units * unit_kv <= gbytes &&
           2LL * ag.group_units <= per_xcd)
      ag.group_units *= 2;
  }
  // Causal, unpadded: when the average work per resident workgroup is less
  // than 1.5 times the longest block's key tiles (short sequences, e.g. T =
  // 1024 with 8 query blocks per head), that block's chain of tiles bounds
  // the launch and its waves get issue priority; at T = 4096 (176 tiles per
  // slot against 64) priority only cost time.
  ag.prio_maxt = 0;
  if (a.causal && !a.mbits) {
    // block j < nqb - 1 of a head walks (j + 1) bm / BLOCK_N key tiles (bm is
    // a multiple of BLOCK_N), the last one all maxt of them
    static_assert(BLOCK_N == 64, "tile count below");
    const long long maxt = (a.T_k + BLOCK_N - 1) / BLOCK_N;
    const long long nqb = (a.T_q + bm - 1) / bm, per = bm / BLOCK_N;
    const long long tiles = (per * (nqb - 1) * nqb / 2 + maxt) * a.h * a.B;
    const long long slots = 256LL * (d_k == 128 ? 2 : 3);
    if (2 * tiles < 3 * maxt * slots) ag.prio_maxt = (int)maxt;
  }
  ag.wo_slots = 0;
  if (a.wo.W) {
    if (a.wo.K < 1 || a.wo.N < 1 || a.wo.K % 8 != 0 || a.wo.N % 8 != 0 || !a.wo.WT)
      return hipErrorInvalidValue;
    ag.wo_slots = (transpose_tiles(a.wo) + 7) / 8 * 8;
  }
  if ((long long)total + extra + ag.wo_slots > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d_k == 64) return launch_dk<64, MHA_ATTN_NS64>(ag, total, e, extra, s);
  if (d_k == 128) return launch_dk<128, MHA_ATTN_NS128>(ag, total, e, extra, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
