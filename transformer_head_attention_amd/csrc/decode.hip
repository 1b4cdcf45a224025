// One generation step against a KV cache (itwiki "멀티 헤드 어텐션", section
// 추론 비용과 변형: each step reads every cached key and value, so the step is
// bound by memory bandwidth; iamjaehka13.blog "[Deep Learning 5]", §21: the
// cache keeps the earlier tokens' keys and values so that they are not
// recomputed).
//
// Kernels, in launch order:
//   proj_kernel<QkvRouteEpi>  [Q|K|V] of the new tokens (M = B*T_new rows
//                         times the row-major W_QKV, MFMA with the weight slab
//                         transposed through LDS), bias, and the column
//                         routing: Q (fp32 and fp16, pre-scaled), K and V
//                         (fp32 copies for this step; bf16 rows appended to the
//                         caches).
//   decode_split_kernel   attention of the new query rows over one chunk of
//                         cached keys: partial (max, sum, unnormalised output)
//                         per query row. One wave per (chunk, key/value set,
//                         32-row query block, batch element).
//   decode_merge_kernel   merges the chunks, adds the new tokens' own keys
//                         (causal among the new tokens) in fp32, normalises.
//   proj_kernel<OutStoreEpi>  Y = O . W_O + b_O (fp32 O split into bf16 hi + lo).
#include "device_common.h"
#include "kernels.h"

#ifndef MHA_DECODE_KB64
#define MHA_DECODE_KB64 1
#endif

namespace mha {

namespace {

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
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
// Skinny product of a few rows X (M x K, bf16, or fp32 split into bf16 hi + lo
// for two MFMAs) with a row-major bf16 weight W (K x N), full K per
// workgroup, result handed to an epilogue functor epi(m, n, sum).
// Workgroup: 8 waves on a 32-column slab; the K rows are cut into 64-row
// chunks dealt round-robin to the waves. Each wave issues the loads of all its
// chunks at once, stages each chunk in its own LDS slab (row-major) and
// gathers the MFMA B operand (8 k-values of one column per lane) from there.
// The eight partial 32 x 32 tiles are summed through LDS in a fixed order.
#ifndef MHA_PJ_WAVES
#define MHA_PJ_WAVES 8
#endif
#ifndef MHA_PJ_XCD
#define MHA_PJ_XCD 0
#endif
constexpr int PJ_WAVES = MHA_PJ_WAVES;
constexpr int PJ_NT = PJ_WAVES * 64;
constexpr int PJ_N = 32;
constexpr int PJ_K = 64;
constexpr int PJ_SLAB_LD = PJ_N + 8;   // halves per staged row (80 bytes)
constexpr int PJ_SMEM = PJ_WAVES * PJ_K * PJ_SLAB_LD * 2;   // 40960 B, also the reduction buffer
static_assert(PJ_WAVES * 32 * 33 * 4 <= PJ_SMEM, "reduction buffer");

// Raw X values behind one MFMA A fragment: row m, 8 consecutive k from kx
// (bf16: one 16-byte load; fp32: two). Rows past M read as zero.
// Raw X values behind one MFMA A fragment: row m, 8 consecutive k from kx
// (bf16: one 16-byte load; fp32: two).
template <bool X_F32>
struct XRaw {
  u32x4 v[X_F32 ? 2 : 1];
};

template <bool X_F32>
__device__ __forceinline__ XRaw<X_F32> x_load(const void* Xv, int K, int m, int kx) {
  XRaw<X_F32> r;
  if constexpr (X_F32) {
    const float* xr = static_cast<const float*>(Xv) + (size_t)m * K + kx;
    r.v[0] = *reinterpret_cast<const u32x4*>(xr);
    r.v[1] = *reinterpret_cast<const u32x4*>(xr + 4);
  } else {
    r.v[0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Xv) + (size_t)m * K + kx);
  }
  return r;
}

// A operand(s) from raw X: bf16 as is; fp32 split into bf16 hi and lo parts.
template <bool X_F32>
__device__ __forceinline__ void x_operands(const XRaw<X_F32>& r, u32x4& a, u32x4& alo) {
  if constexpr (X_F32) {
    float xv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = __uint_as_float(r.v[0][i]);
      xv[4 + i] = __uint_as_float(r.v[1][i]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h = pack_bf16x2(xv[2 * e], xv[2 * e + 1]);
      a[e] = h;
      alo[e] = pack_bf16x2(xv[2 * e] - __uint_as_float(h << 16),
                           xv[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
    }
  } else {
    a = r.v[0];
    alo = u32x4{0u, 0u, 0u, 0u};
  }
}

// One launch covers at most 32 rows of X (the host launches one per 32-row
// block). Loads are unconditional with clamped addresses: rows past M and
// columns past N only feed outputs that are never stored; chunks past the
// end of K are skipped as a whole (uniform per wave).
template <bool X_F32, int CPW, typename Epi>
__global__ void __launch_bounds__(PJ_NT)
proj_kernel(const void* __restrict__ Xv, int M, int K, const uint16_t* __restrict__ W, int N,
            Epi epi) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PJ_SMEM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, kg = lane >> 5;
  int slab_id = blockIdx.x;
  if (MHA_PJ_XCD) {   // consecutive slabs (the two halves of each 128-byte row segment) on one XCD
    const int per = gridDim.x / 8;
    if (slab_id < per * 8) slab_id = (slab_id % 8) * per + slab_id / 8;
  }
  const int n0 = slab_id * PJ_N, nchunks = K / PJ_K;
  uint16_t* slab = reinterpret_cast<uint16_t*>(smem) + wave * PJ_K * PJ_SLAB_LD;
  float* red = reinterpret_cast<float*>(smem);
  const int lrow = lane >> 2, lcol = (lane & 3) * 8;   // this lane's 16 bytes of a staged row group
  const int wcol = min(n0 + lcol, N - 8);
  const int xm = min(lq, M - 1);

  f32x16_t acc = {};
  for (int c0 = 0; c0 < nchunks; c0 += PJ_WAVES * CPW) {
    // All of this group's weight and X loads in flight at once.
    u32x4 raw[CPW][4];
    XRaw<X_F32> xf[CPW][PJ_K / 16];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = min(c0 + wave + PJ_WAVES * i, nchunks - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        raw[i][j] = *reinterpret_cast<const u32x4*>(W + (size_t)(c * PJ_K + 16 * j + lrow) * N + wcol);
#pragma unroll
      for (int st = 0; st < PJ_K / 16; ++st)
        xf[i][st] = x_load<X_F32>(Xv, K, xm, c * PJ_K + 16 * st + 8 * kg);
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const bool live = c0 + wave + PJ_WAVES * i < nchunks;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4*>(slab + (16 * j + lrow) * PJ_SLAB_LD + lcol) = raw[i][j];
      __syncthreads();
      if (live) {
#pragma unroll
        for (int s = 0; s < PJ_K / 16; ++s) {
          u32x4 b;
          const int r0 = 16 * s + 8 * kg;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            b[e] = slab[(r0 + 2 * e) * PJ_SLAB_LD + lq] |
                   (uint32_t)slab[(r0 + 2 * e + 1) * PJ_SLAB_LD + lq] << 16;
          u32x4 xa, xlo;
          x_operands<X_F32>(xf[i][s], xa, xlo);
          acc = mfma32x32x16<BF16>(xa, b, acc);
          if constexpr (X_F32) acc = mfma32x32x16<BF16>(xlo, b, acc);
        }
      }
    }
  }
  // Sum the eight waves' tiles in a fixed order; each result to the epilogue.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i)
    red[(wave * 32 + 8 * (i >> 2) + 4 * kg + (i & 3)) * 33 + lq] = acc[i];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 1024 / PJ_NT; ++j) {
    const int idx = tid + PJ_NT * j, r = idx >> 5, cc = idx & 31;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < PJ_WAVES; ++w) v += red[(w * 32 + r) * 33 + cc];
    if (r < M && n0 + cc < N) epi(r, n0 + cc, v);
  }
}

__device__ __forceinline__ int clamp_len(const int* len, int b, int T_max, int T_new) {
  return min(max(len[b], 0), T_max - T_new);
}

// Epilogue of the QKV product: bias, then route by column of [Q | K | V]:
// Q pre-scaled to fp32 and fp16, K and V to fp32 copies and to bf16 cache rows.
struct QkvRouteEpi {
  DecodeArgs a;
  int m0;   // first row of this launch
  __device__ __forceinline__ void operator()(int mr, int n, float v) const {
    const int m = m0 + mr;
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
};

// Epilogue of the output projection: y = sum + b_O.
struct OutStoreEpi {
  const uint16_t* bias;
  float* y;   // first row of this launch
  int N;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    y[(size_t)m * N + n] = v + (bias ? bf16_bits_to_float(bias[n]) : 0.0f);
  }
};

// ---------------------------------------------------------------------------
// Attention of up to 32 query rows (the query heads of one key/value set times
// the new tokens) over cached keys [p*CW, min((p+1)*CW, L)), in tiles of
// 32*KB keys. S^T = K Q^T with the K rows read from the cache straight into
// the MFMA A operand (bf16 -> fp16, exact); each lane owns one query row's
// scores. V is staged transposed in LDS (fp16), in the slot order of the P
// operand. The next tile's K and V loads are issued before the current tile
// is processed. Output: the running max, sum and unnormalised O of every row,
// in log2 units (Q carries log2(e)/sqrt(d_k)).
template <int DK, int KB>
__global__ void __launch_bounds__(64)
decode_split_kernel(DecodeArgs a) {
  constexpr int KSTEP = DK / 16, DB = DK / 32, TK = 32 * KB, PST = TK / 16;
  __shared__ __attribute__((aligned(16))) uint16_t vts[DK][TK + 8];
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
  // Keys past the chunk end read row kend - 1 (in bounds; masked below).
  auto load_tile = [&](int t0, u32x4 (&kr)[KB][KSTEP], u32x4 (&vr)[KB][KSTEP])
      __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = min(t0 + kb * 32 + lq, kend - 1);
#pragma unroll
      for (int s = 0; s < KSTEP; ++s)
        kr[kb][s] = *reinterpret_cast<const u32x4*>(Kc + (size_t)key * DK + 16 * s + 8 * kg);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = min(t0 + kb * 32 + lq, kend - 1);
#pragma unroll
      for (int s = 0; s < KSTEP; ++s)
        vr[kb][s] = *reinterpret_cast<const u32x4*>(Vc + (size_t)key * DK + 16 * s + 8 * kg);
    }
  };

  f32x16_t o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  // One tile: scores, online softmax, V staged transposed, O^T += V^T P^T.
  auto process = [&](int t0, const u32x4 (&kr)[KB][KSTEP], const u32x4 (&vr)[KB][KSTEP])
      __attribute__((always_inline)) {
    f32x16_t sc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sc[kb] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KSTEP; ++s) sc[kb] = mfma32x32x16<F16>(bf16x8_to_f16x8(kr[kb][s]), qf[s], sc[kb]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
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
    u32x4 pf[PST];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
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
    for (int kb = 0; kb < KB; ++kb) {
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
#pragma unroll
    for (int st = 0; st < PST; ++st)
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(&vts[d * 32 + lq][16 * st + 8 * kg]);
        o[d] = mfma32x32x16<F16>(va, pf[st], o[d]);
      }
  };

  // Two register buffers in turn: the loads of tile i+1 are in flight while
  // tile i is processed (no copies between the buffers, which would wait for
  // the loads).
  u32x4 ka[KB][KSTEP], va[KB][KSTEP], kb2[KB][KSTEP], vb2[KB][KSTEP];
  load_tile(kbeg, ka, va);
  for (int t0 = kbeg; t0 < kend; t0 += 2 * TK) {
    load_tile(t0 + TK, kb2, vb2);
    process(t0, ka, va);
    if (t0 + TK >= kend) break;
    load_tile(t0 + 2 * TK, ka, va);
    process(t0 + TK, kb2, vb2);
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
  constexpr int BATCH = 8;      // partial rows read together
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
  for (int p0 = 0; p0 < np; p0 += BATCH) {
    float w[BATCH], ls[BATCH], ov[BATCH][PL];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = min(p0 + u, np - 1);
      const size_t r = (unit0 + p) * 32 + j;
      w[u] = a.part_m[r];
      ls[u] = a.part_l[r];
#pragma unroll
      for (int e = 0; e < PL; ++e) ov[u][e] = a.part_o[r * DK + lane + 64 * e];
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float wt = p0 + u < np ? exp2f(w[u] - mstar) : 0.0f;
      l += ls[u] * wt;
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] += ov[u][e] * wt;
    }
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

// X: rows of one launch (M <= 32).
template <bool X_F32, typename Epi>
hipError_t launch_proj(const void* X, int M, int K, const uint16_t* W, int N, const Epi& epi,
                       hipStream_t s) {
  if (K % PJ_K != 0 || N % 8 != 0 || M < 1 || M > 32) return hipErrorInvalidValue;
  const int cpw = (K / PJ_K + PJ_WAVES - 1) / PJ_WAVES;   // chunks per wave
  dim3 grid((N + PJ_N - 1) / PJ_N);
  if (cpw <= 1)
    hipLaunchKernelGGL((proj_kernel<X_F32, 1, Epi>), grid, dim3(PJ_NT), 0, s, X, M, K, W, N, epi);
  else   // larger K runs in groups of two chunks per wave
    hipLaunchKernelGGL((proj_kernel<X_F32, 2, Epi>), grid, dim3(PJ_NT), 0, s, X, M, K, W, N, epi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_qkv(const DecodeArgs& a, const uint16_t* x, const uint16_t* w_qkv,
                             hipStream_t s) {
  const int M = a.B * a.T_new;
  for (int m0 = 0; m0 < M; m0 += 32) {
    QkvRouteEpi epi{a, m0};
    const hipError_t e = launch_proj<false>(x + (size_t)m0 * a.D, min(32, M - m0), a.D, w_qkv,
                                            a.D + 2 * a.Dkv, epi, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_decode_attention(const DecodeArgs& a, hipStream_t s) {
  if (a.h_kv < 1 || a.h % a.h_kv != 0 || a.CW % 64 != 0 || a.CW < 64) return hipErrorInvalidValue;
  if (a.h > 65535 || (long long)a.h_kv * a.nqb > 65535 || a.B > 65535) return hipErrorInvalidValue;
  dim3 g1(a.nparts, a.h_kv * a.nqb, a.B);
  dim3 g2(a.T_new, a.h, a.B);
  if (a.d_k == 64) {
    hipLaunchKernelGGL((decode_split_kernel<64, MHA_DECODE_KB64>), g1, dim3(64), 0, s, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, g2, dim3(64), 0, s, a);
  } else if (a.d_k == 128) {
    hipLaunchKernelGGL((decode_split_kernel<128, 1>), g1, dim3(64), 0, s, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, g2, dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_out(const float* o32, int M, int D, const uint16_t* w_o,
                             const uint16_t* bias, float* y, hipStream_t s) {
  for (int m0 = 0; m0 < M; m0 += 32) {
    OutStoreEpi epi{bias, y + (size_t)m0 * D, D};
    const hipError_t e = launch_proj<true>(o32 + (size_t)m0 * D, min(32, M - m0), D, w_o, D, epi, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mha
