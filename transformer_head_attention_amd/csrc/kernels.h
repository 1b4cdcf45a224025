// Internal launch interface between the C ABI (mha_api.cpp) and the kernels.
// Not part of the public ABI; every pointer here is a device pointer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mha {

// Rows of each causal sequence that the bf16 path evaluates a second time in
// fp32 (query rows t < kEarlyRows attend only to keys t' <= t < kEarlyRows).
constexpr int kEarlyRows = 64;

// ---- preparation ---------------------------------------------------------
// WT[n][k] = W[k][n] for a (K x N) bf16 matrix; converted to fp16 if to_f16.
struct TransposeJob {
  const uint16_t* W;
  uint16_t* WT;
  int K, N;
  int to_f16;
  int* overflow;         // with to_f16: set to 1 if a converted value is not finite, or null
};
// Scan of a (B, T_k) padding mask (nonzero = ignore): kend[b] = 1 + last index
// j with mask[b][j] == 0, or 0 if every key is masked; bits[b][tile] (two
// uint32): bit j set if key tile*64+j is masked or >= T_k.
struct MaskScan {
  const uint8_t* mask;   // null: no scan
  int B, T_k;
  int* kend;
  uint32_t* bits;
};
// Element-wise transpose of a small (K x N) bf16 matrix, any N: WT[n][k] = W[k][n].
struct SmallTranspose {
  const uint16_t* W;   // null: nothing to do
  uint16_t* WT;
  int K, N;
};
// The transposes j0 and (if non-null) j1, the small transpose and the mask
// scan, in one launch.
hipError_t launch_prep(const TransposeJob& j0, const TransposeJob* j1, const SmallTranspose& st,
                       const MaskScan& ms, hipStream_t s);
// order[r] = the batch element with the r-th largest kend (ties by index).
constexpr int kMaskOrderMaxB = 1024;
hipError_t launch_mask_order(const int* kend, int B, int* order, hipStream_t s);

// ---- 16-bit MFMA GEMMs (C = A . Bt^T, both operands K-contiguous) -------
// Columns of [Q | K | V]: Q is D wide (h heads), K and V are Dkv = h_kv * d_k
// wide each (h_kv key/value sets); N_qkv = D + 2 Dkv.
struct QkvEpilogue {
  int T;                 // rows of A per batch element (m = b*T + t)
  int Tpad_q;            // padded sequence length of the q buffer
  int Tpad_kv;           // padded sequence length of the k and vt buffers
  int D, h, d_k;
  int h_kv, Dkv;         // key/value sets and the width of the K and V blocks
  int n_base;            // global column (0..N_qkv) of GEMM column 0
  const uint16_t* bias;  // (N_qkv) bf16, or null
  uint16_t* q;           // (B, h, Tpad_q, d_k) fp16 -- columns [0, D)
  uint16_t* k;           // (B, h_kv, Tpad_kv, d_k) fp16 -- columns [D, D + Dkv)
  uint16_t* vt;          // (B, h_kv, d_k, Tpad_kv) fp16 -- columns [D + Dkv, N_qkv),
                         // transposed; position t stored at vt_pos(t) (bits 2 and 3 swapped)
  float* early;          // (B, early_rows, N_qkv) fp32 copy of rows t < early_rows, or null
  int early_rows;
  float q_scale;         // multiplies the fp16 Q (the fp32 early copy is unscaled)
  int* overflow;         // set to 1 if a stored fp16 value is not finite, or null
};
// A: (M x K) bf16; W: column n_base of the (K x N_qkv) bf16 weights, row
// stride ldw (N, ldw multiples of 8, K of 64).
hipError_t launch_gemm_qkv(const uint16_t* A, int M, int K, const uint16_t* W, int ldw, int N,
                           const QkvEpilogue& e, hipStream_t s);
// Where and how the output projection stores Y.
struct OutOptions {
  void* y;                // (M x N) fp32, or bf16 (round to nearest even) with y_bf16
  int y_bf16;
  const uint16_t* resid;  // (M x N) bf16 added to Y (the query-side input), or null
};
// A: (M x K) fp16, Bt: (N x K) fp16; Y (M x N) = A . Bt^T + bias (bf16, nullable) [+ resid].
hipError_t launch_gemm_out(const uint16_t* A, int M, int K, const uint16_t* Bt, int N,
                           const uint16_t* bias, const OutOptions& opt, hipStream_t s);

// Early causal rows: Y[b*T_q + t] = O32[b*R + t] . W_O + bias [+ resid] for t < R, from
// fp32 O32 (M = B*R rows x K) and fp16 W_O^T (N x K); N % 32 == 0, K % 64 == 0.
// gate (nullable): gated attention, head i's columns [i*d_k, (i+1)*d_k) of O32
// row (b, t) times 1 / (1 + exp(-gate[(b*T_q + t)*h + i])); d_k % 64 == 0.
hipError_t launch_early_out(const float* O32, int M, int K, const uint16_t* WoT, int N,
                            const uint16_t* bias, const OutOptions& opt, int R, int T_q,
                            const float* gate, int h, int d_k, hipStream_t s);

// ---- fused attention, fp16 operands, fp32 softmax state ------------------
struct AttnF16Args {
  const uint16_t* q;   // (B, h, Tqp, d_k) fp16, pre-multiplied by log2(e)/sqrt(d_k)
  const uint16_t* k;   // (B, h_kv, Tkp, d_k) fp16; query head i reads set i / (h / h_kv)
  const uint16_t* vt;  // (B, h_kv, d_k, Tkp) fp16, positions permuted as the QKV epilogue stores them
  uint16_t* o;         // (B, T_q, D) fp16, head i at columns [i*d_k, (i+1)*d_k)
  const uint32_t* mbits;  // (B, mbits_ld, 2) ignore bitmask per 64-key tile, or null
  int mbits_ld;           // 64-key tiles per batch element (attn_mask_tiles(T_k))
  const int* kend;     // (B) key extent from the mask; read only with mbits
  const int* order;    // (B) batch elements by key extent, longest first; read only
                       // with mbits; null: natural order
  const float* gate;   // (B*T_q, h) gate pre-activations g (row b*T_q + t): head i's output
                       // row t is multiplied by 1 / (1 + exp(-g)); null: no gate
  int B, h, h_kv, T_q, T_k, Tqp, Tkp, D, causal;
  // W_O -> W_O^T in fp16 for the output projection, by extra workgroups at
  // the start of the launch (independent of the attention; W null: none)
  TransposeJob wo;
  int group_units;     // set by launch_attn_f16 (causal query-block interleave)
  int wo_slots;        // set by launch_attn_f16: workgroups of the W_O job
  int prio_maxt;       // set by launch_attn_f16: key tiles of the longest causal block when
                       // those bound the launch (waves of long blocks get issue priority), else 0
};
int attn_f16_block_m(int d_k);   // query rows per workgroup (Tqp, Tkp must be multiples)
int attn_mask_tiles(int T_k);    // 64-key tiles covering T_k
// early (nullable): the fp32 early causal rows (rows <= T_k <= 64), evaluated
// by extra workgroups at the start of the same launch.
struct AttnF32Args;
hipError_t launch_attn_f16(const AttnF16Args& a, int d_k, const AttnF32Args* early,
                           hipStream_t s);

// ---- fp32 path -----------------------------------------------------------
// C[map(m)][n] = sum_k A[m][k] * B[k][n] + bias[n], with
// map(m) = (m / rows_in) * rows_out + m % rows_in (identity when equal).
// B and bias are fp32 or bf16 (b_bf16); bias may be null.
hipError_t launch_gemm_f32(const float* A, int lda, int M, int K, const void* B, int ldb, int N,
                           bool b_bf16, const void* bias, float* C, int ldc, int rows_in,
                           int rows_out, hipStream_t s);

struct AttnF32Args {
  const float* q; long q_bstride; int q_ld;    // q[b*q_bstride + t*q_ld + head*d_k + c]
  // k[b*kv_bstride + t*kv_ld + (head/group)*d_k + c], likewise v
  const float* k; const float* v; long kv_bstride; int kv_ld;
  int group;                                    // query heads per key/value set (>= 1)
  float* o; long o_bstride; int o_ld;
  const uint8_t* mask;                          // (B, mask_ld) nonzero = ignore, or null
  int mask_ld;
  const float* gate; long gate_bstride;         // gate[b*gate_bstride + t*h + head], or null
  int B, h, rows, T_k, causal;                 // rows = query rows evaluated (t = 0..rows-1)
};
hipError_t launch_attn_f32(const AttnF32Args& a, int d_k, hipStream_t s);
// y[i] += x[i] for i < n (fp32).
hipError_t launch_add_residual_f32(float* y, const float* x, size_t n, hipStream_t s);

// ---- gated attention ------------------------------------------------------
// g[m][n] = x[m] . W_G[:, n] + b_G[n] (fp32) for M rows and h gates.
// bf16: x (M x D), wgT = W_G^T (h x D), bias (h) or null; D % 128 == 0.
hipError_t launch_gate_bf16(const uint16_t* x, int M, int D, const uint16_t* wgT,
                            const uint16_t* bias, int h, float* g, hipStream_t s);
// fp32: x (M x D), wg = W_G (D x h) row-major, bias (h) or null.
hipError_t launch_gate_f32(const float* x, int M, int D, const float* wg, const float* bias, int h,
                           float* g, hipStream_t s);

// ---- attention weights (inspection output) --------------------------------
// A[b][head][t][j] (or the mean over heads) = softmax over keys j of
// score_scale * (q . k), masked like the attention (causal, padding, j < T_k).
// q row (b, head, t) at q + b*q_bs + head*q_hs + t*q_ld; k row (b, set, j) at
// k + b*k_bs + set*k_hs + j*k_ld, set = head / group. Elements fp16 (F16) or fp32.
struct WeightsArgs {
  const void* q; long q_bs, q_hs; int q_ld;
  const void* k; long k_bs, k_hs; int k_ld;
  int f16;                     // element type of q and k
  float score_scale;           // multiplies q . k; scores are then in log2 units
  const uint8_t* mask;         // (B, T_k) nonzero = ignore, or null
  int B, h, group, T_q, T_k, d_k, causal, average;
  float* out;                  // (B, h, T_q, T_k) or, with average, (B, T_q, T_k)
};
hipError_t launch_attn_weights(const WeightsArgs& a, hipStream_t s);
constexpr int kWeightsMaxKeys = 4096;

// ---- generation step against a KV cache (bf16 handles) ------------------
struct DecodeArgs {
  int B, T_new, T_max, D, h, h_kv, d_k, Dkv;
  float q_scale;              // log2(e) / sqrt(d_k)
  const uint16_t* b_qkv;      // (D + 2 Dkv) bf16 or null
  const int* cache_len;       // (B) valid cached rows, clamped to [0, T_max - T_new]
  uint16_t* k_cache;          // (B, h_kv, T_max, d_k) bf16; rows [len, len + T_new) written
  uint16_t* v_cache;          // (B, h_kv, T_max, d_k) bf16
  float* q32;                 // (B*T_new, D) pre-scaled Q
  uint16_t* q16;              // (B, h, T_new, d_k) fp16 pre-scaled Q
  float* k32;                 // (B*T_new, Dkv) this step's K
  float* v32;                 // (B*T_new, Dkv) this step's V
  int nqb;                    // 32-row query blocks per key/value set: ceil(h/h_kv * T_new / 32)
  int CW;                     // cached keys per split-K chunk (multiple of 64)
  int nparts;                 // ceil(T_max / CW)
  float* part_m;              // (B, h_kv, nqb, nparts, 32)
  float* part_l;              // same
  float* part_o;              // (B, h_kv, nqb, nparts, 32, d_k)
  float* o32;                 // (B*T_new, D) attention output
};
// [Q|K|V] of the new tokens x (B*T_new x D bf16) with W_QKV (D x N_qkv bf16,
// row-major), routed: q32, q16, k32, v32 and the cache rows. D % 64 == 0.
hipError_t launch_decode_qkv(const DecodeArgs& a, const uint16_t* x, const uint16_t* w_qkv,
                             hipStream_t s);
hipError_t launch_decode_attention(const DecodeArgs& a, hipStream_t s);
// y (M x D fp32) = o32 (M x D fp32) . W_O (D x D bf16) + bias (bf16, nullable).
hipError_t launch_decode_out(const float* o32, int M, int D, const uint16_t* w_o,
                             const uint16_t* bias, float* y, hipStream_t s);

}  // namespace mha
