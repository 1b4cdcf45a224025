/*
 * mha.h -- C ABI of the MI355X (gfx950) multi-head attention forward pass.
 *
 * What is computed (fused projection, head split, scaled scores with an
 * optional causal or key-padding mask, row softmax, weighted sum, head concat,
 * output projection):
 *
 *   itwiki "멀티 헤드 어텐션", section 수식:
 *     Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V,
 *     MultiHead = Concat(head_1, ..., head_h) W^O, d_k = d_v = d_model / h.
 *   same page, section 텐서 모양으로 본 계산: the three D x D projections are
 *     one D x 3D matrix; a head is a column slice of its output.
 *   iamjaehka13.blog "[Deep Learning 5] Attention의 내부 계산", §9 (causal mask:
 *     key j > query i gets -inf, so its weight is exactly 0), §10 (row
 *     softmax), §13 (O = A V), §18 (concat, one d_model x d_model W_O),
 *     §19 (cross-attention: Q from the target, K and V from the source).
 *   molayo1419.me "MHA란 무엇인가?", trap 2 (key_padding_mask: nonzero/True
 *     means IGNORE the key) and trap 3 (every key ignored -> 0/0 -> NaN).
 *   itwiki "멀티 헤드 어텐션", section 추론 비용과 변형 (variants table):
 *     grouped key/value heads -- h query heads share n_g key/value sets
 *     (GQA; n_g = 1 is MQA, n_g = h plain multi-head attention).
 *
 * Conventions:
 *   - Batch-first only: every activation is (B, T, D) row-major.
 *   - Weights multiply from the right, y = x . W + b. W_QKV is (D, N_qkv)
 *     row-major, N_qkv = D + 2 * n_g * d_k (= 3D when n_g = h), with column
 *     blocks [Q (D wide) | K (n_g*d_k) | V (n_g*d_k)]; query head i owns
 *     columns [i*d_k, (i+1)*d_k) of the Q block, key/value set g owns
 *     columns [g*d_k, (g+1)*d_k) of the K and of the V block, and query head
 *     i reads set i / (h / n_g) (consecutive query heads form a group).
 *     W_O is (D, D) row-major. (torch.nn.Linear / nn.MultiheadAttention
 *     store the transpose.)
 *   - Cross-attention (x_kv != NULL): Q = x_q W_QKV[:, 0:D] + b_QKV[0:D],
 *     [K | V] = x_kv W_QKV[:, D:N_qkv] + b_QKV[D:N_qkv].
 *   - KEY PADDING MASK: NONZERO = THIS KEY IS IGNORED (nn.MultiheadAttention's
 *     key_padding_mask convention, NOT the SDPA boolean attn_mask convention).
 *   - causal = 1 masks keys j > i (requires T_q == T_k). It is a real mask,
 *     not a hint that some other mask is causal.
 *   - A query row whose keys are all masked yields NaN in that row of the
 *     attention output, hence in that row of y.
 *   - dtype MHA_F32: every input, weight and bias is fp32 and the path
 *     computes in fp32. dtype MHA_BF16: inputs, weights and biases are bf16;
 *     products accumulate in fp32 and y is always fp32.
 *
 * Memory and execution:
 *   - Every data pointer is a DEVICE pointer on the current HIP device and
 *     must be 16-byte aligned. The caller owns all buffers, including the
 *     workspace; the library allocates no device memory.
 *   - mha_forward enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns without waiting. Argument errors are
 *     returned before anything is enqueued; launch failures return
 *     MHA_ERR_HIP; faults during execution surface at the next
 *     synchronisation, as with any HIP call.
 *   - A handle is immutable after mha_create, except for the profiling state
 *     below. Calls on one handle may run concurrently only if their
 *     workspaces differ and no profiling is active.
 *
 * Supported on the GPU: d_k = D / h in {64, 128}, D a multiple of 128,
 * n_g dividing h, B, T_q, T_k >= 1. fp16 range (bf16 path, which holds W_O
 * and the intermediates in fp16): every W_O entry, every projected Q, K, V
 * value and every attention output must stay below 65504 in magnitude; a
 * larger one becomes +-inf and propagates into y without an error status
 * (the fp16_overflow option of mha_forward_ex reports it on the device).
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mha_handle* mha_handle_t;

typedef enum { MHA_F32 = 0, MHA_BF16 = 1 } mha_dtype_t;

typedef enum {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = 1, /* bad sizes, NULL/misaligned pointers, D % h != 0, causal with T_q != T_k */
  MHA_ERR_UNSUPPORTED = 2, /* valid MHA, but outside what the kernels handle (d_k, D % 128) */
  MHA_ERR_WORKSPACE = 3,   /* workspace smaller than mha_workspace_size() */
  MHA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} mha_status_t;

/* Create a handle for d_model = D, h heads and the given dtype (host only,
 * no device work). D % h != 0 -> MHA_ERR_INVALID_ARG (embed_dim must be
 * divisible by num_heads); d_k not in {64, 128} or D % 128 != 0 ->
 * MHA_ERR_UNSUPPORTED. On error *out is set to NULL. */
mha_status_t mha_create(mha_handle_t* out, int d_model, int num_heads, mha_dtype_t dtype);

/* As mha_create, with num_kv_heads = n_g key/value sets shared by groups of
 * num_heads / n_g consecutive query heads (itwiki "멀티 헤드 어텐션",
 * 추론 비용과 변형: GQA, and MQA for n_g = 1). W_QKV and b_QKV are then
 * D + 2 * n_g * d_k wide. num_kv_heads < 1 or not dividing num_heads ->
 * MHA_ERR_INVALID_ARG. mha_create(.., h, ..) equals num_kv_heads = h. */
mha_status_t mha_create_grouped(mha_handle_t* out, int d_model, int num_heads, int num_kv_heads,
                                mha_dtype_t dtype);

/* Bytes of device workspace mha_forward needs for these sizes (0 if the
 * handle or sizes are invalid). Pass T_k = T_q for self-attention. */
size_t mha_workspace_size(mha_handle_t handle, int B, int T_q, int T_k);

/* One forward pass: y = MultiHead(x_q, x_kv) as described above.
 *   x_q   (B, T_q, D)  dtype   queries (and keys/values if x_kv == NULL)
 *   x_kv  (B, T_k, D)  dtype   keys/values source, or NULL for self-attention
 *                              (then T_k must equal T_q)
 *   w_qkv (D, N_qkv)   dtype   row-major, y = x . W; N_qkv = D + 2 n_g d_k
 *   b_qkv (N_qkv)      dtype   or NULL (zero bias)
 *   w_o   (D, D)       dtype   row-major
 *   b_o   (D)          dtype   or NULL (zero bias)
 *   causal             0 or 1
 *   key_padding_mask   (B, T_k) uint8, NONZERO = IGNORE, or NULL
 *   y     (B, T_q, D)  fp32    output, fully overwritten
 *   workspace          device scratch of >= workspace_bytes bytes, contents
 *                      undefined on entry and exit; must not overlap any
 *                      other argument
 *   stream             hipStream_t or NULL
 * Sizes: B, T_q, T_k >= 1; B * max(T_q, T_k) < 2^30 and max(T_q, T_k) <
 * 2^29 - 256 (32-bit row arithmetic); T_k rounded up to a multiple of 256,
 * times d_k, <= 2^30 (a key/value set's K and V blocks are addressed with
 * 32-bit byte offsets: about 16M keys at d_k = 64, 8M at d_k = 128). Other
 * sizes -> MHA_ERR_INVALID_ARG.
 */
mha_status_t mha_forward(mha_handle_t handle,
                         const void* x_q, const void* x_kv,
                         const void* w_qkv, const void* b_qkv,
                         const void* w_o, const void* b_o,
                         int B, int T_q, int T_k, int causal,
                         const unsigned char* key_padding_mask,
                         float* y,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* ---- Generation step against a KV cache ----------------------------------
 * itwiki "멀티 헤드 어텐션", section 추론 비용과 변형 (autoregressive
 * generation keeps earlier tokens' keys and values in a KV cache and reads
 * all of it at every step), iamjaehka13.blog "[Deep Learning 5]", §21.
 *
 * Batch element b holds cache_len[b] earlier tokens; the step takes T_new
 * new tokens at positions cache_len[b] .. cache_len[b] + T_new - 1:
 *   [Q | K | V] = x W_QKV + b_QKV for the new tokens only; new token j
 *   attends to the cached keys 0 .. cache_len[b]-1 and to new tokens 0 .. j
 *   (causal); y = Concat(heads) W_O + b_O.
 * The new tokens' keys and values are written into the caches at rows
 * cache_len[b] .. cache_len[b] + T_new - 1, rounded to bf16 (round to
 * nearest even); the step's own attention uses them unrounded (fp32).
 *
 *   x          (B, T_new, D)          bf16   the new tokens
 *   w_qkv, b_qkv, w_o, b_o                   as mha_forward (b_* may be NULL)
 *   k_cache    (B, n_g, T_max, d_k)   bf16   DEVICE, read rows [0, len),
 *   v_cache    (B, n_g, T_max, d_k)   bf16   written rows [len, len + T_new)
 *   cache_len  (B)                    int32  DEVICE; must satisfy
 *              0 <= cache_len[b] <= T_max - T_new. Not modified (advance it
 *              by T_new after the step). Values outside are clamped into
 *              that range by the kernels (no out-of-bounds access; the
 *              result is then that of the clamped length).
 *   y          (B, T_new, D)          fp32   output, fully overwritten
 *   workspace  >= mha_decode_workspace_size(handle, B, T_new, T_max) bytes
 * Requires a MHA_BF16 handle (MHA_ERR_UNSUPPORTED otherwise), 1 <= T_new <=
 * T_max, B <= 65535; data pointers 16-byte aligned, cache_len 4-byte
 * aligned. Stream, ownership and error behaviour as mha_forward; stage
 * timing records "qkv_proj", "attention" and "out_proj". */
size_t mha_decode_workspace_size(mha_handle_t handle, int B, int T_new, int T_max);
mha_status_t mha_decode(mha_handle_t handle, const void* x,
                        const void* w_qkv, const void* b_qkv,
                        const void* w_o, const void* b_o,
                        int B, int T_new,
                        void* k_cache, void* v_cache, int T_max, const int* cache_len,
                        float* y,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* ---- Output options of the forward pass ----------------------------------
 * residual         1: y = x_q + MultiHead(...) (iamjaehka13.blog "[Deep
 *                  Learning 5]", §14 and the residual row of its §23 table:
 *                  the layer output is added to the query-side input).
 * y_bf16           1: y is stored as bf16 (round to nearest even) instead of
 *                  fp32; MHA_BF16 handles only (MHA_ERR_UNSUPPORTED otherwise).
 * attn_weights     NULL, or a DEVICE buffer, 16-byte aligned, receiving the
 *                  softmax weights as nn.MultiheadAttention returns them
 *                  (molayo1419.me, return values): per head (B, h, T_q, T_k)
 *                  fp32, or with average_weights = 1 their mean over heads
 *                  (B, T_q, T_k). Masked keys get weight 0; a row whose keys
 *                  are all masked is NaN. Inspection output for small
 *                  problems: T_k <= 4096 and B <= 65535, else
 *                  MHA_ERR_UNSUPPORTED. On the bf16 path the weights come
 *                  from the fp16 Q and K of the computation (relative error
 *                  about 1e-3), on the fp32 path from fp32 Q and K. Recorded
 *                  in the "attention" stage of the timing hooks.
 * gate_w, gate_b   gated attention (itwiki "멀티 헤드 어텐션", 추론 비용과
 *                  변형, last paragraph: each head's scaled dot-product
 *                  attention output is multiplied by a sigmoid gate of its
 *                  own). gate_w NULL: no gate. Otherwise a DEVICE (D, h)
 *                  matrix of the handle's dtype, row-major, and gate_b a
 *                  DEVICE (h) vector or NULL (zero), both 16-byte aligned:
 *                  head i's output at query row t of batch b is multiplied
 *                  by 1 / (1 + exp(-g)), g = x_q[b, t, :] . gate_w[:, i] +
 *                  gate_b[i], before the concat and W_O. gate_b without
 *                  gate_w -> MHA_ERR_INVALID_ARG. The attention weights
 *                  output is not gated. Recorded in the "qkv_proj" stage.
 * fp16_overflow    NULL, or a DEVICE int, 4-byte aligned (else
 *                  MHA_ERR_INVALID_ARG), that the kernels set to 1 when a
 *                  value they store in fp16 is not finite: the fp16 copy of
 *                  W_O, or a projected Q (as stored, times log2(e)/sqrt(d_k)),
 *                  K or V value of magnitude 65520 or more (past the fp16
 *                  range) or NaN (a non-finite input). The library never
 *                  clears it: zero it before the calls it should cover. The
 *                  attention output needs no check (each of its values is a
 *                  weighted mean of V values, times a gate in (0, 1)). The
 *                  fp32 path stores nothing in fp16 and never writes it.
 * Zero-initialise the struct (all fields 0 / NULL are the defaults). */
typedef struct {
  int residual;
  int y_bf16;
  float* attn_weights;
  int average_weights;
  const void* gate_w;
  const void* gate_b;
  int* fp16_overflow;
} mha_forward_options;

/* mha_forward with options (opts may be NULL: the defaults, all zero, are
 * exactly mha_forward). y is (B, T_q, D) fp32, or bf16 with opts->y_bf16. */
mha_status_t mha_forward_ex(mha_handle_t handle,
                            const void* x_q, const void* x_kv,
                            const void* w_qkv, const void* b_qkv,
                            const void* w_o, const void* b_o,
                            int B, int T_q, int T_k, int causal,
                            const unsigned char* key_padding_mask,
                            void* y,
                            void* workspace, size_t workspace_bytes,
                            const mha_forward_options* opts,
                            void* stream);

/* ---- Forward pass without caller-provided memory -----------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation. Same computation, arguments and options as
 * mha_forward_ex, without the workspace: the scratch comes from a
 * MHA_NOALLOC_SCRATCH_BYTES array that the library holds in each GPU's
 * memory from the first call on that GPU until the process ends. No device
 * memory is allocated or freed by the call.
 *   - Sizes whose mha_workspace_size() exceeds MHA_NOALLOC_SCRATCH_BYTES are
 *     rejected with MHA_ERR_WORKSPACE before anything is enqueued.
 *   - Every call on one GPU uses that GPU's one array (whatever the handle):
 *     calls that overlap in time on one GPU (different streams, threads or
 *     processes' graphs replayed concurrently) race and give undefined
 *     results. Calls on one stream are ordered and safe.
 *   - The array keeps the last call's contents; nothing in it needs to start
 *     at zero.
 * Errors as mha_forward_ex; a failure to look up the array's device address
 * returns MHA_ERR_HIP. */
#define MHA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mha_status_t mha_forward_noalloc(mha_handle_t handle,
                                 const void* x_q, const void* x_kv,
                                 const void* w_qkv, const void* b_qkv,
                                 const void* w_o, const void* b_o,
                                 int B, int T_q, int T_k, int causal,
                                 const unsigned char* key_padding_mask,
                                 void* y,
                                 const mha_forward_options* opts,
                                 void* stream);

/* Release a handle (NULL is accepted). */
mha_status_t mha_destroy(mha_handle_t handle);

/* Static, human-readable name of a status code. */
const char* mha_status_string(mha_status_t status);

/* Description of the HIP error behind the most recent MHA_ERR_HIP returned
 * on the calling thread ("no error" if there was none). Static storage. */
const char* mha_hip_error_string(void);

/* ---- Per-stage timing (measurement only; no effect on results) ----------
 * mha_profile_begin: subsequent mha_forward calls on this handle record HIP
 * events around each stage, for at most max_calls calls.
 * mha_profile_end: waits for the recorded events, writes the AVERAGE duration
 * in milliseconds of each stage over the recorded calls into
 * stage_ms[0 .. MHA_NUM_STAGES-1] (host array), the number of recorded calls
 * into *n_calls, and stops recording. Stages that did not run read 0. */
#define MHA_NUM_STAGES 5
mha_status_t mha_profile_begin(mha_handle_t handle, int max_calls);
mha_status_t mha_profile_end(mha_handle_t handle, float* stage_ms, int* n_calls);
/* Static name of stage s ("prep", "qkv_proj", "attention", "out_proj",
 * "early_rows"), or NULL. */
const char* mha_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
