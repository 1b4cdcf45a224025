// C ABI of the multi-head attention forward pass (declared in include/mha.h).
//
// Host-side code: argument validation, workspace layout and the launch
// sequence (plus the device-resident scratch array of mha_forward_noalloc).
// Every step of the computation runs in the kernels of prep.hip, gemm16.hip,
// attn16.hip and fp32_path.hip.
//
// bf16 inputs (stages):
//   prep       W_QKV -> W_QKV^T (bf16) and W_O -> W_O^T (fp16) so both MFMA
//              operands of the projections are K-contiguous; key extent of
//              the padding mask.
//   qkv_proj   [Q|K|V] = X . W_QKV + b (cross-attention: Q from x_q,
//              K and V from x_kv), fp32 accumulate, head split into fp16
//              Q (B,h,T,d_k), K (B,h_kv,T,d_k) and V^T (B,h_kv,d_k,T), h_kv
//              being the number of key/value sets (h unless grouped).
//   attention  fused masked softmax(QK^T/sqrt(d_k)) V -> O (B,T_q,D) fp16.
//   out_proj   Y = O . W_O + b_O, fp32.
//   early_rows causal only: rows t < 64 of every sequence, which average
//              over at most 64 keys and therefore carry the largest outputs,
//              are recomputed from fp32 copies of their Q/K/V: attention in
//              fp32, then the output projection with the fp32 result split
//              into fp16 hi + lo parts; they overwrite those rows of Y.
// fp32 inputs: qkv_proj, attention and out_proj run the fp32 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "mha.h"   // include/ (on the include path)
#include "kernels.h"

struct mha_handle {
  int D, h, d_k;
  int h_kv;      // key/value sets (h for plain multi-head attention)
  int Dkv;       // h_kv * d_k: width of the K and of the V block of [Q|K|V]
  int Nqkv;      // D + 2 Dkv
  mha_dtype_t dtype;
  // profiling state
  int prof_max = 0;
  int prof_calls = 0;
  std::vector<hipEvent_t> prof_ev;   // prof_max * (MHA_NUM_STAGES + 1)
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int round_up(int x, int a) { return (x + a - 1) / a * a; }

struct Layout {
  // byte offsets into the workspace
  size_t woT = 0, q = 0, k = 0, vt = 0, o = 0, kend = 0, order = 0, mbits = 0, eqkv = 0,
         eo = 0, wgT = 0, gate = 0;
  size_t f_q = 0, f_kv = 0, f_o = 0;
  size_t total = 0;
  int Tqp = 0, Tkp = 0, R = 0;
};

Layout make_layout(const mha_handle* hd, int B, int T_q, int T_k) {
  Layout L;
  const size_t D = (size_t)hd->D;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, kAlign);
    return at;
  };
  if (hd->dtype == MHA_BF16) {
    const int bm = mha::attn_f16_block_m(hd->d_k);
    L.Tqp = round_up(T_q, bm);
    L.Tkp = round_up(T_k, bm);
    L.R = std::min(mha::kEarlyRows, T_q);
    const size_t Dkv = (size_t)hd->Dkv, Nqkv = (size_t)hd->Nqkv;
    L.woT = take(D * D * 2);
    L.q = take((size_t)B * L.Tqp * D * 2);
    L.k = take((size_t)B * L.Tkp * Dkv * 2);
    L.vt = take((size_t)B * L.Tkp * Dkv * 2);
    L.o = take((size_t)B * T_q * D * 2);
    L.kend = take((size_t)B * 4);
    L.order = take((size_t)B * 4);
    L.mbits = take((size_t)B * mha::attn_mask_tiles(T_k) * 8);
    L.eqkv = take((size_t)B * L.R * Nqkv * 4);
    L.eo = take((size_t)B * L.R * D * 4);
    L.wgT = take((size_t)hd->h * D * 2);
    L.gate = take((size_t)B * T_q * hd->h * 4);
  } else {
    // One region: self-attention uses it as a single (B*T, N_qkv) buffer;
    // cross-attention as Q (B*T_q, D) followed by [K|V] (B*T_k, 2 Dkv).
    const size_t Dkv = (size_t)hd->Dkv;
    L.f_q = take((size_t)B * T_q * D * 4 + (size_t)B * T_k * 2 * Dkv * 4);
    L.f_kv = L.f_q + (size_t)B * T_q * D * 4;
    L.f_o = take((size_t)B * T_q * D * 4);
    L.gate = take((size_t)B * T_q * hd->h * 4);
  }
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool sizes_ok(const mha_handle* hd, int B, int T_q, int T_k) {
  if (B < 1 || T_q < 1 || T_k < 1) return false;
  const long long D = hd->D;
  // every row index (B*T) and every element count per buffer must fit the
  // kernels' 32-bit row arithmetic
  const long long rows = (long long)B * std::max(T_q, T_k);
  if (rows > INT_MAX / 2) return false;
  if ((long long)std::max(T_q, T_k) + 256 > INT_MAX / 4) return false;
  // the attention kernel addresses one key/value set's K (T_k x d_k) and V^T
  // (d_k x T_k) blocks, padded to 256 keys, with 32-bit byte offsets
  if (((long long)T_k + 255) / 256 * 256 * hd->d_k * 2 > INT_MAX) return false;
  (void)D;
  return true;
}

// Every argument check of the forward pass except the workspace's.
mha_status_t check_forward_args(const mha_handle* hd, const void* x_q, const void* x_kv,
                                const void* w_qkv, const void* b_qkv, const void* w_o,
                                const void* b_o, int B, int T_q, int T_k, int causal,
                                const void* y, const mha_forward_options* opts) {
  if (!hd) return MHA_ERR_INVALID_ARG;
  if (!x_q || !w_qkv || !w_o || !y) return MHA_ERR_INVALID_ARG;
  const int residual = opts ? opts->residual : 0;
  const int y_bf16 = opts ? opts->y_bf16 : 0;
  const float* weights = opts ? opts->attn_weights : nullptr;
  const int average = opts ? opts->average_weights : 0;
  if ((residual != 0 && residual != 1) || (y_bf16 != 0 && y_bf16 != 1) ||
      (average != 0 && average != 1))
    return MHA_ERR_INVALID_ARG;
  if (weights && !aligned16(weights)) return MHA_ERR_INVALID_ARG;
  const void* gate_w = opts ? opts->gate_w : nullptr;
  const void* gate_b = opts ? opts->gate_b : nullptr;
  if ((gate_b && !gate_w) || (gate_w && !aligned16(gate_w)) || (gate_b && !aligned16(gate_b)))
    return MHA_ERR_INVALID_ARG;
  const int* ovf = opts ? opts->fp16_overflow : nullptr;
  if (ovf && (reinterpret_cast<uintptr_t>(ovf) & 3)) return MHA_ERR_INVALID_ARG;
  if (y_bf16 && hd->dtype != MHA_BF16) return MHA_ERR_UNSUPPORTED;
  if (weights && (T_k > mha::kWeightsMaxKeys || B > 65535)) return MHA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return MHA_ERR_INVALID_ARG;
  if (!x_kv && T_k != T_q) return MHA_ERR_INVALID_ARG;
  if (causal && T_k != T_q) return MHA_ERR_INVALID_ARG;
  if (!sizes_ok(hd, B, T_q, T_k)) return MHA_ERR_INVALID_ARG;
  const void* ptrs[] = {x_q, x_kv, w_qkv, b_qkv, w_o, b_o, y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

thread_local hipError_t g_last_hip_error = hipSuccess;

// Largest d_model whose W_O conversion runs inside the attention launch.
constexpr int kWoInAttentionMaxD = 2048;

// Scratch of mha_forward_noalloc: one copy per GPU, loaded with the code
// object. Host code never passes `scratch` itself (on the host it only names
// the symbol): each device's address is looked up once, with that device
// current, and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[MHA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // indexed by device ordinal

// Device address of the current device's scratch array (looked up on the
// first call on that device), or the HIP error of the lookup.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Workspace of one generation step (bf16 handles).
struct DecodeLayout {
  size_t q32 = 0, q16 = 0, k32 = 0, v32 = 0, o32 = 0, pm = 0, pl = 0, po = 0;
  size_t total = 0;
  int nqb = 1, CW = 64, nparts = 1;
};

bool decode_sizes_ok(int B, int T_new, int T_max) {
  if (B < 1 || B > 65535 || T_new < 1 || T_max < T_new) return false;
  if ((long long)B * T_new > 65535LL * 32) return false;
  if ((long long)T_max + 256 > INT_MAX / 4) return false;
  return true;
}

// Split-K chunk width: about 2048 waves over the cache capacity, at most 32
// chunks per query row (the merge reads every chunk), whole 64-key tiles.
int decode_chunk(long long rows_x_keys, int T_max) {
  long long cw = (rows_x_keys + 2047) / 2048;
  cw = std::max<long long>(cw, ((long long)T_max + 31) / 32);
  cw = std::max(64LL, (cw + 63) / 64 * 64);
  return (int)std::min<long long>(cw, ((long long)T_max + 63) / 64 * 64);
}

DecodeLayout make_decode_layout(const mha_handle* hd, int B, int T_new, int T_max) {
  DecodeLayout L;
  const size_t D = (size_t)hd->D, Dkv = (size_t)hd->Dkv, Nqkv = (size_t)hd->Nqkv;
  const int M = B * T_new;
  const int G = (hd->h / hd->h_kv) * T_new;
  L.nqb = (G + 31) / 32;
  L.CW = decode_chunk((long long)B * hd->h_kv * L.nqb * T_max, T_max);
  L.nparts = (T_max + L.CW - 1) / L.CW;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, kAlign);
    return at;
  };
  (void)Nqkv;
  L.q32 = take((size_t)M * D * 4);
  L.q16 = take((size_t)M * D * 2);
  L.k32 = take((size_t)M * Dkv * 4);
  L.v32 = take((size_t)M * Dkv * 4);
  L.o32 = take((size_t)M * D * 4);
  const size_t rows = (size_t)B * hd->h_kv * L.nqb * L.nparts * 32;
  L.pm = take(rows * 4);
  L.pl = take(rows * 4);
  L.po = take(rows * hd->d_k * 4);
  L.total = off;
  return L;
}

#define MHA_HIP(call)                       \
  do {                                      \
    const hipError_t e_ = (call);           \
    if (e_ != hipSuccess) {                 \
      g_last_hip_error = e_;                \
      return MHA_ERR_HIP;                   \
    }                                       \
  } while (0)

}  // namespace

extern "C" {

mha_status_t mha_create(mha_handle_t* out, int d_model, int num_heads, mha_dtype_t dtype) {
  return mha_create_grouped(out, d_model, num_heads, num_heads, dtype);
}

mha_status_t mha_create_grouped(mha_handle_t* out, int d_model, int num_heads, int num_kv_heads,
                                mha_dtype_t dtype) {
  if (!out) return MHA_ERR_INVALID_ARG;
  *out = nullptr;
  if (d_model <= 0 || num_heads <= 0 || d_model % num_heads != 0) return MHA_ERR_INVALID_ARG;
  if (num_kv_heads < 1 || num_heads % num_kv_heads != 0) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_F32 && dtype != MHA_BF16) return MHA_ERR_INVALID_ARG;
  const int d_k = d_model / num_heads;
  if ((d_k != 64 && d_k != 128) || d_model % 128 != 0) return MHA_ERR_UNSUPPORTED;
  mha_handle* hd = new (std::nothrow) mha_handle();
  if (!hd) return MHA_ERR_INVALID_ARG;
  hd->D = d_model;
  hd->h = num_heads;
  hd->d_k = d_k;
  hd->h_kv = num_kv_heads;
  hd->Dkv = num_kv_heads * d_k;
  hd->Nqkv = d_model + 2 * hd->Dkv;
  hd->dtype = dtype;
  *out = hd;
  return MHA_OK;
}

size_t mha_workspace_size(mha_handle_t hd, int B, int T_q, int T_k) {
  if (!hd || !sizes_ok(hd, B, T_q, T_k)) return 0;
  return make_layout(hd, B, T_q, T_k).total;
}

mha_status_t mha_destroy(mha_handle_t hd) {
  if (!hd) return MHA_OK;
  for (hipEvent_t e : hd->prof_ev) (void)hipEventDestroy(e);
  delete hd;
  return MHA_OK;
}

const char* mha_status_string(mha_status_t s) {
  switch (s) {
    case MHA_OK: return "MHA_OK";
    case MHA_ERR_INVALID_ARG: return "MHA_ERR_INVALID_ARG: invalid argument";
    case MHA_ERR_UNSUPPORTED: return "MHA_ERR_UNSUPPORTED: configuration not supported by the kernels";
    case MHA_ERR_WORKSPACE: return "MHA_ERR_WORKSPACE: workspace too small";
    case MHA_ERR_HIP: return "MHA_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown mha_status_t";
}

const char* mha_hip_error_string(void) { return hipGetErrorString(g_last_hip_error); }

const char* mha_stage_name(int s) {
  static const char* names[MHA_NUM_STAGES] = {"prep", "qkv_proj", "attention", "out_proj",
                                              "early_rows"};
  return (s >= 0 && s < MHA_NUM_STAGES) ? names[s] : nullptr;
}

mha_status_t mha_profile_begin(mha_handle_t hd, int max_calls) {
  if (!hd || max_calls < 1) return MHA_ERR_INVALID_ARG;
  for (hipEvent_t e : hd->prof_ev) (void)hipEventDestroy(e);
  hd->prof_ev.assign((size_t)max_calls * (MHA_NUM_STAGES + 1), nullptr);
  // Timing-only events: no system-scope fence (no cache write-back and
  // invalidation at every stage boundary, which would perturb what is timed).
  for (auto& e : hd->prof_ev) MHA_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
  hd->prof_max = max_calls;
  hd->prof_calls = 0;
  return MHA_OK;
}

mha_status_t mha_profile_end(mha_handle_t hd, float* stage_ms, int* n_calls) {
  if (!hd || !stage_ms || !n_calls) return MHA_ERR_INVALID_ARG;
  for (int s = 0; s < MHA_NUM_STAGES; ++s) stage_ms[s] = 0.0f;
  const int n = hd->prof_calls;
  *n_calls = n;
  mha_status_t st = MHA_OK;
  if (n > 0) {
    const size_t per = MHA_NUM_STAGES + 1;
    if (hipEventSynchronize(hd->prof_ev[(size_t)(n - 1) * per + MHA_NUM_STAGES]) != hipSuccess)
      st = MHA_ERR_HIP;
    for (int c = 0; c < n && st == MHA_OK; ++c)
      for (int s = 0; s < MHA_NUM_STAGES; ++s) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, hd->prof_ev[c * per + s], hd->prof_ev[c * per + s + 1]) !=
            hipSuccess) {
          st = MHA_ERR_HIP;
          break;
        }
        stage_ms[s] += ms / n;
      }
  }
  for (hipEvent_t e : hd->prof_ev) (void)hipEventDestroy(e);
  hd->prof_ev.clear();
  hd->prof_max = 0;
  hd->prof_calls = 0;
  return st;
}

mha_status_t mha_forward(mha_handle_t hd, const void* x_q, const void* x_kv, const void* w_qkv,
                         const void* b_qkv, const void* w_o, const void* b_o, int B, int T_q,
                         int T_k, int causal, const unsigned char* key_padding_mask, float* y,
                         void* workspace, size_t workspace_bytes, void* stream_) {
  return mha_forward_ex(hd, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k, causal,
                        key_padding_mask, y, workspace, workspace_bytes, nullptr, stream_);
}

mha_status_t mha_forward_ex(mha_handle_t hd, const void* x_q, const void* x_kv, const void* w_qkv,
                            const void* b_qkv, const void* w_o, const void* b_o, int B, int T_q,
                            int T_k, int causal, const unsigned char* key_padding_mask, void* y,
                            void* workspace, size_t workspace_bytes,
                            const mha_forward_options* opts, void* stream_) {
  if (!workspace || !aligned16(workspace)) return MHA_ERR_INVALID_ARG;
  const mha_status_t chk = check_forward_args(hd, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k,
                                              causal, y, opts);
  if (chk != MHA_OK) return chk;
  const int residual = opts ? opts->residual : 0;
  const int y_bf16 = opts ? opts->y_bf16 : 0;
  float* weights = opts ? opts->attn_weights : nullptr;
  const int average = opts ? opts->average_weights : 0;
  const void* gate_w = opts ? opts->gate_w : nullptr;
  const void* gate_b = opts ? opts->gate_b : nullptr;
  int* const f16_overflow = opts ? opts->fp16_overflow : nullptr;
  const Layout L = make_layout(hd, B, T_q, T_k);
  if (workspace_bytes < L.total) return MHA_ERR_WORKSPACE;
  // gate pre-activations (B*T_q, h), fp32 (gated attention only)
  float* gpre = gate_w ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.gate) : nullptr;

  hipStream_t s = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  const int D = hd->D, h = hd->h, d_k = hd->d_k, h_kv = hd->h_kv, Dkv = hd->Dkv,
            Nqkv = hd->Nqkv;
  const bool cross = x_kv != nullptr;
  mha::WeightsArgs wa{};
  wa.mask = key_padding_mask;
  wa.B = B;
  wa.h = h;
  wa.group = h / h_kv;
  wa.T_q = T_q;
  wa.T_k = T_k;
  wa.d_k = d_k;
  wa.causal = causal;
  wa.average = average;
  wa.out = weights;

  // stage boundary events (measurement only)
  hipEvent_t* ev = nullptr;
  if (hd->prof_calls < hd->prof_max) {
    ev = &hd->prof_ev[(size_t)hd->prof_calls * (MHA_NUM_STAGES + 1)];
    ++hd->prof_calls;
  }
  auto mark = [&](int i) -> bool {
    if (!ev) return true;
    const hipError_t e = hipEventRecord(ev[i], s);
    if (e != hipSuccess) g_last_hip_error = e;
    return e == hipSuccess;
  };
  // Launch errors are read back with hipGetLastError: clear whatever an
  // earlier, unrelated call left there so it is not reported as ours.
  (void)hipGetLastError();
  if (!mark(0)) return MHA_ERR_HIP;

  if (hd->dtype == MHA_BF16) {
    const uint16_t* xq = static_cast<const uint16_t*>(x_q);
    const uint16_t* xkv = static_cast<const uint16_t*>(x_kv);
    uint16_t* woT = reinterpret_cast<uint16_t*>(ws + L.woT);
    uint16_t* q = reinterpret_cast<uint16_t*>(ws + L.q);
    uint16_t* k = reinterpret_cast<uint16_t*>(ws + L.k);
    uint16_t* vt = reinterpret_cast<uint16_t*>(ws + L.vt);
    uint16_t* o = reinterpret_cast<uint16_t*>(ws + L.o);
    int* kend = reinterpret_cast<int*>(ws + L.kend);
    uint32_t* mbits = reinterpret_cast<uint32_t*>(ws + L.mbits);
    int* order = reinterpret_cast<int*>(ws + L.order);
    // padding masks: batch elements by key extent for the attention launch's
    // longest-first order (natural order past kMaskOrderMaxB)
    const bool ordered = key_padding_mask && B <= mha::kMaskOrderMaxB;
    float* eqkv = reinterpret_cast<float*>(ws + L.eqkv);
    float* eo = reinterpret_cast<float*>(ws + L.eo);
    const uint16_t* bq = static_cast<const uint16_t*>(b_qkv);
    const uint16_t* wq = static_cast<const uint16_t*>(w_qkv);

    // prep: W_O's transposed fp16 copy for the output projection, the gate
    // weights' transpose and the mask scan, in one launch (W_QKV is read as
    // given). With neither mask nor gate and D <= kWoInAttentionMaxD, W_O is
    // converted by the attention launch's first workgroups instead and there
    // is no prep launch: at D = 512 and 1024 that saves the launch; at D =
    // 4096 the 32 MiB conversion slowed the attention by more than it cost
    // here.
    uint16_t* wgT = reinterpret_cast<uint16_t*>(ws + L.wgT);
    const mha::TransposeJob to{static_cast<const uint16_t*>(w_o), woT, D, D, 1, f16_overflow};
    const mha::SmallTranspose tg{static_cast<const uint16_t*>(gate_w), wgT, D, h};
    const mha::MaskScan ms{key_padding_mask, B, T_k, kend, mbits};
    const bool wo_in_attention = !key_padding_mask && !gate_w && D <= kWoInAttentionMaxD;
    if (!wo_in_attention) MHA_HIP(mha::launch_prep(to, nullptr, tg, ms, s));
    if (ordered) MHA_HIP(mha::launch_mask_order(kend, B, order, s));
    if (!mark(1)) return MHA_ERR_HIP;

    // gated attention: gate pre-activations from the query-side input
    if (gate_w)
      MHA_HIP(mha::launch_gate_bf16(xq, B * T_q, D, wgT, static_cast<const uint16_t*>(gate_b), h,
                                    gpre, s));

    // qkv_proj
    mha::QkvEpilogue e{};
    e.Tpad_q = L.Tqp;
    e.Tpad_kv = L.Tkp;
    e.D = D;
    e.h = h;
    e.d_k = d_k;
    e.h_kv = h_kv;
    e.Dkv = Dkv;
    e.bias = bq;
    e.q = q;
    e.k = k;
    e.vt = vt;
    e.early = causal ? eqkv : nullptr;
    e.early_rows = L.R;
    // Q is stored pre-multiplied by log2(e)/sqrt(d_k): the attention kernel
    // then exponentiates scores with exp2 directly.
    e.q_scale = (float)(1.4426950408889634 / std::sqrt((double)d_k));
    e.overflow = f16_overflow;
    if (!cross) {
      e.T = T_q;
      e.n_base = 0;
      MHA_HIP(mha::launch_gemm_qkv(xq, B * T_q, D, wq, Nqkv, Nqkv, e, s));
    } else {
      e.T = T_q;
      e.n_base = 0;
      MHA_HIP(mha::launch_gemm_qkv(xq, B * T_q, D, wq, Nqkv, D, e, s));
      e.T = T_k;
      e.n_base = D;
      MHA_HIP(mha::launch_gemm_qkv(xkv, B * T_k, D, wq + D, Nqkv, 2 * Dkv, e, s));
    }
    if (!mark(2)) return MHA_ERR_HIP;

    // attention
    mha::AttnF16Args a{};
    a.q = q;
    a.k = k;
    a.vt = vt;
    a.o = o;
    a.mbits = key_padding_mask ? mbits : nullptr;
    a.mbits_ld = mha::attn_mask_tiles(T_k);
    a.kend = key_padding_mask ? kend : nullptr;
    a.order = ordered ? order : nullptr;
    a.gate = gpre;
    a.B = B;
    a.h = h;
    a.h_kv = h_kv;
    a.T_q = T_q;
    a.T_k = T_k;
    a.Tqp = L.Tqp;
    a.Tkp = L.Tkp;
    a.D = D;
    a.causal = causal;
    if (wo_in_attention) a.wo = to;
    // Early causal rows, re-evaluated in fp32 by workgroups appended to the
    // attention launch (their output projection follows out_proj).
    mha::AttnF32Args f{};
    if (causal) {
      f.q = eqkv;
      f.k = eqkv + D;
      f.v = eqkv + D + Dkv;
      f.q_ld = f.kv_ld = Nqkv;
      f.q_bstride = f.kv_bstride = (long)L.R * Nqkv;
      f.group = h / h_kv;
      f.o = eo;
      f.o_ld = D;
      f.o_bstride = (long)L.R * D;
      f.mask = key_padding_mask;
      f.mask_ld = T_k;
      f.B = B;
      f.h = h;
      f.rows = L.R;
      f.T_k = L.R;
      f.causal = 1;
    }
    MHA_HIP(mha::launch_attn_f16(a, d_k, causal ? &f : nullptr, s));
    if (weights) {
      wa.q = q;
      wa.q_hs = (long)L.Tqp * d_k;
      wa.q_bs = wa.q_hs * h;
      wa.q_ld = d_k;
      wa.k = k;
      wa.k_hs = (long)L.Tkp * d_k;
      wa.k_bs = wa.k_hs * h_kv;
      wa.k_ld = d_k;
      wa.f16 = 1;
      wa.score_scale = 1.0f;   // Q already carries log2(e)/sqrt(d_k)
      MHA_HIP(mha::launch_attn_weights(wa, s));
    }
    if (!mark(3)) return MHA_ERR_HIP;

    // out_proj
    mha::OutOptions oo{y, y_bf16, residual ? xq : nullptr};
    MHA_HIP(mha::launch_gemm_out(o, B * T_q, D, woT, D, static_cast<const uint16_t*>(b_o), oo, s));
    if (!mark(4)) return MHA_ERR_HIP;

    // early_rows
    if (causal) {
      MHA_HIP(mha::launch_early_out(eo, B * L.R, D, woT, D, static_cast<const uint16_t*>(b_o), oo,
                                    L.R, T_q, gpre, h, d_k, s));
    }
    if (!mark(5)) return MHA_ERR_HIP;
  } else {
    const float* xq = static_cast<const float*>(x_q);
    const float* xkv = static_cast<const float*>(x_kv);
    const float* W = static_cast<const float*>(w_qkv);
    const float* bqkv = static_cast<const float*>(b_qkv);
    float* fq = reinterpret_cast<float*>(ws + L.f_q);
    float* fkv = reinterpret_cast<float*>(ws + L.f_kv);
    float* fo = reinterpret_cast<float*>(ws + L.f_o);
    if (!mark(1)) return MHA_ERR_HIP;

    mha::AttnF32Args f{};
    if (!cross) {
      // one (B*T, N_qkv) product; Q, K, V are column blocks of it
      MHA_HIP(mha::launch_gemm_f32(xq, D, B * T_q, D, W, Nqkv, Nqkv, false, bqkv, fq, Nqkv,
                                   B * T_q, B * T_q, s));
      f.q = fq;
      f.k = fq + D;
      f.v = fq + D + Dkv;
      f.q_ld = f.kv_ld = Nqkv;
      f.q_bstride = f.kv_bstride = (long)T_q * Nqkv;
    } else {
      MHA_HIP(mha::launch_gemm_f32(xq, D, B * T_q, D, W, Nqkv, D, false, bqkv, fq, D, B * T_q,
                                   B * T_q, s));
      MHA_HIP(mha::launch_gemm_f32(xkv, D, B * T_k, D, W + D, Nqkv, 2 * Dkv, false,
                                   bqkv ? bqkv + D : nullptr, fkv, 2 * Dkv, B * T_k, B * T_k, s));
      f.q = fq;
      f.q_ld = D;
      f.q_bstride = (long)T_q * D;
      f.k = fkv;
      f.v = fkv + Dkv;
      f.kv_ld = 2 * Dkv;
      f.kv_bstride = (long)T_k * 2 * Dkv;
    }
    f.group = h / h_kv;
    if (gate_w) {
      MHA_HIP(mha::launch_gate_f32(xq, B * T_q, D, static_cast<const float*>(gate_w),
                                   static_cast<const float*>(gate_b), h, gpre, s));
      f.gate = gpre;
      f.gate_bstride = (long)T_q * h;
    }
    if (!mark(2)) return MHA_ERR_HIP;
    f.o = fo;
    f.o_ld = D;
    f.o_bstride = (long)T_q * D;
    f.mask = key_padding_mask;
    f.mask_ld = T_k;
    f.B = B;
    f.h = h;
    f.rows = T_q;
    f.T_k = T_k;
    f.causal = causal;
    MHA_HIP(mha::launch_attn_f32(f, d_k, s));
    if (weights) {
      wa.q = f.q;
      wa.q_bs = f.q_bstride;
      wa.q_hs = d_k;
      wa.q_ld = f.q_ld;
      wa.k = f.k;
      wa.k_bs = f.kv_bstride;
      wa.k_hs = d_k;
      wa.k_ld = f.kv_ld;
      wa.f16 = 0;
      wa.score_scale = (float)(1.4426950408889634 / std::sqrt((double)d_k));
      MHA_HIP(mha::launch_attn_weights(wa, s));
    }
    if (!mark(3)) return MHA_ERR_HIP;
    float* yf = static_cast<float*>(y);
    MHA_HIP(mha::launch_gemm_f32(fo, D, B * T_q, D, w_o, D, D, false, b_o, yf, D, B * T_q, B * T_q,
                                 s));
    if (residual) MHA_HIP(mha::launch_add_residual_f32(yf, xq, (size_t)B * T_q * D, s));
    if (!mark(4) || !mark(5)) return MHA_ERR_HIP;
  }
  return MHA_OK;
}

mha_status_t mha_forward_noalloc(mha_handle_t hd, const void* x_q, const void* x_kv,
                                 const void* w_qkv, const void* b_qkv, const void* w_o,
                                 const void* b_o, int B, int T_q, int T_k, int causal,
                                 const unsigned char* key_padding_mask, void* y,
                                 const mha_forward_options* opts, void* stream_) {
  const mha_status_t chk = check_forward_args(hd, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k,
                                              causal, y, opts);
  if (chk != MHA_OK) return chk;
  if (make_layout(hd, B, T_q, T_k).total > MHA_NOALLOC_SCRATCH_BYTES) return MHA_ERR_WORKSPACE;
  void* ws = nullptr;
  MHA_HIP(scratch_ptr(&ws));
  return mha_forward_ex(hd, x_q, x_kv, w_qkv, b_qkv, w_o, b_o, B, T_q, T_k, causal,
                        key_padding_mask, y, ws, MHA_NOALLOC_SCRATCH_BYTES, opts, stream_);
}

size_t mha_decode_workspace_size(mha_handle_t hd, int B, int T_new, int T_max) {
  if (!hd || hd->dtype != MHA_BF16 || !decode_sizes_ok(B, T_new, T_max)) return 0;
  return make_decode_layout(hd, B, T_new, T_max).total;
}

mha_status_t mha_decode(mha_handle_t hd, const void* x, const void* w_qkv, const void* b_qkv,
                        const void* w_o, const void* b_o, int B, int T_new, void* k_cache,
                        void* v_cache, int T_max, const int* cache_len, float* y,
                        void* workspace, size_t workspace_bytes, void* stream_) {
  if (!hd) return MHA_ERR_INVALID_ARG;
  if (!x || !w_qkv || !w_o || !k_cache || !v_cache || !cache_len || !y || !workspace)
    return MHA_ERR_INVALID_ARG;
  if (!decode_sizes_ok(B, T_new, T_max)) return MHA_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w_qkv, b_qkv, w_o, b_o, k_cache, v_cache, y, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MHA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(cache_len) & 3u) != 0) return MHA_ERR_INVALID_ARG;
  if (hd->dtype != MHA_BF16) return MHA_ERR_UNSUPPORTED;
  const DecodeLayout L = make_decode_layout(hd, B, T_new, T_max);
  if (workspace_bytes < L.total) return MHA_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  const int D = hd->D, M = B * T_new;
  hipEvent_t* ev = nullptr;
  if (hd->prof_calls < hd->prof_max) {
    ev = &hd->prof_ev[(size_t)hd->prof_calls * (MHA_NUM_STAGES + 1)];
    ++hd->prof_calls;
  }
  auto mark = [&](int i) -> bool {
    if (!ev) return true;
    const hipError_t e = hipEventRecord(ev[i], s);
    if (e != hipSuccess) g_last_hip_error = e;
    return e == hipSuccess;
  };
  (void)hipGetLastError();
  if (!mark(0) || !mark(1)) return MHA_ERR_HIP;

  mha::DecodeArgs a{};
  a.B = B;
  a.T_new = T_new;
  a.T_max = T_max;
  a.D = D;
  a.h = hd->h;
  a.h_kv = hd->h_kv;
  a.d_k = hd->d_k;
  a.Dkv = hd->Dkv;
  a.q_scale = (float)(1.4426950408889634 / std::sqrt((double)hd->d_k));
  a.b_qkv = static_cast<const uint16_t*>(b_qkv);
  a.cache_len = cache_len;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.q32 = reinterpret_cast<float*>(ws + L.q32);
  a.q16 = reinterpret_cast<uint16_t*>(ws + L.q16);
  a.k32 = reinterpret_cast<float*>(ws + L.k32);
  a.v32 = reinterpret_cast<float*>(ws + L.v32);
  a.nqb = L.nqb;
  a.CW = L.CW;
  a.nparts = L.nparts;
  a.part_m = reinterpret_cast<float*>(ws + L.pm);
  a.part_l = reinterpret_cast<float*>(ws + L.pl);
  a.part_o = reinterpret_cast<float*>(ws + L.po);
  a.o32 = reinterpret_cast<float*>(ws + L.o32);

  // qkv_proj
  MHA_HIP(mha::launch_decode_qkv(a, static_cast<const uint16_t*>(x),
                                 static_cast<const uint16_t*>(w_qkv), s));
  if (!mark(2)) return MHA_ERR_HIP;
  // attention
  MHA_HIP(mha::launch_decode_attention(a, s));
  if (!mark(3)) return MHA_ERR_HIP;
  // out_proj
  MHA_HIP(mha::launch_decode_out(a.o32, M, D, static_cast<const uint16_t*>(w_o),
                                 static_cast<const uint16_t*>(b_o), y, s));
  if (!mark(4) || !mark(5)) return MHA_ERR_HIP;
  return MHA_OK;
}

}  // extern "C"
