// Device-side building blocks shared by the gfx950 kernels: 16-bit element
// types, MFMA wrappers and small vector helpers.
//
// MFMA operand/result lane layouts relied on (wave64, gfx950):
//   v_mfma_f32_32x32x16_{f16,bf16}: lane l supplies row (A) / column (B)
//     l % 32 and 8 k-values selected by l / 32; A and B use the same k map.
//     Result: lane l holds column j = l % 32, and for r = 0..15 the row
//     i = 8*(r/4) + 4*(l/32) + (r%4).
//   v_mfma_f32_16x16x4_f32: lane l supplies row (A) / column (B) l % 16 at
//     k = l / 16. Result: lane l holds column l % 16, rows 4*(l/16) + r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
// Plain clang vectors for raw 16/8-byte moves (HIP's uint4 is a struct that
// keeps register arrays of it from being promoted out of scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Tag types for the two 16-bit MFMA input formats.
struct BF16 {};
struct F16 {};

template <typename Tag>
__device__ __forceinline__ f32x16_t mfma32x32x16(const u32x4& a, const u32x4& b, f32x16_t c);

template <>
__device__ __forceinline__ f32x16_t mfma32x32x16<BF16>(const u32x4& a, const u32x4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16_t mfma32x32x16<F16>(const u32x4& a, const u32x4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// Asynchronous global -> LDS copy (global_load_lds): every active lane copies
// BYTES bytes from its own global address; lane L's bytes land at
// lds_base + BYTES * L. lds_base must be the same for the whole wave. Counted
// by vmcnt like any vector load. (Kept out of templates: calling the builtin
// directly in a kernel template left the template's host stub undefined.)
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
// Buffer-addressed copies: a resource over a block of global memory (its
// base in scalar registers) and per-lane and per-copy scalar byte offsets, so
// a copy needs no vector address arithmetic. Resource word 3 selects raw
// 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, voff, soff, 0, 0);
}
// Transposing LDS read of 16-bit values (gfx950). In each group of 16 lanes,
// lane 4 e + q names 8 bytes holding row e, columns 4 q .. 4 q + 3 of a 4 x 16
// block; lane j of the group receives column j, rows 0..3 (row 0 in the low
// 16 bits). Written as assembly: with the builtin form the compiler waits for
// every global->LDS copy in flight before the read (it does not tell the
// copies' targets from the read's address), which would serialise a copy
// pipeline. The caller guarantees the bytes read are not being copied into,
// and waits for the result with lds_tr_wait before using it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Waits for every LDS read in flight and makes the values in v and w depend
// on it, so nothing reading them is scheduled before the wait (and the
// compiler, which cannot see the wait, adds none of its own for them).
template <int N, int M>
__device__ __forceinline__ void lds_tr_wait(u32x4 (&v)[N], u32x4 (&w)[M]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]));
#pragma unroll
  for (int i = 1; i < N; ++i) asm volatile("" : "+v"(v[i]));
#pragma unroll
  for (int i = 0; i < M; ++i) asm volatile("" : "+v"(w[i]));
}
__device__ __forceinline__ void lds_dma4(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma16x16x4f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_float(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t float_to_f16_bits(float x) {
  _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Two fp32 -> packed fp16x2 (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  half2_t h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even (gfx950
// converts in hardware).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float f16_bits_to_float(uint16_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, v));
}

// Load one element of a bias vector stored as bf16 or fp32 bits.
__device__ __forceinline__ float load_bias_bf16(const uint16_t* b, int i) {
  return b ? bf16_bits_to_float(b[i]) : 0.0f;
}

// 1 / (1 + e^-x), the gate of gated attention, with the hardware exp2 and
// reciprocal (each about 1 ulp). e^-x is exp2(-x log2 e): +inf for very
// negative x (rcp(inf) = 0), 0 for very large x (result 1).
__device__ __forceinline__ float gate_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// Maximum of three / two floats. __builtin_elementwise_maximum (IEEE
// maximum: a NaN operand gives NaN) lowers to gfx950's v_maximum3_f32, which
// takes its operands as they are: fmaxf (maxnum) on values the compiler
// cannot prove canonical, such as MFMA results, first canonicalises each
// input with an extra v_max_f32 x, x. Being ordinary compiler-visible
// instructions, these also get the wait states a VALU read of an MFMA result
// needs from the compiler's hazard recogniser.
// The smallest magnitude that fp16 conversion (round to nearest even) turns
// into infinity: halfway between 65504 and 2^16.
constexpr float kF16Overflow = 65520.0f;

// flag (if non-null) := 1 when amax, the largest magnitude a lane converted
// to fp16, is past the fp16 range or NaN. Lanes that find it write the same
// value, with a plain vector store.
__device__ __forceinline__ void flag_f16_overflow(int* flag, float amax) {
  if (flag && !(amax < kF16Overflow)) *flag = 1;
}

__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float vmax2(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap: a VALU
// exchange of the two lane halves, no LDS round trip). Swapping v with itself
// leaves each lane's own value in one result and its partner's in the other.
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return vmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mha
