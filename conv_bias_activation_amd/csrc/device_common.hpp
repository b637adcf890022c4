// device_common.hpp — gfx950 device helpers shared by the biasact kernels:
// element traits, buffer-resource loads/stores (out-of-range reads return 0,
// out-of-range writes are dropped), activation, output casts and the
// 32x32 MFMA step.
//
// Page legend used in comments:
//   [MLR] "CANN pyasc MatmulLeakyRelu 融合算子实战" (lshu.cn/news/76032)
//   [FMR] ops-nn fused_matmul_relu article (mlqm.cn/news/1824)
//   [FCT] multimodal-ops "Fused ConvTanh" article (wmrh.cn/news/81139)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace biasact {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_I32 = 4 };
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_LEAKY = 2, ACT_TANH = 3, ACT_GELU = 4, ACT_SIGMOID = 5 };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;   // LDS destination of direct loads

// Offset used for a masked-off access: beyond every num_records the library
// creates (all tensors are < 2^31 bytes), so the hardware range check turns
// the load into 0 and the store into a no-op.
constexpr uint32_t kOOB = 0x80000000u;

// Element traits.  A "chunk" is 16 bytes of consecutive reduction-index (k)
// values: 16 for int8, 8 for 16-bit inputs, 4 for fp32.  int32 appears only
// as a bias and an output type.
template <int DT> struct Elem;
template <> struct Elem<DT_F32>  { static constexpr int bytes = 4, epc = 4; };
template <> struct Elem<DT_F16>  { static constexpr int bytes = 2, epc = 8; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2, epc = 8; };
template <> struct Elem<DT_I8>   { static constexpr int bytes = 1, epc = 16; };
template <> struct Elem<DT_I32>  { static constexpr int bytes = 4, epc = 4; };

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data format for gfx9-family buffers.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 ld_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t ld_b16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint8_t ld_b8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ void st_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void st_b64(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void st_b32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void st_b16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// ---- scalar conversions --------------------------------------------------

// Exact widening of one stored element to fp32.
template <int DT> __device__ __forceinline__ float widen(uint32_t w);
template <> __device__ __forceinline__ float widen<DT_F32>(uint32_t w) { return __uint_as_float(w); }
// int32 values travel through the float-typed epilogue as their bit pattern
template <> __device__ __forceinline__ float widen<DT_I32>(uint32_t w) { return __uint_as_float(w); }
template <> __device__ __forceinline__ float widen<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}
template <> __device__ __forceinline__ float widen<DT_BF16>(uint32_t w) {
  return __uint_as_float(w << 16);   // bf16 is the upper half of a binary32
}

// Narrowing fp32 -> output element bits, round to nearest even (the hardware
// conversions v_cvt_f16_f32 / v_cvt_pk_bf16_f32 round to nearest even).
template <int DT> __device__ __forceinline__ uint32_t narrow(float v);
template <> __device__ __forceinline__ uint32_t narrow<DT_F32>(float v) { return __float_as_uint(v); }
template <> __device__ __forceinline__ uint32_t narrow<DT_I32>(float v) { return __float_as_uint(v); }
template <> __device__ __forceinline__ uint32_t narrow<DT_F16>(float v) {
  // The opaque copy keeps the compiler from folding a multiply that produced
  // v into a mixed-precision multiply-add rounding straight to fp16: that
  // rounds once instead of twice and turns -0 into +0, so whether it fires
  // would depend on the surrounding kernel.  Every path rounds to fp32 first.
  asm("" : "+v"(v));
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}
template <> __device__ __forceinline__ uint32_t narrow<DT_BF16>(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---- activation ----------------------------------------------------------
// LeakyReLU keeps non-negative values and scales negative ones by alpha
// ([MLR] 概述); ReLU maps non-positive values to +0 ([FMR] host loop); tanh
// is the hyperbolic tangent of [FCT] (K2 chain).

// tanh in fp32.  For |x| >= 0.625 the identity tanh|x| = 1 - 2 / (e^{2|x|} + 1)
// with the hardware base-2 exponential and reciprocal (an overflowing
// exponential gives exactly 1, so large arguments stay finite); below 0.625
// the odd polynomial x * P(x^2) whose coefficients fit_tanh.py derives.
// Relative error below 2e-7 everywhere; the sign comes from x, NaN propagates.
// The activation helpers below turn off implicit multiply-add contraction and
// state every fused multiply-add they use, so each compiles to the same
// instruction sequence in every kernel: the fused epilogue and the two-kernel
// path's act_cast_kernel give bitwise equal results.
__device__ __forceinline__ float tanh_f32(float x) {
#pragma clang fp contract(off)
  const float ax = __builtin_fabsf(x);
  const float e = __builtin_amdgcn_exp2f(ax * 2.885390082f);     // e^{2|x|} = 2^{2|x| / ln 2}
  const float big = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
  const float t = x * x;
  float p = -5.664775148e-03f;
  p = __builtin_fmaf(p, t, 2.059567906e-02f);
  p = __builtin_fmaf(p, t, -5.372267962e-02f);
  p = __builtin_fmaf(p, t, 1.333114952e-01f);
  p = __builtin_fmaf(p, t, -3.333326280e-01f);
  p = __builtin_fmaf(p, t, 1.0f);
  const float r = ax < 0.625f ? ax * p : big;
  return __builtin_copysignf(r, x);
}

// tanh for a result that is next rounded to fp16 or bf16, whose half ulp is
// at least 2^-12 of the value: the identity tanh|x| = 1 - 2 / (e^{2|x|} + 1)
// from |x| >= 2^-6 (its fp32 roundings, about 2^-22 absolute, are then at
// most 2^-16 relative), and below that the first two terms of the series,
// x (1 - x^2 / 3), whose truncation is below 2^-26 relative.  Five fewer
// VALU instructions than tanh_f32; fp32 outputs keep tanh_f32.
__device__ __forceinline__ float tanh_f32_short(float x) {
#pragma clang fp contract(off)
  const float ax = __builtin_fabsf(x);
  const float e = __builtin_amdgcn_exp2f(ax * 2.885390082f);     // e^{2|x|}
  const float big = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
  const float small = ax * __builtin_fmaf(x * x, -0.333333343f, 1.0f);
  return __builtin_copysignf(ax < 0x1p-6f ? small : big, x);
}

// 2^s in fp32, subnormal results included.  The hardware base-2 exponential
// returns 0 for results below the smallest normal (2^-126), which bf16
// outputs would see as an error of up to 2^7 of their subnormal spacing;
// there the exponent is raised by 64 and the result scaled back by an exact
// power of two, whose multiply rounds once onto the subnormal grid.
__device__ __forceinline__ float exp2_f32(float s) {
#pragma clang fp contract(off)
  const bool tiny = s < -126.0f;
  const float r = __builtin_amdgcn_exp2f(tiny ? s + 64.0f : s);
  return tiny ? r * 0x1p-64f : r;
}

// Sigmoid(z) = 1 / (1 + e^-z), evaluated as s(|z|) = 1 / (1 + u) with
// u = e^-|z| in (0, 1] (the hardware base-2 exponential and reciprocal), and
// s(z) = u * s(|z|) = e^z / (1 + e^z) for negative z: nothing overflows, and
// far-negative results that fall below the fp32 normal range keep their
// subnormal value.  Each step is within about an ulp, so the result is
// within a few fp32 ulps of the definition (plus the rounding of the
// exponent's argument, |z| * 2^-24 relative).
__device__ __forceinline__ float sigmoid_f32(float z) {
#pragma clang fp contract(off)
  const float u = exp2_f32(__builtin_fabsf(z) * -1.442695041f);
  const float r = __builtin_amdgcn_rcpf(1.0f + u);
  return z < 0.0f ? u * r : r;
}

// erfc(x) for x >= 0 as t * e^(-x^2 + P(t)), t = 1 / (1 + x/2), P of degree 9:
// the functional form of the Chebyshev-fitted erfc in Numerical Recipes
// (section 6.2), with this project's own least-squares coefficients
// (csrc/fit_erfc.py, which also reports the float32 error: relative
// 4e-7 on [0, 1], 2e-6 on [1, 4], 8e-6 on [4, 9], the last dominated by the
// rounding of the exponent's argument).  erfc(-x) = 2 - erfc(x).
__device__ __forceinline__ float erfc_f32(float x) {
#pragma clang fp contract(off)
  const float ax = __builtin_fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, ax, 1.0f));
  float p = 1.449302137e-01f;
  p = __builtin_fmaf(p, t, -6.808272004e-01f);
  p = __builtin_fmaf(p, t, 1.156733751e+00f);
  p = __builtin_fmaf(p, t, -6.962518692e-01f);
  p = __builtin_fmaf(p, t, -8.028043061e-02f);
  p = __builtin_fmaf(p, t, 1.267586369e-03f);
  p = __builtin_fmaf(p, t, 3.460279852e-02f);
  p = __builtin_fmaf(p, t, 3.866403997e-01f);
  p = __builtin_fmaf(p, t, 9.986327887e-01f);
  p = __builtin_fmaf(p, t, -1.265447974e+00f);
  const float e = __builtin_fmaf(-ax, ax, p);
  // below 2^-126 the product is formed at 2^64 times its size, then scaled
  // back exactly (see exp2_f32): one rounding onto the subnormal grid
  const float s = e * 1.442695041f;
  const bool tiny = s < -126.0f;
  float r = t * __builtin_amdgcn_exp2f(tiny ? s + 64.0f : s);
  r = tiny ? r * 0x1p-64f : r;
  return x < 0.0f ? 2.0f - r : r;
}

// GELU(z) = z * Phi(z), Phi(z) = erfc(-z / sqrt 2) / 2: the complementary
// error function keeps Phi's relative accuracy in the negative tail, where
// the 1 + erf form cancels.
__device__ __forceinline__ float gelu_f32(float z) {
#pragma clang fp contract(off)
  return 0.5f * z * erfc_f32(z * -0.7071067812f);
}

// The activation in fp32 for an output of type DTO (tanh is evaluated to
// the accuracy the output format keeps).
template <int ACT, int DTO>
__device__ __forceinline__ float act_fn(float z, float alpha) {
  if constexpr (ACT == ACT_RELU) return z > 0.0f ? z : 0.0f;
  else if constexpr (ACT == ACT_LEAKY) return z >= 0.0f ? z : alpha * z;
  else if constexpr (ACT == ACT_TANH) return DTO == DT_F16 || DTO == DT_BF16 ? tanh_f32_short(z) : tanh_f32(z);
  else if constexpr (ACT == ACT_GELU) return gelu_f32(z);
  else if constexpr (ACT == ACT_SIGMOID) return sigmoid_f32(z);
  else return z;
}

// Runs f(std::integral_constant<bool, HAS_R>{}): the epilogue with the residual
// loads and adds, or without them.
template <class F>
__device__ __forceinline__ void with_residual(bool has_r, F&& f) {
  if (has_r) f(std::integral_constant<bool, true>{});
  else f(std::integral_constant<bool, false>{});
}

// Runs f(std::integral_constant<int, ACT>{}) for the runtime activation code:
// an epilogue is instantiated once per activation and branches once, not per
// element.
template <class F>
__device__ __forceinline__ void with_act(int act, F&& f) {
  switch (act) {
    case ACT_RELU: f(std::integral_constant<int, ACT_RELU>{}); break;
    case ACT_LEAKY: f(std::integral_constant<int, ACT_LEAKY>{}); break;
    case ACT_TANH: f(std::integral_constant<int, ACT_TANH>{}); break;
    case ACT_GELU: f(std::integral_constant<int, ACT_GELU>{}); break;
    case ACT_SIGMOID: f(std::integral_constant<int, ACT_SIGMOID>{}); break;
    default: f(std::integral_constant<int, ACT_NONE>{}); break;
  }
}

// ---- MFMA ----------------------------------------------------------------
// One 16-byte chunk per lane of each operand.  For 16-bit inputs that is one
// v_mfma_f32_32x32x16 (8 k-values per lane); for fp32 it is four
// v_mfma_f32_32x32x2_f32, element e of the chunk feeding the e-th one.  The
// two operands always use the same (lane, element) -> k assignment, so the
// instruction sums every k of the chunk pair exactly once.
template <int DT> __device__ __forceinline__ void mfma_chunk(f32x16& acc, u32x4 a, u32x4 b);
template <> __device__ __forceinline__ void mfma_chunk<DT_BF16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mfma_chunk<DT_F16>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}
// int8: one v_mfma_i32_32x32x32_i8 (16 k-values per lane); the int32
// accumulators live in the float-typed accumulator registers as bit patterns.
template <> __device__ __forceinline__ void mfma_chunk<DT_I8>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                       __builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b),
                                       __builtin_bit_cast(i32x16, acc), 0, 0, 0));
}
template <> __device__ __forceinline__ void mfma_chunk<DT_F32>(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Unsigned division by a runtime-invariant divisor via a precomputed
// multiplier (round-up method of Granlund & Montgomery, "Division by
// Invariant Integers using Multiplication", 1994): q = (umulhi(n, mul) + n) >> shift
// for 0 <= n < 2^31.
struct FastDiv {
  uint32_t div, mul, shift;
};
__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.div = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;     // s = ceil(log2 d)
  f.shift = s;
  // mul = floor(2^32 * (2^s - d) / d) + 1
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.mul) + n) >> f.shift;
}

}  // namespace biasact
