// epilogue.hpp — bias fetch and output stores shared by the biasact kernels.
#pragma once

#include "device_common.hpp"

namespace biasact {

// Per-element bias fetch (fp32, fp16 or bf16 storage), exact widening.
__device__ __forceinline__ float load_bias(__amdgpu_buffer_rsrc_t r, int dt, uint32_t idx) {
  if (dt == DT_F32) return __uint_as_float(ld_b32(r, idx * 4));
  const uint32_t w = ld_b16(r, idx * 2);
  return dt == DT_F16 ? widen<DT_F16>(w) : widen<DT_BF16>(w);
}

// NV bias values bias[idx[v]] (0 where idx[v] >= lim or without bias), all
// loads issued before the first use; the element-type branch is uniform.
template <int NV>
__device__ __forceinline__ void load_bias_vec(const void* bias, uint32_t nbytes, int dt,
                                              const uint32_t (&idx)[NV], uint32_t lim,
                                              float (&out)[NV]) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(bias, nbytes);
  if (dt == DT_F32 || dt == DT_I32) {        // int32: the bit pattern, for int8 GEMMs
#pragma unroll
    for (int v = 0; v < NV; ++v) out[v] = __uint_as_float(ld_b32(r, idx[v] < lim ? idx[v] * 4u : kOOB));
  } else if (dt == DT_F16) {
#pragma unroll
    for (int v = 0; v < NV; ++v) out[v] = widen<DT_F16>(ld_b16(r, idx[v] < lim ? idx[v] * 2u : kOOB));
  } else if (dt == DT_BF16) {
#pragma unroll
    for (int v = 0; v < NV; ++v) out[v] = widen<DT_BF16>(ld_b16(r, idx[v] < lim ? idx[v] * 2u : kOOB));
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) out[v] = 0.0f;
  }
}

// Residual values at four consecutive outputs (the layout of store4), or at
// one, widened exactly to fp32; 0 where !ok.
template <int DTO>
__device__ __forceinline__ void load4(__amdgpu_buffer_rsrc_t r, uint32_t off_elems, bool ok,
                                      float (&v)[4]) {
  const uint32_t off = ok ? off_elems * Elem<DTO>::bytes : kOOB;
  if constexpr (Elem<DTO>::bytes == 4) {
    const u32x4 w = ld_b128(r, off);
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  } else {
    const u32x2 w = ld_b64(r, off);
    v[0] = widen<DTO>(w.x & 0xffffu); v[1] = widen<DTO>(w.x >> 16);
    v[2] = widen<DTO>(w.y & 0xffffu); v[3] = widen<DTO>(w.y >> 16);
  }
}

template <int DTO>
__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, uint32_t off_elems, bool ok) {
  const uint32_t off = ok ? off_elems * Elem<DTO>::bytes : kOOB;
  if constexpr (Elem<DTO>::bytes == 4) return __uint_as_float(ld_b32(r, off));
  else return widen<DTO>(ld_b16(r, off));
}

// The value an epilogue stores for one accumulator register z.  With int8
// operands the register holds the exact int32 sum (bias included): an int32
// output keeps the integer (ReLU applied on it; the planner admits no other
// activation there), any other output takes it rounded to fp32 and applies
// the activation in fp32.
template <int DTI, int DTO, int ACT>
__device__ __forceinline__ float out_value(float z, float alpha) {
  if constexpr (DTI == DT_I8) {
    const int zi = __float_as_int(z);
    if constexpr (DTO == DT_I32) return __int_as_float(ACT == ACT_RELU ? (zi > 0 ? zi : 0) : zi);
    else return act_fn<ACT, DTO>((float)zi, alpha);
  } else {
    return act_fn<ACT, DTO>(z, alpha);
  }
}

// Store four consecutive outputs (one accumulator register group).
template <int DTO>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off_elems, bool ok,
                                       float v0, float v1, float v2, float v3) {
  const uint32_t off = ok ? off_elems * Elem<DTO>::bytes : kOOB;
  if constexpr (Elem<DTO>::bytes == 4) {
    u32x4 o;
    o.x = __float_as_uint(v0); o.y = __float_as_uint(v1);
    o.z = __float_as_uint(v2); o.w = __float_as_uint(v3);
    st_b128(r, off, o);
  } else {
    u32x2 o;
    o.x = narrow<DTO>(v0) | (narrow<DTO>(v1) << 16);
    o.y = narrow<DTO>(v2) | (narrow<DTO>(v3) << 16);
    st_b64(r, off, o);
  }
}

template <int DTO>
__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, uint32_t off_elems, bool ok, float v) {
  const uint32_t off = ok ? off_elems * Elem<DTO>::bytes : kOOB;
  if constexpr (Elem<DTO>::bytes == 4) st_b32(r, off, __float_as_uint(v));
  else st_b16(r, off, (uint16_t)narrow<DTO>(v));
}

}  // namespace biasact
