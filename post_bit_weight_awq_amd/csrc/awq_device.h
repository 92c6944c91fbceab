// Device-side helpers shared by the gfx950 kernels of the AWQ search library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 128;

// Bit pattern of -0.0f.  Used as the addend of the mixed-precision FMAs below:
// a*b + (-0) equals the rounded product a*b for every a, b (signed zeros
// included), so those FMAs are exact products with a single rounding.
__device__ __forceinline__ float neg_zero() { return __uint_as_float(0x80000000u); }

// -0.0f in a register whose value the compiler cannot see.  Passed as the
// addend of mul_f16_f32, it keeps that function one mixed-precision FMA
// (v_fma_mix_f32): with a known -0 the compiler would fold the FMA into a
// conversion and a multiply.  Take it once per kernel.
__device__ __forceinline__ float opaque_neg_zero() {
  float r;
  asm volatile("v_mov_b32 %0, 0x80000000" : "=v"(r));
  return r;
}

// fp32(h * s) where h is the low (HI=false) or high (HI=true) fp16 half of `w2`.
// The fp16 operand is widened exactly and nz is -0, so this equals
// fp32(fp32(h) * s) with a single rounding; written in C so the compiler
// knows the instruction it selects (no padding for an unknown inline asm).
template <bool HI>
__device__ __forceinline__ float mul_f16_f32(uint32_t w2, float s, float nz) {
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(HI ? (w2 >> 16) : (w2 & 0xffffu)));
  return __builtin_fmaf((float)h, s, nz);
}

// The same with a wavefront-uniform scale held in a scalar register (saves the
// copy into a vector register; at most one scalar operand per instruction).
template <bool HI>
__device__ __forceinline__ float mul_f16_f32_s(uint32_t w2, float s_uniform, float nz) {
  float r;
  if (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r) : "v"(w2), "s"(s_uniform), "v"(nz));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r) : "v"(w2), "s"(s_uniform), "v"(nz));
  return r;
}

// Two fp16 values packed in one register: lo = fp16(a0 * b0), hi = fp16(a1 * b1),
// each product of two fp32 values rounded ONCE (to nearest even) to fp16.
__device__ __forceinline__ uint32_t mul_f32_to_f16x2(float a0, float b0, float a1, float b1,
                                                     float nz) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]"
      : "=v"(r) : "v"(a0), "v"(b0), "v"(nz));
  asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]"
      : "+v"(r) : "v"(a1), "v"(b1), "v"(nz));
  return r;
}

// As mul_f32_to_f16x2 with wavefront-uniform b0, b1 in scalar registers.
__device__ __forceinline__ uint32_t mul_f32_to_f16x2_s(float a0, float b0_uniform, float a1,
                                                       float b1_uniform, float nz) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]"
      : "=v"(r) : "v"(a0), "s"(b0_uniform), "v"(nz));
  asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel_hi:[0,0,0]"
      : "+v"(r) : "v"(a1), "s"(b1_uniform), "v"(nz));
  return r;
}

// Packed fp16 a - b, each half rounded once (IEEE, to nearest even).
__device__ __forceinline__ uint32_t sub_f16x2(uint32_t a, uint32_t b) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v r = __builtin_bit_cast(half2v, a) - __builtin_bit_cast(half2v, b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Quantizer parameters of one (grid point, output row, group of 128):
// step = (max - min) / 15, its binary32 reciprocal, and the clamp bounds of
// (q - zero): lo = -zero, hi = 15 - zero.
struct GroupParams {
  float step, inv_step, lo, hi;
};

__device__ __forceinline__ float med3(float x, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(x, lo, hi);
}

}  // namespace awq
