// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 packed little-endian (a in the low half), round to
// nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 -> two OCP e4m3fn codes in the low 16 bits (round to nearest even).
// Callers clamp to [-448, 448] first.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Four fp32 -> four e4m3fn codes packed little-endian in a 32-bit word.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ float clamp448(float v) {
  return fminf(fmaxf(v, -448.0f), 448.0f);
}

// Physical workgroup id -> logical tile id so that each XCD (workgroups are
// dealt round robin over the 8 XCDs) gets one contiguous run of logical tiles;
// neighbouring logical tiles then share operands in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int ntiles) {
  constexpr int kXcd = 8;
  int q = ntiles / kXcd, r = ntiles % kXcd;
  int x = bid % kXcd, j = bid / kXcd;
  return x * q + (x < r ? x : r) + j;
}

}  // namespace moe
