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

// e4m3fn input of a per-row quantisation: clamp(RN(x / s), -448, 448), the
// quotient correctly rounded in fp32, from r = RN(1 / s) computed once per row
// (Markstein's correction): q0 = RN(x * r) is within one ulp of x / s, the
// remainder x - s * q0 is exact in one fma, and RN(q0 + rem * r) = RN(x / s)
// whenever the quotient is a normal number. Smaller quotients encode to a
// (signed) zero code either way. The last step is taken negated,
// -RN(-rem * r - q0): rounding to nearest even is symmetric, so the value is
// the same, and a zero x (q0 = x, rem = +0) comes out with x's sign, which
// RN(rem * r + q0) would turn into +0 for x = -0.
__device__ __forceinline__ float quant_div(float x, float s, float r) {
  const float q0 = x * r;
  const float rem = fmaf(-q0, s, x);
  return clamp448(-fmaf(-rem, r, -q0));
}

// Shared exponent of an MX block with E4M3 elements (OCP Microscaling): the
// largest magnitude amax sets x = floor(log2 amax) - 8, 8 being the exponent
// of E4M3's largest normal (448 = 1.75 * 2^8), clamped to the E8M0 range
// [-127, 127]; an all-zero block gets 0. The E8M0 code is x + 127. floor(log2)
// of a normal float is its unbiased exponent field; a subnormal amax is below
// 2^-126, so its x clamps to -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.0f) return 0;
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return ef == 0 ? -127 : max(ef - 127 - 8, -127);
}

// 2^-x for an exponent from mx_exponent (x <= 119, so 127 - x is in [8, 254]:
// a normal float). Multiplying by it is exact wherever the product is a normal
// float; smaller products encode to a zero e4m3fn code either way.
__device__ __forceinline__ float mx_inv_scale(int x) {
  return __uint_as_float((uint32_t)(127 - x) << 23);
}

// n / k for 0 <= n < 2^30 and 1 <= k <= 32 with magic = ceil(2^35 / k):
// n*magic / 2^35 = n/k + n*(magic*k - 2^35)/(k*2^35), and the added term is
// below (k-1)/(32k), too small to carry the fraction of n/k (at most
// (k-1)/k) past the next integer, so the quotient is exact. A multiply
// instead of a division keeps the compiler from branching around it.
__device__ __forceinline__ uint32_t div_k(int n, uint64_t magic) {
  return (uint32_t)(((uint64_t)(uint32_t)n * magic) >> 35);
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
