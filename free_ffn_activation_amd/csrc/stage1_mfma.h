// Helpers shared by the Stage-1 kernels that run the INT4 proxy on the
// matrix cores (v_mfma_f32_16x16x32_f16).
#pragma once

#include "prox_device.h"

namespace prox {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// Eight stored nibbles (code + 8) of one column, rows in the order
// 0, 4, 1, 5, 2, 6, 3, 7 of the dword, as signed f16 codes: a nibble n put
// under the exponent of 1024 (v_bfi_b32 with the bias in a register) is the
// f16 1024 + n (1024 + 16 n for a high nibble), and one packed f16
// subtraction of 1032 (1152) leaves exactly n - 8 (16 (n - 8)).  Signed codes
// keep the matrix core's rounding of each product unbiased across columns;
// with offset codes every product carries the sign of its weight a and the
// rounding adds up over the rows.
__device__ __forceinline__ f16x8_t codes_to_f16(uint32_t w) {
  const uint32_t t = w >> 8;
  const uint32_t bias = 0x64006400u;
  uint32_t q0, q1, q2, q3;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(q0) : "s"(0x000F000Fu), "v"(w), "v"(bias));
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(q1) : "s"(0x00F000F0u), "v"(w), "v"(bias));
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(q2) : "s"(0x000F000Fu), "v"(t), "v"(bias));
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(q3) : "s"(0x00F000F0u), "v"(t), "v"(bias));
  const f16x2_t lo_fix = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const f16x2_t hi_fix = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  const f16x2_t p0 = __builtin_bit_cast(f16x2_t, q0) + lo_fix;
  const f16x2_t p1 = __builtin_bit_cast(f16x2_t, q1) + hi_fix;
  const f16x2_t p2 = __builtin_bit_cast(f16x2_t, q2) + lo_fix;
  const f16x2_t p3 = __builtin_bit_cast(f16x2_t, q3) + hi_fix;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// exponent e with m < 2^e (frexp), clamped so 2^(15-e) and 2^(e-15) stay normal
__device__ __forceinline__ int scale_exponent(float m) {
  if (!(m > 0.f)) return 0;
  int e;
  (void)frexpf(m, &e);
  return max(-111, min(118, e));
}

}  // namespace prox
