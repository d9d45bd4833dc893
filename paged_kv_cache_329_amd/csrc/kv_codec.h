// Element codecs shared by the HIP kernels that write the KV cache.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

// float32 -> OCP e4m3fn code: clamp to +-448, round to nearest, ties to even mantissa.
// Below 2^-6 the format is the uniform grid m * 2^-9, so the code is the even-rounded
// integer of |y| * 512 (an exact scaling); a result of 8 is the smallest normal, code 8.
// Otherwise the float32 mantissa is rounded from 23 to 3 bits (add half-ulp minus one plus
// the kept lsb, then truncate) and the exponent is rebased from 127 to 7.  Both results are
// computed and one is selected, so a wave never diverges on the magnitude.
__device__ __forceinline__ uint32_t e4m3fn_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  const uint32_t small = uint32_t(__builtin_rintf(a * 512.0f));
  uint32_t ua = __float_as_uint(a);
  ua += 0x7FFFFu + ((ua >> 20) & 1u);
  const uint32_t normal = (((ua >> 23) - 120u) << 3) | ((ua >> 20) & 7u);
  const uint32_t code = a < 0.015625f ? small : normal;
  return y != y ? (sign | 0x7Fu) : (sign | code);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

}  // namespace pkv
