// Codes of the quantising cache write, shared by pa_quantize_and_cache and
// the write fused into pa_decode (the same arithmetic, so both store the
// same bytes): a value x of a row with fp32 scale s becomes the code of
// r = x / s (correctly rounded fp32 division), int8 by rounding to the
// nearest integer (ties to even) clamped to [-127, 127], E4M3 by the
// encoder below ("Quantization du KV cache" in the ia-vox KV-cache sizing
// article; E4M3 is the OCP 8-bit format).
#pragma once

namespace pa {

// Nearest OCP E4M3 code to v: ties to the even mantissa, magnitudes above
// 448 saturate, NaN -> 0x7F.  Normal range: keep 3 of fp32's 23 mantissa
// bits with round-to-nearest-even on the 20 dropped bits (a carry moves to
// the exponent), then rebias the exponent from 127 to 7.  Below 2^-6 the
// codes are the multiples of 2^-9 (code 8 being the smallest normal).
__device__ __forceinline__ unsigned e4m3_encode(float v) {
  const unsigned sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a != a) return 0x7Fu;
  if (a > 448.f) return sign | 0x7Eu;
  unsigned code;
  if (a < 0.015625f) {
    code = (unsigned)rintf(a * 512.f);
  } else {
    const unsigned ab = __float_as_uint(a);
    code = ((ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | code;
}

// the code byte of r = x / s: E4M3, or int8 rounded and clamped
template <bool FP8>
__device__ __forceinline__ unsigned quant_code(float r) {
  if constexpr (FP8) {
    return e4m3_encode(r);
  } else {
    const float c = fminf(fmaxf(rintf(r), -127.f), 127.f);
    return (unsigned)(int)c & 0xFFu;
  }
}

// the largest code magnitude: a per-token scale is amax / quant_max (1 for
// an all-zero row)
template <bool FP8>
__device__ __forceinline__ float quant_max() {
  return FP8 ? 448.f : 127.f;
}

}  // namespace pa
