// Device-side numerics shared by the kernels: bfloat16 rounding, the 3D
// rotary rotation and its factors, and the MXFP8 (E4M3 codes, E8M0 scales)
// conversions.  One definition each, so that the publish, the fused QKV
// projection and the 8-bit attention round identically.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wf {

// ---- bfloat16 ----------------------------------------------------------------
// float -> bfloat16 with round-to-nearest-even; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Two floats -> two bfloat16 in one word (a in the low half), by the
// packed conversion instruction (v_cvt_pk_bf16_f32): round-to-nearest-even
// with fp32 denormals kept (the kernels run with denormals enabled), so
// equal to f32_to_bf16_rne for every non-NaN input (a NaN stays a NaN,
// possibly with another payload).
typedef __bf16 wf_bf16x2 __attribute__((ext_vector_type(2)));
typedef float wf_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((wf_f32x2){a, b}, wf_bf16x2));
}

// ---- 3D rotary embedding ("Wave Forcing: Towards Speed-of-Light Streaming
// Video Generation", §4.2: K is rotated before it is published) -------------
// Factors of one element pair at integer position pos on the pair's axis:
// the angle pos * omega (omega = theta^(-2i/d_a)) and its cosine and sine in
// double precision, each rounded to float.  Returned as (cos, sin).
__device__ __forceinline__ float2 rotary_factors(int32_t pos, double omega) {
  const double phi = (double)pos * omega;
  double sn, cn;
  sincos(phi, &sn, &cn);
  return make_float2((float)cn, (float)sn);
}

// y0 = x0*c - x1*s, y1 = x0*s + x1*c with cs = (c, s); each product and the
// sum or difference rounded on its own (no fused multiply-add).
__device__ __forceinline__ void rotate_pair(float x0, float x1, float2 cs, float& y0,
                                            float& y1) {
#pragma clang fp contract(off)
  const float a = x0 * cs.x;
  const float b = x1 * cs.y;
  const float c = x0 * cs.y;
  const float d = x1 * cs.x;
  y0 = a - b;
  y1 = c + d;
}

// ---- MXFP8 (OCP microscaling: E4M3 codes, one E8M0 scale per 32 elements)
// ("Wave Forcing", §5.5: attention with 8-bit QK^T) ---------------------------
// Shared scale code of a block whose largest magnitude is amax:
// floor(log2 amax) - 8 + 127 clamped at 0, i.e. the float exponent field of
// amax minus 8 (0 for zero and for amax below 2^-119).
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 8;
  return (uint32_t)max(e, 0);
}

// E4M3 code of y (finite): the nearest E4M3 value with ties to even,
// saturating at +-448; the sign of zero is kept.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t s = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  uint32_t c;
  if (a < 0.015625f) {
    c = (uint32_t)__builtin_rintf(a * 512.0f);   // subnormal grid, step 2^-9
  } else {
    // keep 3 of the 23 mantissa bits, rounding to nearest even; a carry
    // moves into the exponent; rebias 127 -> 7
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    c = (b >> 20) - (120u << 3);
  }
  return s | c;
}

}  // namespace wf
