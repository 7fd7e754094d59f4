// Device helpers shared by the gfx950 kernels of the W8A8 layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kQmax = 127;   // symmetric int8 grid [-127, 127]
constexpr float kF8max = 448.0f;   // largest finite FP8 E4M3 value

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bfloat16, nearest with ties to even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (f != f) ? 0x7FC0u : r;
}

// Two binary32 values -> a bfloat16 pair (a in the low half) by one hardware
// conversion (v_cvt_pk_bf16_f32, nearest with ties to even).  For every non-NaN
// binary32 input it gives the bits of f32_to_bf16 (checked on the GPU over all
// 2^32 patterns, subnormals and overflow to infinity included); a NaN stays a NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Correctly rounded binary32 quotient a / b from a binary64 reciprocal:
//   RN32(a / b) == (float)((double)a * rb)   with rb = RN64(1 / (double)b).
// Why: a/b is never a binary32 rounding midpoint, and for 24-bit a and b it
// stays at least 2^-49 (relative) away from every midpoint, while the binary64
// product differs from a/b by less than 2^-51 (relative).  The two therefore
// round to the same binary32 value.  Costs a multiply and two conversions in
// place of the long IEEE division sequence.
__device__ __forceinline__ float div_by_recip(float a, double rb) {
  return (float)((double)a * rb);
}

// One int8 code of the symmetric quantiser: clamp(round_half_even(v / scale)).
__device__ __forceinline__ int quant_code(float v, double rscale) {
  float q = __builtin_rintf(div_by_recip(v, rscale));
  q = __builtin_fminf(__builtin_fmaxf(q, -(float)kQmax), (float)kQmax);
  return (int)q;
}

// Code of the symmetric quantiser as the low byte of a binary32 bit pattern.
// q = RN32(v / scale) is clamped to [-127, 127] (for integer bounds, clamping
// before rounding gives the same integer as rounding first), then adding
// 1.5 * 2^23 rounds it to an integer, ties to even, in the binary32 add itself;
// the low byte of the sum's bit pattern is that integer in two's complement.
__device__ __forceinline__ uint32_t quant_code_bits(float v, double rscale) {
  const float q = __builtin_amdgcn_fmed3f(div_by_recip(v, rscale), -(float)kQmax, (float)kQmax);
  return __float_as_uint(q + 12582912.0f);
}

// FP8 E4M3 (OCP: bias 7, 3 mantissa bits, exponent field 0 = subnormals m * 2^-9,
// largest finite 448) code of the binary32 value q: nearest E4M3 value, ties to
// the even code, saturated at +-448; the sign of q is kept (-0 -> 0x80).
//   |q| < 2^-6: the subnormal grid has step 2^-9, so the code is rne(|q| * 512)
//               (0..8; 8 is the smallest normal, code 0x08);
//   otherwise:  rounding the binary32 mantissa to 3 bits (ties to even, a carry
//               moves into the exponent) and re-biasing the exponent from 127 to 7.
__host__ __device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, q) >> 24) & 0x80u;
  const float a = __builtin_fminf(__builtin_fabsf(q), 448.0f);
  if (a < 0.015625f) {
    const float m = (a * 512.0f + 12582912.0f) - 12582912.0f;   // exact scaling, then rne
    return sign | (uint32_t)m;
  }
  uint32_t b = __builtin_bit_cast(uint32_t, a);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  return sign | (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
}

// Four E4M3 codes (byte i from q[i]) by the hardware conversion, on inputs
// clamped to +-448 first.  On clamped inputs it rounds exactly as e4m3_code
// (checked on the GPU on every binary32 value in [-448, 448] with its top 20 bits
// varied and 5 low-bit patterns, subnormal results and signed zeros included).
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
  auto c = [](float q) { return __builtin_amdgcn_fmed3f(q, -kF8max, kF8max); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c(q0), c(q1), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c(q2), c(q3), lo, true);
}

// Binary32 value of an E4M3 code (exact).
__host__ __device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e == 0 ? (float)m * 0.001953125f                       // m * 2^-9
                         : __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// Low bytes of four words -> one word (byte i from word i).
__device__ __forceinline__ uint32_t pack4_lowbytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)d << 24);
}

// Maximum over the 64 lanes of a non-negative value (so the integer order of the
// bit patterns is the numeric order), by DPP lane exchanges: pairs, quads, half
// rows, rows, then row 0 -> 1 and 2 -> 3, then row 1 -> 2..3; lane 63 ends with
// the total, which is broadcast.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));  // row_mirror
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false));  // row_bcast15
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false));  // row_bcast31
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace sq
