// Shared device-side definitions of libv4attn (gfx950 / CDNA4 only).
//
// Number formats follow the OCP 8-bit floating point specification (E4M3,
// "fn" variant: no infinities, S.1111.111 = NaN, max 448) and the OCP
// Microscaling v1.0 specification (FP4 E2M1 elements, E8M0 block scales).
// Encoders are written from those definitions with integer / exact float
// operations so that every rounding decision is round-to-nearest-even and
// reproducible; decoders use the gfx950 conversion instructions, which are
// exact for these formats.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace v4a {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------------ e4m3fn

constexpr float kE4M3Max = 448.0f;

// Encode |x| <= 448 (the caller clamps) to e4m3fn, RNE.  Normal e4m3 values
// keep 3 of fp32's 23 mantissa bits; below 2^-6 the grid is uniform with
// spacing 2^-9 (subnormals), where x * 2^9 rounded to an integer is the code.
__device__ __forceinline__ uint32_t enc_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  float af = __uint_as_float(a);
  if (af >= kE4M3Max) return sign | 0x7Eu;
  if (af < 0.015625f) {                       // below 2^-6: subnormal grid
    uint32_t n = (uint32_t)__builtin_rintf(af * 512.0f);   // 0..8, 8 = 2^-6
    return sign | n;
  }
  uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);            // RNE at bit 20
  int e = (int)(r >> 23) - 127;                            // -6 .. 8
  return sign | ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
}

// ------------------------------------------------------------------ e2m1

// Encode a value already divided by its block scale to e2m1 (4-bit code),
// RNE with saturation at +-6.  Grid spacing: 0.5 below 2, 1 in [2,4), 2 in [4,6].
// Branch-free: the region picks an exact power-of-two step and a code offset
// (below 2: rint(2a) = codes 0..4; [2,4): rint(a) + 2 = codes 4..6; [4,6):
// rint(a/2) + 4 = codes 6..7), then saturation.
__device__ __forceinline__ uint32_t enc_e2m1(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  const float a = fabsf(x);
  const float step = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
  const uint32_t off = a < 2.0f ? 0u : (a < 4.0f ? 2u : 4u);
  uint32_t c = (uint32_t)__builtin_rintf(a * step) + off;
  c = a >= 6.0f ? 7u : c;
  return sign | c;
}

// floor(log2 a) for a > 0 finite (fp32, including subnormals).
__device__ __forceinline__ int ilog2f(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF);
  if (e == 0) return -127 - __builtin_clz(u & 0x7FFFFF) + 9 - 1;  // subnormal
  return e - 127;
}

// OCP MX shared exponent for FP4 (emax = 2); amax == 0 -> -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = ilog2f(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ------------------------------------------------------------------ misc

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float load_as_f32(const void* p, int dtype_bf16, size_t i) {
  if (dtype_bf16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// ------------------------------------------------------------------ rotary angles

// Sine and cosine of an fp32 angle a (any magnitude a RoPE angle reaches, well
// below 2^40), evaluated in fp64 and rounded to fp32: Cody-Waite reduction
// by pi/2 with the constant split in two doubles and FMA (r = a - k pi/2 to
// ~1e-30 absolute for |k| < 2^40), then the Taylor series of sin and cos on
// |r| <= pi/4 (terms through r^17 / r^16: truncation < 1e-18), then the
// quadrant's swap and signs.  (fp64 runs at the fp32 VALU rate here; the
// fp32 library routines take a slow path for large arguments.)
__device__ __forceinline__ void sincos_angle(float a, float* s, float* c) {
  constexpr double kTwoOverPi = 0.63661977236758134308;
  constexpr double kPio2Hi = 1.5707963267948966192;         // nearest double to pi/2
  constexpr double kPio2Lo = 6.123233995736766036e-17;       // pi/2 - kPio2Hi
  const double x = (double)a;
  const double kd = rint(x * kTwoOverPi);
  double r = fma(-kd, kPio2Hi, x);
  r = fma(-kd, kPio2Lo, r);
  const double r2 = r * r;
  // sin r = r (1 - r2/3! + r2^2/5! - ... + r2^8/17!), cos r = 1 - r2/2! + ... + r2^8/16!
  double ps = 1.0 / 355687428096000.0;                       // 1/17!
  ps = fma(ps, r2, -1.0 / 1307674368000.0);                  // 1/15!
  ps = fma(ps, r2, 1.0 / 6227020800.0);                      // 1/13!
  ps = fma(ps, r2, -1.0 / 39916800.0);                       // 1/11!
  ps = fma(ps, r2, 1.0 / 362880.0);                          // 1/9!
  ps = fma(ps, r2, -1.0 / 5040.0);                           // 1/7!
  ps = fma(ps, r2, 1.0 / 120.0);                             // 1/5!
  ps = fma(ps, r2, -1.0 / 6.0);                              // 1/3!
  const double sr = fma(ps * r2, r, r);
  double pc = 1.0 / 20922789888000.0;                        // 1/16!
  pc = fma(pc, r2, -1.0 / 87178291200.0);                    // 1/14!
  pc = fma(pc, r2, 1.0 / 479001600.0);                       // 1/12!
  pc = fma(pc, r2, -1.0 / 3628800.0);                        // 1/10!
  pc = fma(pc, r2, 1.0 / 40320.0);                           // 1/8!
  pc = fma(pc, r2, -1.0 / 720.0);                            // 1/6!
  pc = fma(pc, r2, 1.0 / 24.0);                              // 1/4!
  pc = fma(pc, r2, -0.5);                                    // 1/2!
  const double cr = fma(pc, r2, 1.0);
  const int q = (int)((long long)kd & 3);
  const double sv = (q == 0) ? sr : (q == 1) ? cr : (q == 2) ? -sr : -cr;
  const double cv = (q == 0) ? cr : (q == 1) ? -sr : (q == 2) ? -cr : sr;
  *s = (float)sv;
  *c = (float)cv;
}

// Monotone map of fp32 to uint32: a < b (as floats) <=> key(a) < key(b).
// -0.0 and +0.0 map to neighbouring keys (-0 below +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace v4a
