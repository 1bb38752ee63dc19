// Counter-based Gaussian noise: Philox4x32-10 + Box-Muller in a fixed fp32
// operation sequence.
//
// The pages fix only the law of the noise, N(0, sigma^2 C^2 I) (FPC Gaussian
// mechanism; SEDP eq. (2.1)). The generator is Philox4x32-10 as defined by
// Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): 10 rounds, each multiplying words 0 and 2 by M0/M1 into 64-bit
// products whose hi halves are xored with words 1/3 and the round key; the
// key advances by the Weyl constants W0/W1 between rounds.
//
// Stream: key = (seed lo32, seed hi32); element e of a flat output uses lane
// e % 4 of the block at counter (e / 4, 2*layer + which, step, tag).
// Box-Muller on (x0, x1) and (x2, x3): u1 = ((x >> 8) + 1) * 2^-24,
// v = x' >> 8, quadrant q = v >> 22, in-quadrant fraction f = (v mod 2^22) * 2^-22,
// r = sqrt(-2 ln u1), (cos, sin)(2 pi u2) from quarter-turn polynomials.
// Every operation is an IEEE fp32 add/sub/mul rounded on its own (contraction
// is off in these functions); there is no division or square root: both are
// fixed Newton sequences from integer-bit initial guesses, so that a CPU
// replica can follow the same operations exactly.
// rcp(b):   r = bits(0x7EF311C3 - bits(b)), 3 x  r = r * (2 - b*r)
// rsqrt(t): y = bits(0x5F3759DF - (bits(t) >> 1)), h = t/2, 3 x  y = y * (1.5 - h*(y*y))
// ln: u1 = m 2^e, m in [2^-1/2, 2^1/2], s = (m-1) * rcp(m+1),
//     ln m = 2s * (1 + s^2/3 + s^4/5 + ... + s^10/11) (atanh series, Horner in s^2).
// r = t * rsqrt(t) for t = -2 ln u1 > 0, else 0.
// sin/cos of phi = g*pi/2, g = f or 1-f (then swapped), Taylor to phi^9 / phi^10.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpk {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    // each 64-bit product is one v_mad_u64_u32 (both halves), not a mul_lo + mul_hi pair
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c.x;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
  }
  return c;
}

// Reciprocal of b in [1.7, 2.5]: three Newton steps (relative error < 2e-7).
__device__ __forceinline__ float rcp_spec(float b) {
#pragma clang fp contract(off)
  float r = __uint_as_float(0x7EF311C3u - __float_as_uint(b));
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    float t = b * r;
    t = 2.0f - t;
    r = r * t;
  }
  return r;
}

// 1/sqrt(t) for t > 0: three Newton steps (relative error < 2e-7).
__device__ __forceinline__ float rsqrt_spec(float t) {
#pragma clang fp contract(off)
  float y = __uint_as_float(0x5F3759DFu - (__float_as_uint(t) >> 1));
  const float h = 0.5f * t;
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    const float y2 = y * y;
    const float pr = h * y2;
    const float q = 1.5f - pr;
    y = y * q;
  }
  return y;
}

__device__ __forceinline__ float ln_spec(float u) {
#pragma clang fp contract(off)
  const float kLn2 = 0x1.62e430p-1f;
  const float kSqrt2 = 0x1.6a09e6p+0f;
  const uint32_t bits = __float_as_uint(u);
  int e = (int)(bits >> 23) - 127;
  float m = __uint_as_float((bits & 0x007FFFFFu) | 0x3F800000u);
  if (m > kSqrt2) {
    m = m * 0.5f;
    e = e + 1;
  }
  const float s = (m - 1.0f) * rcp_spec(m + 1.0f);
  const float s2 = s * s;
  float p = 0x1.745d18p-4f;   // 1/11
  p = p * s2 + 0x1.c71c72p-4f;  // 1/9
  p = p * s2 + 0x1.24924ap-3f;  // 1/7
  p = p * s2 + 0x1.99999ap-3f;  // 1/5
  p = p * s2 + 0x1.555556p-2f;  // 1/3
  p = p * s2 + 1.0f;
  const float lnm = (s + s) * p;
  return (float)e * kLn2 + lnm;
}

// (sin, cos) of (pi/2) * f for f in [0, 1).
__device__ __forceinline__ void sincos_quarter_spec(float f, float* so, float* co) {
#pragma clang fp contract(off)
  const bool swap = f > 0.5f;
  const float g = swap ? (1.0f - f) : f;
  const float phi = g * 0x1.921fb6p+0f;
  const float p2 = phi * phi;
  float ps = 0x1.71de3ap-19f;      // 1/9!
  ps = ps * p2 + -0x1.a01a02p-13f;  // -1/7!
  ps = ps * p2 + 0x1.111112p-7f;    // 1/5!
  ps = ps * p2 + -0x1.555556p-3f;   // -1/3!
  const float sin_phi = phi + phi * (p2 * ps);
  float pc = -0x1.27e4fcp-22f;      // -1/10!
  pc = pc * p2 + 0x1.a01a02p-16f;   // 1/8!
  pc = pc * p2 + -0x1.6c16c2p-10f;  // -1/6!
  pc = pc * p2 + 0x1.555556p-5f;    // 1/4!
  pc = pc * p2 + -0x1.000000p-1f;   // -1/2
  const float cos_phi = 1.0f + p2 * pc;
  *so = swap ? cos_phi : sin_phi;
  *co = swap ? sin_phi : cos_phi;
}

__device__ __forceinline__ void box_muller_spec(uint32_t xa, uint32_t xb, float* z0, float* z1) {
#pragma clang fp contract(off)
  const float u1 = (float)((xa >> 8) + 1u) * 0x1p-24f;
  const uint32_t v = xb >> 8;
  const uint32_t q = v >> 22;
  const float f = (float)(v & 0x3FFFFFu) * 0x1p-22f;
  const float t = -2.0f * ln_spec(u1);
  const float r = t > 0.0f ? t * rsqrt_spec(t > 0.0f ? t : 1.0f) : 0.0f;
  float s, c;
  sincos_quarter_spec(f, &s, &c);
  // rotate (c, s) by q quarter turns without branches: odd q swaps the pair,
  // q in {1, 2} negates the cosine, q in {2, 3} negates the sine
  const uint32_t odd = q & 1u;
  const float a = odd ? s : c;
  const float b = odd ? c : s;
  const uint32_t neg_c = ((q == 1u) | (q == 2u)) ? 0x80000000u : 0u;
  const uint32_t neg_s = (q >= 2u) ? 0x80000000u : 0u;
  const float ct = __uint_as_float(__float_as_uint(a) ^ neg_c);
  const float st = __uint_as_float(__float_as_uint(b) ^ neg_s);
  *z0 = r * ct;
  *z1 = r * st;
}

// The four normals of group j of stream (key, word1, step, tag).
__device__ __forceinline__ f32x4 normals4(uint32_t j, uint32_t word1, uint32_t step, uint32_t tag,
                                           uint32_t k0, uint32_t k1) {
  const uint4 x = philox4x32_10(make_uint4(j, word1, step, tag), k0, k1);
  float a, b, c, d;
  box_muller_spec(x.x, x.y, &a, &b);
  box_muller_spec(x.z, x.w, &c, &d);
  f32x4 z;
  z[0] = a;
  z[1] = b;
  z[2] = c;
  z[3] = d;
  return z;
}

// out = (S + (sigma*C) * z) * inv_denom, each operation rounded to fp32;
// inv_denom is 1/denom rounded once on the host (exact for powers of two).
__device__ __forceinline__ float noised_mean_spec(float S, float sc, float z, float inv_denom) {
#pragma clang fp contract(off)
  const float n = sc * z;
  const float o = S + n;
  return o * inv_denom;
}

}  // namespace dpk
