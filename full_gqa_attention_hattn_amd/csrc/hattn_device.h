// Device-side helpers shared by the hattn kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hattn {

// Model shape: 16 query heads share 4 KV heads of head_dim 256 ([T1] "GQA, fused projection
// and output gating").
constexpr int kD = 256;
constexpr int kHq = 16;
constexpr int kHkv = 4;
constexpr int kGroup = kHq / kHkv;
constexpr int kMaxHalfRot = 128;  // rot_dim / 2 for the widest rotary span
constexpr float kE4m3Max = 448.f;  // largest finite E4M3 value (8-bit KV cache)
constexpr int kProjHidden = 2560;  // model hidden size (the projections' other side)

typedef uint16_t bf16_t;  // raw bf16 word
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// RoPE inverse frequencies omega_i = fp32(theta ** (-2 i / rot_dim)), computed on the host
// in double and passed by value in the kernel argument segment.
struct RopeTable {
  float inv_freq[kMaxHalfRot];
  int rot_dim;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round two floats to bf16 (nearest-even, v_cvt_pk_bf16_f32) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Round one float to bf16 (nearest-even).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sin and cos of an fp32 angle, with an absolute error below 1e-7 (checked against fp64 sin
// and cos over every RoPE angle p * omega_i with p < 2^20 + 4096: 7.4e-8).
// Range reduction below 2^21: Cody and Waite's additive reduction by pi/2, in fp32 with a
// three-part constant: C1 = fp32(pi/2), C2 = fp32(pi/2 - C1), C3 = -2^-49 the next piece.
// Each product k * Ci is exact inside its fma, and x - k * C1 is exact (a multiple of 2^-23
// below 1 in magnitude).  k = rint(x * 2/pi) rounded in fp32 can miss the nearest quadrant
// by a little, so |r| <= 0.88.  From 2^21 on (positions past two million tokens) the fp32
// quotient can miss the quadrant by many periods, so the reduction runs in fp64 instead:
// k = rint(x * 2/pi) is exact there (x < 2^32), x - k * P1 with P1 = fp64(pi/2) is exact
// inside its fma and rounded once, and P2 = pi/2 - P1 adds the remainder, which leaves r
// within about 1e-16 of the true reduced angle.  On |r| <= 0.88 the Taylor-Maclaurin series
// of sin to r^9 and of cos to r^10 are truncated below 6e-9.
__device__ __forceinline__ void sincos_angle(float x, float* s_out, float* c_out) {
  float r;
  int q;
  if (__builtin_expect(x < 2097152.f, 1)) {
    const float k = __builtin_rintf(__fmul_rn(x, 0.636619772f));  // 2/pi
    r = __builtin_fmaf(-k, 1.57079637f, x);                         // C1
    r = __builtin_fmaf(-k, -4.37113883e-08f, r);                    // C2
    r = __builtin_fmaf(-k, -1.77635684e-15f, r);                    // C3
    q = (int)k & 3;
  } else {
    const double xd = (double)x;
    const double kd = __builtin_rint(xd * 0.63661977236758134308);   // 2/pi
    double rd = __builtin_fma(-kd, 1.5707963267948966192, xd);      // P1
    rd = __builtin_fma(-kd, 6.1232339957367660359e-17, rd);         // P2
    r = (float)rd;
    q = (int)((long long)kd & 3);
  }
  const float r2 = r * r;
  // sin r = r (1 - r^2/3! + r^4/5! - r^6/7! + r^8/9!)
  float sp = 2.75573192e-06f;                        // 1/9!
  sp = __builtin_fmaf(sp, r2, -1.98412698e-04f);     // -1/7!
  sp = __builtin_fmaf(sp, r2, 8.33333333e-03f);      // 1/5!
  sp = __builtin_fmaf(sp, r2, -1.66666667e-01f);     // -1/3!
  const float sn = __builtin_fmaf(sp * r2, r, r);
  // cos r = 1 - r^2/2! + r^4/4! - r^6/6! + r^8/8! - r^10/10!
  float cp = -2.75573192e-07f;                       // -1/10!
  cp = __builtin_fmaf(cp, r2, 2.48015873e-05f);      // 1/8!
  cp = __builtin_fmaf(cp, r2, -1.38888889e-03f);     // -1/6!
  cp = __builtin_fmaf(cp, r2, 4.16666667e-02f);      // 1/4!
  cp = __builtin_fmaf(cp, r2, -0.5f);
  const float cs = __builtin_fmaf(cp, r2, 1.0f);
  float s, c;
  switch (q) {
    case 0: s = sn; c = cs; break;
    case 1: s = cs; c = -sn; break;
    case 2: s = -sn; c = -cs; break;
    default: s = -cs; c = sn; break;
  }
  *s_out = s;
  *c_out = c;
}

// RoPE angle of frequency index i at position p: one fp32 multiply, rounded to nearest.
__device__ __forceinline__ float rope_angle(int p, float inv_freq) {
  return __fmul_rn((float)p, inv_freq);
}

// One rotate-half pair (x_i, x_{i+r/2}) turned by the angle whose cosine and sine are
// (c, s):  y_i = x_i c - x_{i+r/2} s,  y_{i+r/2} = x_{i+r/2} c + x_i s.  The product with s
// is rounded first and the one with c fused into it, written out so that every kernel
// that rotates (standalone RoPE, the rotating append, the fused Q prologues) produces the
// same bits.
__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, float* ya,
                                          float* yb) {
  *ya = __builtin_fmaf(a, c, -__fmul_rn(b, s));
  *yb = __builtin_fmaf(b, c, __fmul_rn(a, s));
}

// Rotates the rotate-half pairs held by one lane in two 8-element Q fragments: xa holds
// dims d .. d + 7 and xb their partners d + r/2 .. d + r/2 + 7; cs(e) returns the (cos, sin)
// of element e's angle.  The results are rounded to bf16 in place.
template <class CosSin>
__device__ __forceinline__ void rope_fragments(bf16x8& xa, bf16x8& xb, CosSin cs) {
  f32x4 ya0, ya1, yb0, yb1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const f32x2 c = cs(e);
    float ya, yb;
    rope_pair((float)xa[e], (float)xb[e], c.x, c.y, &ya, &yb);
    if (e < 4) { ya0[e] = ya; yb0[e] = yb; } else { ya1[e - 4] = ya; yb1[e - 4] = yb; }
  }
  const bf16x4 a0 = __builtin_convertvector(ya0, bf16x4), a1 = __builtin_convertvector(ya1, bf16x4);
  const bf16x4 b0 = __builtin_convertvector(yb0, bf16x4), b1 = __builtin_convertvector(yb1, bf16x4);
  xa = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  xb = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace hattn
