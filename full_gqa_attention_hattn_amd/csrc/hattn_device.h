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

// sin and cos of an fp32 angle, accurate to well below one fp32 ulp for |x| < 2^30.
// Range reduction: Cody and Waite's additive reduction by pi/2 with a two-word pi/2 in
// double precision and fused multiply-adds (k * C1 is exact inside the fma, the residual
// C2 = pi/2 - C1 carries the next 53 bits).  Kernels: Taylor-Maclaurin series of sin and
// cos on |r| <= pi/4, truncated where the next term is below 1e-11.
__device__ __forceinline__ void sincos_angle(float xf, float* s_out, float* c_out) {
  const double x = (double)xf;
  const double kTwoOverPi = 0.63661977236758134308;
  const double kC1 = 1.5707963267948965580e+00;  // pi/2 rounded to double
  const double kC2 = 6.1232339957367658e-17;     // pi/2 - kC1
  const double k = __builtin_rint(x * kTwoOverPi);
  double r = __builtin_fma(-k, kC1, x);
  r = __builtin_fma(-k, kC2, r);
  const double r2 = r * r;
  // sin r = r (1 - r^2/3! + r^4/5! - r^6/7! + r^8/9! - r^10/11!)
  double sp = -2.5052108385441718775e-08;         // -1/11!
  sp = __builtin_fma(sp, r2, 2.7557319223985890653e-06);   // 1/9!
  sp = __builtin_fma(sp, r2, -1.9841269841269841270e-04);  // -1/7!
  sp = __builtin_fma(sp, r2, 8.3333333333333333333e-03);   // 1/5!
  sp = __builtin_fma(sp, r2, -1.6666666666666666667e-01);  // -1/3!
  const double sn = __builtin_fma(sp * r2, r, r);
  // cos r = 1 - r^2/2! + r^4/4! - r^6/6! + r^8/8! - r^10/10! + r^12/12!
  double cp = 2.0876756987868098979e-09;          // 1/12!
  cp = __builtin_fma(cp, r2, -2.7557319223985890653e-07);  // -1/10!
  cp = __builtin_fma(cp, r2, 2.4801587301587301587e-05);   // 1/8!
  cp = __builtin_fma(cp, r2, -1.3888888888888888889e-03);  // -1/6!
  cp = __builtin_fma(cp, r2, 4.1666666666666666667e-02);   // 1/4!
  cp = __builtin_fma(cp, r2, -0.5);
  const double cs = __builtin_fma(cp, r2, 1.0);
  const int q = (int)((long long)k & 3);
  double s, c;
  switch (q) {
    case 0: s = sn; c = cs; break;
    case 1: s = cs; c = -sn; break;
    case 2: s = -sn; c = -cs; break;
    default: s = -cs; c = sn; break;
  }
  *s_out = (float)s;
  *c_out = (float)c;
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

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace hattn
