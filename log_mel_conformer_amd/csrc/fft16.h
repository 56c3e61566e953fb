// Radix-4 building blocks of the in-register 16-point complex DFTs that
// the log-mel front ends split their 512-point real FFTs into.
#pragma once

#include <hip/hip_runtime.h>

namespace ae {

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
// a * (-i)
__device__ __forceinline__ float2 mul_mi(float2 a) { return make_float2(a.y, -a.x); }

// y_k = sum_m a_m (-i)^{mk}
__device__ __forceinline__ void dft4(float2& a0, float2& a1, float2& a2, float2& a3) {
  const float2 s02 = cadd(a0, a2), d02 = csub(a0, a2);
  const float2 s13 = cadd(a1, a3), d13 = mul_mi(csub(a1, a3));
  a0 = cadd(s02, s13);
  a1 = cadd(d02, d13);
  a2 = csub(s02, s13);
  a3 = csub(d02, d13);
}

// e^{-2 pi i e / 16} for e = 0..15 (cos and sin of multiples of pi/8).
__device__ __forceinline__ float2 w16(int e) {
  constexpr float c1 = 0.92387953251128675613f, s1 = 0.38268343236508977173f;
  constexpr float r2 = 0.70710678118654752440f;
  switch (e & 15) {
    case 0: return make_float2(1.f, 0.f);
    case 1: return make_float2(c1, -s1);
    case 2: return make_float2(r2, -r2);
    case 3: return make_float2(s1, -c1);
    case 4: return make_float2(0.f, -1.f);
    case 6: return make_float2(-r2, -r2);
    case 9: return make_float2(-c1, s1);
    default: return make_float2(0.f, 0.f);  // not used by dft16
  }
}

// 16-point DFT in place: input index m = 4 m1 + m2, output k = k1 + 4 k2.
__device__ __forceinline__ void dft16(float2 (&x)[16]) {
#pragma unroll
  for (int m2 = 0; m2 < 4; ++m2) dft4(x[m2], x[4 + m2], x[8 + m2], x[12 + m2]);
  // x[4 k1 + m2] now holds A[m2][k1]; twiddle by W16^(m2 k1)
#pragma unroll
  for (int m2 = 1; m2 < 4; ++m2)
#pragma unroll
    for (int k1 = 1; k1 < 4; ++k1) x[4 * k1 + m2] = cmul(x[4 * k1 + m2], w16(m2 * k1));
  float2 y[16];
#pragma unroll
  for (int k1 = 0; k1 < 4; ++k1) {
    float2 a0 = x[4 * k1], a1 = x[4 * k1 + 1], a2 = x[4 * k1 + 2], a3 = x[4 * k1 + 3];
    dft4(a0, a1, a2, a3);
    y[k1] = a0;
    y[k1 + 4] = a1;
    y[k1 + 8] = a2;
    y[k1 + 12] = a3;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = y[i];
}

}  // namespace ae
