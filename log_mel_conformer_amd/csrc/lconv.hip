// Light-conv middle: causal depthwise convolution, RMS norm, SiLU and the
// input clamp of linear_end (egemma2_audio.rs, module documentation step 4,
// dwconv and norm_silu). The GLU before it is fused into linear_start's
// GEMM epilogue.
//
// out[t, c] = sum_k w[c][k] u[t - (K-1-k), c], skipping taps that reach
// before the clip start (K-1-k > pos[t]). The taps arrive transposed,
// wt[k][c], so a lane reads four channels of one tap as one float4. One
// wavefront per row, a lane holding d/64 channels (four runs of four); the
// K rows a token reads are its own and its K-1 predecessors, which
// neighbouring wavefronts read too, so they come from cache after the
// first touch.
#include "launch.h"

namespace ae {
namespace {

__device__ __forceinline__ void load4(const float* p, float* v) {
  const float4 a = *(const float4*)p;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 a = *(const bf16x4*)p;
  v[0] = (float)a[0]; v[1] = (float)a[1]; v[2] = (float)a[2]; v[3] = (float)a[3];
}
__device__ __forceinline__ void store4v(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4v(bf16* p, const float* v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 a = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *(bf16x4*)p = a;
}

template <typename T, int VPL>
__global__ void __launch_bounds__(256) k_lconv(const T* __restrict__ u, const float* __restrict__ wt,
                                               int K, const float* __restrict__ wn,
                                               const int32_t* __restrict__ pos, int64_t n, float lo,
                                               float hi, T* __restrict__ out) {
  constexpr int NV = VPL / 4;
  constexpr int d = VPL * 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int pr = pos[row];
  float x[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) x[i] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int back = K - 1 - k;
    if (back > pr || back > row) continue;  // never before the clip or the buffer
    const T* ur = u + (row - back) * d;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int c = q * 256 + lane * 4;
      const float4 w = *(const float4*)(wt + k * d + c);
      float uv[4];
      load4(ur + c, uv);
      x[4 * q] += w.x * uv[0];
      x[4 * q + 1] += w.y * uv[1];
      x[4 * q + 2] += w.z * uv[2];
      x[4 * q + 3] += w.w * uv[3];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) ss += x[i] * x[i];
  const float inv = rsqrtf(wave_sum(ss) * (1.0f / d) + kEps);
  T* orow = out + row * d;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int c = q * 256 + lane * 4;
    const float4 g = *(const float4*)(wn + c);
    const float gg[4] = {g.x, g.y, g.z, g.w};
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float y = x[4 * q + e] * inv * gg[e];
      o[e] = clampf(y * sigmoidf_(y), lo, hi);
    }
    store4v(orow + c, o);
  }
}

// The same computation for the tower's 5-tap kernel with one wavefront per
// RW consecutive rows: the taps stay in registers for all RW rows, and the
// RW + 4 input rows the wavefront reads (its rows and the four before them)
// are all loaded up front, in the storage type, before the first row is
// computed, so the wavefront waits for memory once. Taps reaching before
// the clip start are skipped by the same pos test, which also keeps rows of
// a previous clip out of the sum.
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x4*)p; }
  __device__ __forceinline__ void zero() { v = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f}; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <> struct Raw4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *(const float4*)p; }
  __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ float operator[](int e) const {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  }
};

template <typename T, int VPL, int RW>
__global__ void __launch_bounds__(256) k_lconv5(const T* __restrict__ u, const float* __restrict__ wt,
                                                const float* __restrict__ wn,
                                                const int32_t* __restrict__ pos, int64_t n,
                                                float lo, float hi, T* __restrict__ out) {
  constexpr int K = 5, NV = VPL / 4, d = VPL * 64;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RW;
  if (row0 >= n) return;
  // rows row0 - 4 .. row0 + RW - 1; those outside [0, n) are zeros (a row
  // before the buffer start is never used: pos keeps taps inside the clip)
  Raw4<T> raw[RW + K - 1][NV];
#pragma unroll
  for (int i = 0; i < RW + K - 1; ++i) {
    const int64_t r = row0 - (K - 1) + i;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      if (r >= 0 && r < n) raw[i][q].load(u + r * d + q * 256 + lane * 4);
      else raw[i][q].zero();
    }
  }
  float w[K][VPL], g[VPL];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const float4 v = *(const float4*)(wt + k * d + q * 256 + lane * 4);
      w[k][4 * q] = v.x; w[k][4 * q + 1] = v.y; w[k][4 * q + 2] = v.z; w[k][4 * q + 3] = v.w;
    }
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const float4 v = *(const float4*)(wn + q * 256 + lane * 4);
    g[4 * q] = v.x; g[4 * q + 1] = v.y; g[4 * q + 2] = v.z; g[4 * q + 3] = v.w;
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t row = row0 + r;
    if (row >= n) break;
    const int pr = pos[row];
    float x[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) x[i] = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int back = K - 1 - k;
      if (back > pr) continue;
      // input row row - back sits at raw index r + (K - 1) - back = r + k
#pragma unroll
      for (int q = 0; q < NV; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] += w[k][4 * q + e] * raw[r + k][q][e];
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) ss += x[i] * x[i];
    const float inv = rsqrtf(wave_sum(ss) * (1.0f / d) + kEps);
    T* orow = out + row * d;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = x[4 * q + e] * inv * g[4 * q + e];
        o[e] = clampf(y * sigmoidf_(y), lo, hi);
      }
      store4v(orow + q * 256 + lane * 4, o);
    }
  }
}

}  // namespace

hipError_t launch_lconv(ae_dtype dt, const void* u, const float* w_dwt, int kernel,
                        const float* w_norm, const int32_t* pos, int64_t n, int d, float lo,
                        float hi, void* c, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d != 1024) return hipErrorInvalidValue;
  if (kernel == 5) {
    if (dt == AE_BF16) {
      constexpr int RW = 2;  // fastest of 1, 2, 4, 8 measured on 24000 rows
      hipLaunchKernelGGL((k_lconv5<bf16, 16, RW>), dim3((unsigned)((n + 4 * RW - 1) / (4 * RW))),
                         dim3(256), 0, s, (const bf16*)u, w_dwt, w_norm, pos, n, lo, hi,
                         (bf16*)c);
    } else {
      constexpr int RW = 4;
      hipLaunchKernelGGL((k_lconv5<float, 16, RW>), dim3((unsigned)((n + 4 * RW - 1) / (4 * RW))),
                         dim3(256), 0, s, (const float*)u, w_dwt, w_norm, pos, n, lo, hi,
                         (float*)c);
    }
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((n + 3) / 4);
  if (dt == AE_BF16)
    hipLaunchKernelGGL((k_lconv<bf16, 16>), dim3(grid), dim3(256), 0, s, (const bf16*)u, w_dwt,
                       kernel, w_norm, pos, n, lo, hi, (bf16*)c);
  else
    hipLaunchKernelGGL((k_lconv<float, 16>), dim3(grid), dim3(256), 0, s, (const float*)u, w_dwt,
                       kernel, w_norm, pos, n, lo, hi, (float*)c);
  return hipGetLastError();
}

}  // namespace ae
