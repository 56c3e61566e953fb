// Light-conv middle: causal depthwise convolution, RMS norm, SiLU and the
// input clamp of linear_end (egemma2_audio.rs, module documentation step 4,
// dwconv and norm_silu). The GLU before it is fused into linear_start's
// GEMM epilogue.
//
// out[t, c] = sum_k w[c][k] u[t - (K-1-k), c], skipping taps that reach
// before the clip start (K-1-k > pos[t]). One wavefront per row, a lane
// holding d/64 channels; the K rows a token reads are its own and its
// K-1 predecessors, which neighbouring wavefronts read too, so they come
// from cache after the first touch.
#include "launch.h"

namespace ae {
namespace {

template <typename T, int VPL>
__global__ void __launch_bounds__(256) k_lconv(const T* __restrict__ u, const float* __restrict__ wdw,
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
    if (back > pr || back > row) continue;  // never before the packed buffer
    const T* ur = u + (row - back) * d;
#pragma unroll
    for (int q = 0; q < NV; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = q * 256 + lane * 4 + e;
        x[4 * q + e] += wdw[c * K + k] * to_f32(ur[c]);
      }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) ss += x[i] * x[i];
  const float inv = rsqrtf(wave_sum(ss) * (1.0f / d) + kEps);
  T* orow = out + row * d;
#pragma unroll
  for (int q = 0; q < NV; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = q * 256 + lane * 4 + e;
      const float y = x[4 * q + e] * inv * wn[c];
      orow[c] = from_f32<T>(clampf(y * sigmoidf_(y), lo, hi));
    }
}

}  // namespace

hipError_t launch_lconv(ae_dtype dt, const void* u, const float* w_dw, int kernel,
                        const float* w_norm, const int32_t* pos, int64_t n, int d, float lo,
                        float hi, void* c, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d != 1024) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((n + 3) / 4);
  if (dt == AE_BF16)
    hipLaunchKernelGGL((k_lconv<bf16, 16>), dim3(grid), dim3(256), 0, s, (const bf16*)u, w_dw,
                       kernel, w_norm, pos, n, lo, hi, (bf16*)c);
  else
    hipLaunchKernelGGL((k_lconv<float, 16>), dim3(grid), dim3(256), 0, s, (const float*)u, w_dw,
                       kernel, w_norm, pos, n, lo, hi, (float*)c);
  return hipGetLastError();
}

}  // namespace ae
