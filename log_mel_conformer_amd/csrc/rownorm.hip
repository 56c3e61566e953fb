// Fused row kernels around the residual stream: the RMS norms of the tower
// (x / sqrt(mean(x^2) + 1e-6) times the weight plainly; ltxdit.rs rms_w /
// rms_plain, egemma2_audio.rs module documentation step 4) and the
// residual updates that surround them (egemma2_audio.rs add_normed, ffn,
// encode_locked).
//
// One wavefront per row; a lane holds VPL = d/64 values, loaded as float4
// so that every load instruction of the wavefront covers 1 KB of
// contiguous memory. A row is read once and every norm of the chain
// (post-norm residual, norm_out, the next block's pre-norm and the next
// projection's input clamp) is applied while it sits in registers.
//
// In bf16 models the row kernels of a layer run in pairs: the first of a
// pair writes only the next projection's input and leaves h unwritten; the
// second reads the h the first one read plus both GEMM outputs (bf16),
// applies both residual updates and writes h. A pair then moves 22 bytes a
// value where two launches that each read and write the float h move 24.
#include "launch.h"

namespace ae {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load4(const float* p, float* v) {
  const float4 a = *(const float4*)p;
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
__device__ __forceinline__ void store4v(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4v(bf16* p, const float* v) {
  const bf16x4 a = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *(bf16x4*)p = a;
}

template <typename T, int VPL>
__global__ void __launch_bounds__(256) k_rownorm(RowNormParams p) {
  constexpr int NV = VPL / 4;
  typedef typename std::conditional<std::is_same<T, float>::value, float4, bf16x4>::type Raw;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.n) return;  // uniform per wavefront
  const int d = p.d;
  const float invd = 1.0f / (float)d;
  float x[VPL];
  float* hrow = p.h + row * d;
  // every activation load of the row issued before the first use, so a
  // wavefront waits for memory once rather than once per update (47.6 ->
  // 45.4 us a launch on 24000 rows; loading the weight vectors up front
  // as well gave the same time with 120 registers instead of 78)
  Raw ra[NV], rb[NV];
  if (p.y0) {
#pragma unroll
    for (int q = 0; q < NV; ++q) ra[q] = *(const Raw*)((const T*)p.y0 + row * d + q * 256 + lane * 4);
  }
  if (p.y) {
#pragma unroll
    for (int q = 0; q < NV; ++q) rb[q] = *(const Raw*)((const T*)p.y + row * d + q * 256 + lane * 4);
  }
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const float4 v = *(const float4*)(hrow + q * 256 + lane * 4);
    x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
  }
  auto widen = [&](const Raw& r, float* v) {
    if constexpr (std::is_same<T, float>::value) {
      v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    } else {
      v[0] = (float)r[0]; v[1] = (float)r[1]; v[2] = (float)r[2]; v[3] = (float)r[3];
    }
  };
  auto update = [&](const Raw (&raw)[NV], const float* w_post, const float* wsel, float scale) {
    if (!w_post) {
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        float y[4];
        widen(raw[q], y);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] += scale * y[e];
      }
      return;
    }
    float y[VPL];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < NV; ++q) widen(raw[q], y + 4 * q);
#pragma unroll
    for (int i = 0; i < VPL; ++i) ss += y[i] * y[i];
    const float inv = rsqrtf(wave_sum(ss) * invd + kEps);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      float w[4];
      load4(w_post + q * 256 + lane * 4, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] += scale * (y[4 * q + e] * inv * w[e]);
    }
  };
  if (p.y0) update(ra, p.w_post0, nullptr, p.scale0);
  if (p.y) update(rb, p.w_post, nullptr, p.scale);
  if (p.w_out) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) ss += x[i] * x[i];
    const float inv = rsqrtf(wave_sum(ss) * invd + kEps);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      float w[4];
      load4(p.w_out + q * 256 + lane * 4, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = x[4 * q + e] * inv * w[e];
    }
  }
  if ((p.y || p.w_out) && !p.skip_h) {
#pragma unroll
    for (int q = 0; q < NV; ++q)
      *(float4*)(hrow + q * 256 + lane * 4) =
          make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
  }
  if (p.h_copy) {
    T* crow = (T*)p.h_copy + row * d;
#pragma unroll
    for (int q = 0; q < NV; ++q) store4v(crow + q * 256 + lane * 4, x + 4 * q);
  }
  if (p.w_next || p.plain_next) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) ss += x[i] * x[i];
    const float inv = rsqrtf(wave_sum(ss) * invd + kEps);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      float w[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if (p.w_next) load4(p.w_next + q * 256 + lane * 4, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = x[4 * q + e] * inv * w[e];
    }
    for (int s = 0; s < p.n_out; ++s) {
      T* arow = (T*)p.a[s] + row * d;
      const float lo = p.lo[s], hi = p.hi[s];
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = clampf(x[4 * q + e], lo, hi);
        store4v(arow + q * 256 + lane * 4, v);
      }
    }
  }
}

template <typename T>
hipError_t run(const RowNormParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)((p.n + 3) / 4);
  switch (p.d) {
    case 1024: hipLaunchKernelGGL((k_rownorm<T, 16>), dim3(grid), dim3(256), 0, s, p); break;
    case 1536: hipLaunchKernelGGL((k_rownorm<T, 24>), dim3(grid), dim3(256), 0, s, p); break;
    case 2048: hipLaunchKernelGGL((k_rownorm<T, 32>), dim3(grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rownorm(ae_dtype dt, const RowNormParams& p, hipStream_t s) {
  if (p.n <= 0) return hipSuccess;
  return dt == AE_BF16 ? run<bf16>(p, s) : run<float>(p, s);
}

}  // namespace ae
