// Light-conv middle: causal depthwise convolution, RMS norm, SiLU and the
// input clamp of linear_end (egemma2_audio.rs, module documentation step 4,
// dwconv and norm_silu). The GLU before it is fused into linear_start's
// GEMM epilogue.
//
// out[t, c] = sum_k w[c][k] u[t - (K-1-k), c], skipping taps that reach
// before the clip start (K-1-k > pos[t]). The taps arrive transposed,
// wt[k][c], so a lane reads four channels of one tap as one float4. The
// generic kernel takes one wavefront per row, a lane holding d/64 channels
// (four runs of four); the K rows a token reads are its own and its K-1
// predecessors, which neighbouring wavefronts read too, so they come from
// cache after the first touch. The tower's 5-tap kernel has its own form,
// below.
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

// Four consecutive channels of a row in the storage type.
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x4*)p; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <> struct Raw4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *(const float4*)p; }
  __device__ __forceinline__ float operator[](int e) const {
    return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
  }
};

// The same computation for the tower's 5-tap kernel, one block per RPB
// consecutive rows. Wavefront w takes channels 256 w .. 256 w + 255 of every
// row, four per lane, so a lane keeps its 20 taps and 4 norm weights in
// registers for all RPB rows and each input row is read once per block
// (RPB + 4 rows for RPB outputs, all loads issued before the first use).
// Each wavefront writes its rows' partial sums of squares to LDS; after one
// barrier every lane adds the four partials, in wavefront order, for the
// RMS norm. Taps reaching before the clip start are skipped by the pos test,
// which also keeps rows of a previous clip (and the clamped rows before the
// buffer) out of the sum.
template <typename T, int RPB>
__global__ void __launch_bounds__(256) k_lconv5(const T* __restrict__ u, const float* __restrict__ wt,
                                                const float* __restrict__ wn,
                                                const int32_t* __restrict__ pos, int64_t n,
                                                float lo, float hi, T* __restrict__ out) {
  constexpr int K = 5, d = 1024, NW = 4;
  __shared__ float part[NW][RPB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = 256 * wave + 4 * lane;
  const int64_t row0 = (int64_t)blockIdx.x * RPB;
  // rows row0 - 4 .. row0 + RPB - 1, the index clamped into the buffer
  Raw4<T> raw[RPB + K - 1];
#pragma unroll
  for (int i = 0; i < RPB + K - 1; ++i) {
    int64_t r = row0 - (K - 1) + i;
    r = r < 0 ? 0 : r >= n ? n - 1 : r;
    raw[i].load(u + r * d + c);
  }
  float w[K][4], g[4];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float4 v = *(const float4*)(wt + k * d + c);
    w[k][0] = v.x; w[k][1] = v.y; w[k][2] = v.z; w[k][3] = v.w;
  }
  {
    const float4 v = *(const float4*)(wn + c);
    g[0] = v.x; g[1] = v.y; g[2] = v.z; g[3] = v.w;
  }
  float x[RPB][4];
  // When every row of the block has its four predecessors in its clip (all
  // but the blocks at a clip start), one branch-free path widens each input
  // once; the per-tap tests of the general path below made the compiler
  // widen the bf16 inputs again for every use (26.1 against 27.3 us on
  // 24000 rows, the same sums in the same order)
  int minpos = 1 << 30;
#pragma unroll
  for (int r = 0; r < RPB; ++r) {
    const int64_t row = row0 + r;
    const int pr = pos[row < n ? row : n - 1];
    minpos = pr < minpos ? pr : minpos;
  }
  if (minpos >= K - 1) {
    float uf[RPB + K - 1][4];
#pragma unroll
    for (int i = 0; i < RPB + K - 1; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) uf[i][e] = raw[i][e];
#pragma unroll
    for (int r = 0; r < RPB; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) a += w[k][e] * uf[r + k][e];
        x[r][e] = a;
      }
  } else {
#pragma unroll
  for (int r = 0; r < RPB; ++r) {
    const int64_t row = row0 + r;
    const int pr = pos[row < n ? row : n - 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[r][e] = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (K - 1 - k > pr) continue;
      // input row row - (K - 1 - k) sits at raw index r + k
#pragma unroll
      for (int e = 0; e < 4; ++e) x[r][e] += w[k][e] * raw[r + k][e];
    }
  }
  }
#pragma unroll
  for (int r = 0; r < RPB; ++r) {
    const float ss = wave_sum(x[r][0] * x[r][0] + x[r][1] * x[r][1] + x[r][2] * x[r][2] +
                              x[r][3] * x[r][3]);
    if (lane == 0) part[wave][r] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RPB; ++r) {
    const int64_t row = row0 + r;
    if (row >= n) break;
    const float tot = (part[0][r] + part[1][r]) + (part[2][r] + part[3][r]);
    const float inv = rsqrtf(tot * (1.0f / d) + kEps);
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float y = x[r][e] * inv * g[e];
      o[e] = clampf(y * sigmoidf_(y), lo, hi);
    }
    store4v(out + row * d + c, o);
  }
}

}  // namespace

hipError_t launch_lconv(ae_dtype dt, const void* u, const float* w_dwt, int kernel,
                        const float* w_norm, const int32_t* pos, int64_t n, int d, float lo,
                        float hi, void* c, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d != 1024) return hipErrorInvalidValue;
  if (kernel == 5) {
    // 8 rows a block: 27.1-27.8 us on 24000 rows against 28.1 for 4, 31.2 for
    // 16, 46 for 32 and 33.8 for the wavefront-per-two-rows form before it
    constexpr int RPB = 8;
    const dim3 grid((unsigned)((n + RPB - 1) / RPB));
    if (dt == AE_BF16)
      hipLaunchKernelGGL((k_lconv5<bf16, RPB>), grid, dim3(256), 0, s, (const bf16*)u, w_dwt, w_norm,
                         pos, n, lo, hi, (bf16*)c);
    else
      hipLaunchKernelGGL((k_lconv5<float, RPB>), grid, dim3(256), 0, s, (const float*)u, w_dwt,
                         w_norm, pos, n, lo, hi, (float*)c);
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
