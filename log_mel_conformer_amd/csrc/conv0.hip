// Subsampler layer 0: 3x3 stride-2 convolution from the log-mel plane
// (1 channel) to 128 channels, zero padding 1, no bias, then a LayerNorm
// over the channels (gain only, biased variance, eps 1e-6) and ReLU
// (egemma2_audio.rs, module documentation step 3, AudioTower::subsample and
// layer_norm_relu). Frames past the clip's end are zeros: they are never
// computed, and the padding treats them as absent.
//
// One block per output row t1 (a pair of frames): the three mel rows it
// reads (2 t1 - 1 .. 2 t1 + 1) are staged in LDS with a zero border; each
// wavefront owns 16 of the 64 output frequencies and each lane two of the
// 128 channels, so the channel statistics are wavefront reductions. The
// output is channels-last [row][f][c], which is what conv1's implicit GEMM
// gathers 16-byte chunks from.
#include "launch.h"

namespace ae {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) k_conv0(const float* __restrict__ mel,
                                               const int64_t* __restrict__ frame_off,
                                               const int64_t* __restrict__ row_off, int B,
                                               const float* __restrict__ w0,
                                               const float* __restrict__ g0, T* __restrict__ y0) {
  __shared__ float m[3][kMels + 2];
  const int64_t r = blockIdx.x;
  const int c = find_clip(row_off, B, r);
  const int t1 = (int)(r - row_off[c]);
  const int64_t fbase = frame_off[c];
  const int F = (int)(frame_off[c + 1] - fbase);
  for (int idx = threadIdx.x; idx < 3 * (kMels + 2); idx += 256) {
    const int dt = idx / (kMels + 2), j = idx - dt * (kMels + 2);
    const int ti = 2 * t1 + dt - 1, fi = j - 1;
    float v = 0.f;
    if (ti >= 0 && ti < F && fi >= 0 && fi < kMels) v = mel[(fbase + ti) * kMels + fi];
    m[dt][j] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float wa[9], wb[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    wa[k] = w0[lane * 9 + k];
    wb[k] = w0[(lane + 64) * 9 + k];
  }
  const float ga = g0[lane], gb = g0[lane + 64];
  for (int f = w * 16; f < w * 16 + 16; ++f) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt)
#pragma unroll
      for (int df = 0; df < 3; ++df) {
        const float x = m[dt][2 * f + df];  // column 2f + df - 1, shifted by the border
        a += wa[dt * 3 + df] * x;
        b += wb[dt * 3 + df] * x;
      }
    const float mean = wave_sum(a + b) * (1.0f / kC0);
    const float da = a - mean, db = b - mean;
    const float var = wave_sum(da * da + db * db) * (1.0f / kC0);
    const float inv = rsqrtf(var + kEps);
    T* out = y0 + ((size_t)r * kF1 + f) * kC0;
    out[lane] = from_f32<T>(fmaxf(da * inv * ga, 0.f));
    out[lane + 64] = from_f32<T>(fmaxf(db * inv * gb, 0.f));
  }
}

}  // namespace

hipError_t launch_conv0(ae_dtype dt, const float* mel, const int64_t* frame_off,
                        const int64_t* row_off, int B, int64_t total_rows, const float* w0,
                        const float* g0, void* y0, hipStream_t s) {
  if (total_rows <= 0) return hipSuccess;
  if (dt == AE_BF16)
    hipLaunchKernelGGL(k_conv0<bf16>, dim3((unsigned)total_rows), dim3(256), 0, s, mel, frame_off,
                       row_off, B, w0, g0, (bf16*)y0);
  else
    hipLaunchKernelGGL(k_conv0<float>, dim3((unsigned)total_rows), dim3(256), 0, s, mel,
                       frame_off, row_off, B, w0, g0, (float*)y0);
  return hipGetLastError();
}

}  // namespace ae
