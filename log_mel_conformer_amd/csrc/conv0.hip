// Subsampler layer 0: 3x3 stride-2 convolution from the log-mel plane
// (1 channel) to 128 channels, zero padding 1, no bias, then a LayerNorm
// over the channels (gain only, biased variance, eps 1e-6) and ReLU
// (egemma2_audio.rs, module documentation step 3, AudioTower::subsample and
// layer_norm_relu). Frames past the clip's end are zeros: they are never
// computed, and the padding treats them as absent.
//
// float storage (k_conv0): one block per 8 consecutive output rows t1
// (pairs of frames; packed, so possibly across clips); for each row the three mel rows it reads
// (2 t1 - 1 .. 2 t1 + 1) are staged in LDS with a zero border, while a
// lane's 72 taps and 8 gains stay in registers for all 8 rows. A lane
// owns 8 consecutive channels of one output frequency; 16 lanes cover the
// 128 channels of a frequency, so the channel statistics are 16-lane
// reductions and each lane writes its 8 outputs as one vector. A wavefront
// does 4 frequencies per pass, 16 per block row. The output is
// channels-last [row][f][c], which is what conv1's implicit GEMM gathers
// 16-byte chunks from.
//
// bf16 models run both convolutions in one pass (subsample.hip); the
// matrix-core fragments of their centred taps are packed here: the nine
// taps of a position against 128 channels are a 32 x 128 x 9 contraction,
// run as v_mfma_f32_32x32x16_bf16 with every operand split into bf16 high
// and low parts (the three cross terms hi.hi + hi.lo + lo.hi, 27 of the 32
// k slots, about 2^-16 relative: far below the bf16 rounding of the
// output). The taps are centred first (each tap minus its mean over the
// channels), so the products are already the channel-centred values the
// LayerNorm needs: the mean pass disappears and the norm is the variance.
#include "launch.h"

namespace ae {
namespace {

constexpr int kConv0Rows = 8;  // output rows per block

// The plane is written once and read once by conv1, and it is larger than
// every cache: its stores are non-temporal (they skip cache allocation;
// measured 239 -> 175 us for the 786 MB bf16 plane, and conv1 reading it
// 293 -> 269 us).
typedef float f32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store8(float* p, const float* v) {
  __builtin_nontemporal_store(f32v4{v[0], v[1], v[2], v[3]}, (f32v4*)p);
  __builtin_nontemporal_store(f32v4{v[4], v[5], v[6], v[7]}, (f32v4*)(p + 4));
}

template <typename T>
__global__ void __launch_bounds__(256) k_conv0(const float* __restrict__ mel,
                                               const int64_t* __restrict__ frame_off,
                                               const int64_t* __restrict__ row_off, int B,
                                               int64_t total_rows, const float* __restrict__ w0,
                                               const float* __restrict__ g0, T* __restrict__ y0) {
  __shared__ float m[3][kMels + 2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int fsub = lane >> 4, c0 = (lane & 15) * 8;
  // this lane's 8 channels: 9 taps each and the LayerNorm gains, kept in
  // registers for all the block's rows
  float wk[8][9], g[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int k = 0; k < 9; ++k) wk[c][k] = w0[(c0 + c) * 9 + k];
    g[c] = g0[c0 + c];
  }
  const int64_t r_first = (int64_t)blockIdx.x * kConv0Rows;
  for (int rr = 0; rr < kConv0Rows; ++rr) {
    const int64_t r = r_first + rr;
    if (r >= total_rows) break;
    const int c = find_clip(row_off, B, r);
    const int t1 = (int)(r - row_off[c]);
    const int64_t fbase = frame_off[c];
    const int F = (int)(frame_off[c + 1] - fbase);
    if (rr > 0) __syncthreads();  // the previous row's reads of m are done
    for (int idx = threadIdx.x; idx < 3 * (kMels + 2); idx += 256) {
      const int dt = idx / (kMels + 2), j = idx - dt * (kMels + 2);
      const int ti = 2 * t1 + dt - 1, fi = j - 1;
      float v = 0.f;
      if (ti >= 0 && ti < F && fi >= 0 && fi < kMels) v = mel[(fbase + ti) * kMels + fi];
      m[dt][j] = v;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int f = w * 16 + it * 4 + fsub;
      float x[9];
#pragma unroll
      for (int dt = 0; dt < 3; ++dt)
#pragma unroll
        for (int df = 0; df < 3; ++df) x[dt * 3 + df] = m[dt][2 * f + df];  // column 2f+df-1, shifted
      float a[8];
      float sum = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 9; ++k) acc += wk[cc][k] * x[k];
        a[cc] = acc;
        sum += acc;
      }
      sum = row16_sum(sum);
      const float mean = sum * (1.0f / kC0);
      float q = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        a[cc] -= mean;
        q += a[cc] * a[cc];
      }
      q = row16_sum(q);
      const float inv = rsqrtf(q * (1.0f / kC0) + kEps);
      float o8[8];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) o8[cc] = fmaxf(a[cc] * inv * g[cc], 0.f);
      store8(y0 + ((size_t)r * kF1 + f) * kC0 + c0, o8);
    }
  }
}

// Matrix-core fragments of the centred taps, built once per model:
// [tile ct][k-step ks][lane][8 bf16], lane = h * 32 + channel row, so a
// lane's first-operand fragment is one 16-byte load. Slot k (0..31) of
// channel c holds: k < 9 high(w'[c][k]); 9 <= k < 18 high(w'[c][k - 9]);
// 18 <= k < 27 low(w'[c][k - 18]); zero above, where w' = w - mean_c(w)
// and low(x) = bf16(x - high(x)). The position operand holds, slot for
// slot, high(p), low(p), high(p), zero.
__global__ void k_conv0_pack(const float* __restrict__ w0, uint4* __restrict__ frag) {
  __shared__ float wbar[9];
  if (threadIdx.x < 9) {
    float sum = 0.f;
    for (int c = 0; c < kC0; ++c) sum += w0[c * 9 + threadIdx.x];
    wbar[threadIdx.x] = sum * (1.0f / kC0);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 4 * 2 * 64; e += blockDim.x) {
    const int ct = e >> 7, ks = (e >> 6) & 1, l = e & 63;
    const int c = ct * 32 + (l & 31), hh = l >> 5;
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = ks * 16 + hh * 8 + i;
      float x = 0.f;
      if (k < 27) {
        const int term = k / 9, tap = k - 9 * term;
        const float wc = w0[c * 9 + tap] - wbar[tap];
        const float hi = (float)(bf16)wc;
        x = term == 2 ? wc - hi : hi;
      }
      v[i] = (bf16)x;
    }
    frag[e] = __builtin_bit_cast(uint4, v);
  }
}

}  // namespace

hipError_t launch_conv0_pack(const float* w0, void* frag, hipStream_t s) {
  hipLaunchKernelGGL(k_conv0_pack, dim3(1), dim3(256), 0, s, w0, (uint4*)frag);
  return hipGetLastError();
}

hipError_t launch_conv0(ae_dtype dt, const float* mel, const int64_t* frame_off,
                        const int64_t* row_off, int B, int64_t total_rows, const float* w0,
                        const float* g0, void* y0, hipStream_t s) {
  if (total_rows <= 0) return hipSuccess;
  if (dt == AE_BF16) return hipErrorInvalidValue;  // bf16: launch_subsample_fused
  const unsigned grid = (unsigned)((total_rows + kConv0Rows - 1) / kConv0Rows);
  hipLaunchKernelGGL(k_conv0<float>, dim3(grid), dim3(256), 0, s, mel, frame_off, row_off, B,
                     total_rows, w0, g0, (float*)y0);
  return hipGetLastError();
}

}  // namespace ae
