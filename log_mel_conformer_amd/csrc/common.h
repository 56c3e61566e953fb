// Internal definitions shared by the HIP sources of libae.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/ae.h"

namespace ae {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSampleRate = 16000;
constexpr int kMaxSamples = 480000;
constexpr int kFrame = 320;
constexpr int kHop = 160;
constexpr int kFft = 512;
constexpr int kBins = kFft / 2 + 1;  // 257
constexpr int kMels = 128;
constexpr float kMelFloor = 1e-3f;
constexpr float kEps = 1e-6f;
constexpr int kC0 = 128;   // conv0 channels
constexpr int kC1 = 32;    // conv1 channels
constexpr int kF1 = 64;    // frequencies after conv0
constexpr int kF2 = 32;    // frequencies after conv1

// Error reporting: a thread-local message returned by ae_last_error().
ae_status set_error(ae_status s, const std::string& msg);

#define AE_HIP_TRY(expr)                                                        \
  do {                                                                          \
    hipError_t e_ = (expr);                                                     \
    if (e_ != hipSuccess)                                                       \
      return ::ae::set_error(AE_ERR_HIP, std::string(#expr) + ": " +          \
                                             hipGetErrorString(e_));            \
  } while (0)

// Launch bookkeeping: a kernel launch followed by the error check, with
// optional HIP-event timing for one kernel class.
void timing_begin(int cls, hipStream_t s);
void timing_end(int cls, hipStream_t s);

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Clamp to [lo, hi] as one v_med3_f32: the median of x, lo and hi is the
// clamped value whenever lo <= hi, which every caller guarantees (the model
// checks its clip bounds at creation; unclamped paths pass -inf and inf).
__device__ __forceinline__ float clampf(float x, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(x, lo, hi);
}
// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp) rather than an
// IEEE divide, which costs ten instructions; exp overflow gives 0 and 1 at
// the ends as it should.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Cross-lane moves within rows of 16 lanes (DPP): CTRL is the dpp_ctrl
// field, 0x00-0xFF a permutation inside each quad of lanes, 0x140 mirrors a
// row, 0x141 mirrors each half row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each quad of lanes (4 consecutive lanes); every lane of the quad
// gets the same bits.
// Wave-local LDS hand-off: this wavefront's LDS writes are visible to its
// own later reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_mov<0xB1>(v);  // quad permutation (1,0,3,2): lane ^ 1
  v += dpp_mov<0x4E>(v);  // quad permutation (2,3,0,1): lane ^ 2
  return v;
}

// Sum over each row of 16 lanes; every lane of the row gets the same bits
// (each step adds a lane to its mirror image, like an xor butterfly).
__device__ __forceinline__ float row16_sum(float v) {
  v = quad_sum(v);
  v += dpp_mov<0x141>(v);  // half-row mirror: quad 0 <-> 1, 2 <-> 3
  v += dpp_mov<0x140>(v);  // row mirror: lanes 0-7 <-> 15-8
  return v;
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// Index of the clip holding packed row `r`: the largest c with off[c] <= r,
// for a non-decreasing off[0..B] (binary search).
__device__ __forceinline__ int find_clip(const int64_t* off, int B, int64_t r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace ae
