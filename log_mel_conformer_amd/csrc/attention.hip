// Local attention core (egemma2_audio.rs, module documentation step 4 and
// AudioTower::attention): token t of head h attends to the tokens
// t - d, d < span = min(pos[t] + 1, left), of its own clip; the logit is
// q_t . k_{t-d} + q_t . R[d] (R the relative key of distance d), capped as
// softcap * tanh(logit / softcap), and the output is the softmax-weighted
// sum of v_{t-d}. q and k arrive already scaled by the projection epilogue.
//
// One block per (32 consecutive tokens, head): the K and V rows those
// tokens can reach (32 + left - 1) and R[0..left) of the head are staged
// in LDS as float; 8 lanes serve one token, 16 of the 128 dimensions each,
// and the per-distance dot products reduce over those 8 lanes. Rows before
// the packed buffer or past its end are staged as zeros and masked out, so
// no uninitialised value can reach the weighted sum.
#include "launch.h"

namespace ae {
namespace {

constexpr int QB = 32;          // tokens per block
constexpr int HD = 128;         // head dim
constexpr int MAXL = 12;        // largest window this kernel serves
constexpr int HALO = MAXL - 1;
constexpr int LDR = HD + 4;     // padded LDS row (floats)

template <typename T>
__global__ void __launch_bounds__(256) k_attn(const T* __restrict__ qkv, const float* __restrict__ R,
                                              const int32_t* __restrict__ pos, int64_t n, int d,
                                              int left, float cap, float lo, float hi,
                                              T* __restrict__ o) {
  __shared__ float Ks[QB + HALO][LDR];
  __shared__ float Vs[QB + HALO][LDR];
  __shared__ float Rs[MAXL][LDR];
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * QB;
  const int tid = threadIdx.x;
  const int64_t ld = 3 * (int64_t)d;
  for (int idx = tid; idx < (QB + HALO) * (HD / 4); idx += 256) {
    const int rr = idx / (HD / 4), c4 = (idx - rr * (HD / 4)) * 4;
    const int64_t t = t0 - HALO + rr;
    float kv[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
    if (t >= 0 && t < n) {
      const T* kp = qkv + t * ld + d + h * HD + c4;
      const T* vp = qkv + t * ld + 2 * d + h * HD + c4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[e] = to_f32(kp[e]);
        vv[e] = to_f32(vp[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Ks[rr][c4 + e] = kv[e];
      Vs[rr][c4 + e] = vv[e];
    }
  }
  for (int idx = tid; idx < MAXL * HD; idx += 256) {
    const int dist = idx / HD, c = idx - dist * HD;
    Rs[dist][c] = dist < left ? R[(int64_t)dist * d + h * HD + c] : 0.f;
  }
  __syncthreads();

  const int qi = tid >> 3, part = tid & 7;
  const int64_t t = t0 + qi;
  const bool valid = t < n;
  float q[16];
  const T* qp = qkv + (valid ? t : 0) * ld + h * HD + part * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) q[i] = valid ? to_f32(qp[i]) : 0.f;
  const int span = valid ? min(pos[t] + 1, left) : 1;

  float s[MAXL];
  float mx = -INFINITY;
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    const float* kr = &Ks[qi + HALO - dist][part * 16];
    const float* rr = &Rs[dist][part * 16];
    float ac = 0.f, bd = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ac += q[i] * kr[i];
      bd += q[i] * rr[i];
    }
    float logit = ac + bd;
    logit += __shfl_xor(logit, 4, 64);
    logit += __shfl_xor(logit, 2, 64);
    logit += __shfl_xor(logit, 1, 64);
    const float z = cap * tanhf(logit / cap);
    s[dist] = dist < span ? z : -INFINITY;
    mx = fmaxf(mx, s[dist]);
  }
  float den = 0.f;
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    s[dist] = dist < span ? expf(s[dist] - mx) : 0.f;
    den += s[dist];
  }
  const float rden = 1.0f / den;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    const float pd = s[dist] * rden;
    const float* vr = &Vs[qi + HALO - dist][part * 16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += pd * vr[i];
  }
  if (valid) {
    T* op = o + t * d + h * HD + part * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) op[i] = from_f32<T>(clampf(acc[i], lo, hi));
  }
}

}  // namespace

hipError_t launch_attention(ae_dtype dt, const void* qkv, const float* R, const int32_t* pos,
                            int64_t n, int d, int heads, int left, float softcap, float lo,
                            float hi, void* o, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d != heads * HD || left > MAXL || left < 1) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + QB - 1) / QB), heads);
  if (dt == AE_BF16)
    hipLaunchKernelGGL(k_attn<bf16>, grid, dim3(256), 0, s, (const bf16*)qkv, R, pos, n, d, left,
                       softcap, lo, hi, (bf16*)o);
  else
    hipLaunchKernelGGL(k_attn<float>, grid, dim3(256), 0, s, (const float*)qkv, R, pos, n, d,
                       left, softcap, lo, hi, (float*)o);
  return hipGetLastError();
}

}  // namespace ae
