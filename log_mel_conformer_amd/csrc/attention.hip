// Local attention core (egemma2_audio.rs, module documentation step 4 and
// AudioTower::attention): token t of head h attends to the tokens
// t - d, d < span = min(pos[t] + 1, left), of its own clip; the logit is
// q_t . k_{t-d} + q_t . R[d] (R the relative key of distance d), capped as
// softcap * tanh(logit / softcap), and the output is the softmax-weighted
// sum of v_{t-d}. q and k arrive already scaled by the projection epilogue.
//
// One block per (QB consecutive tokens, head). The K and V rows those
// tokens can reach (QB + left - 1 of them) are staged in LDS in the storage
// type (16-byte loads, all issued before the stores; rows padded to spread
// banks), R[0..left) of the head as float with each 32-dimension part
// padded to a 36-float pitch (bf16 storage: R rounded to bf16, parts at a
// 40-element pitch). Four lanes serve one token, 32 of the 128 dimensions
// each: a lane forms its partial logits for every distance, two cross-lane
// steps give all four lanes the full logits, each lane runs the (identical)
// softmax, then accumulates its 32 output dimensions. In bf16 storage the
// partial logits are q.k + q.R by v_dot2_f32_bf16 on the packed values
// (exact products, float32 sums), four times fewer instructions than
// widening each element first. Rows before the packed buffer or past its
// end are staged as zeros and masked out, so no uninitialised value can
// reach the weighted sum.
#include "launch.h"



namespace ae {
namespace {

constexpr int HD = 128;         // head dim
constexpr int MAXL = 12;        // largest window this kernel serves
constexpr int HALO = MAXL - 1;
constexpr int DPL = 32;         // dimensions per lane

template <typename T> struct Stage;
template <> struct Stage<bf16> {
  static constexpr int LD = HD + 8;  // elements per LDS row (pad 16 bytes)
};
template <> struct Stage<float> {
  static constexpr int LD = HD + 4;
};

__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (bf16)v[i];
  *(bf16x8*)p = a;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
// 8 elements of the storage type in registers (16 bytes of bf16, 32 of float)
template <typename T> struct Chunk8;
template <> struct Chunk8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const uint4*)p; }
  __device__ __forceinline__ void zero() { v = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void store(bf16* p) const { *(uint4*)p = v; }
};
template <> struct Chunk8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const float4*)p;
    b = *(const float4*)(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void store(float* p) const {
    *(float4*)p = a;
    *(float4*)(p + 4) = b;
  }
};

// R in LDS: per distance, the four 32-dimension parts at a pitch of 36
// floats, so the parts the four lanes of a token read start on distinct
// banks (a pitch of 32 would put parts 0 and 2 on the same banks).
constexpr int RPART = DPL + 4;
constexpr int RROW = 4 * RPART;
// bf16 storage: the same layout in bf16 elements, parts 80 bytes apart
constexpr int RPART_B = DPL + 8;
constexpr int RROW_B = 4 * RPART_B;
// R in LDS as the storage type: float parts at a 36-float pitch, bf16
// parts at a 40-element pitch
template <typename T> struct RStage;
template <> struct RStage<float> {
  typedef float E;
  static constexpr int N = MAXL * RROW;
};
template <> struct RStage<bf16> {
  typedef bf16 E;
  static constexpr int N = MAXL * RROW_B;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// a.b over two packed bf16 pairs, plus c (float32 accumulation)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <typename T, int QB, int MINB>
__global__ void __launch_bounds__(4 * QB, MINB) k_attn(
    const T* __restrict__ qkv, const float* __restrict__ R, const int32_t* __restrict__ pos,
    int64_t n, int d, int left, float cap, float lo, float hi, T* __restrict__ o) {
  constexpr int NT = 4 * QB;  // threads: four lanes per token
  constexpr int ROWS = QB + HALO;
  constexpr int LD = Stage<T>::LD;
  constexpr bool kBf = std::is_same<T, bf16>::value;
  __shared__ __attribute__((aligned(16))) T Ks[ROWS * LD];
  __shared__ __attribute__((aligned(16))) T Vs[ROWS * LD];
  __shared__ __attribute__((aligned(16))) typename RStage<T>::E Rst[RStage<T>::N];
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * QB;
  const int tid = threadIdx.x;
  const int64_t ld = 3 * (int64_t)d;
  // stage K and V: rows t0 - HALO .. t0 + QB - 1, 8 elements per chunk; all
  // of a thread's loads are issued before its first LDS store
  constexpr int CH = ROWS * (HD / 8);
  constexpr int IT = (CH + NT - 1) / NT;
  Chunk8<T> kc[IT], vc[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NT;
    const int rr = idx / (HD / 8), c = (idx - rr * (HD / 8)) * 8;
    const int64_t t = t0 - HALO + rr;
    if (idx < CH && t >= 0 && t < n) {
      kc[it].load(qkv + t * ld + d + h * HD + c);
      vc[it].load(qkv + t * ld + 2 * d + h * HD + c);
    } else {
      kc[it].zero();
      vc[it].zero();
    }
  }
  // the token's query part and span: loaded before the staging stores so
  // their latency overlaps them
  const int qi = tid >> 2, part = tid & 3;
  const int64_t t = t0 + qi;
  const bool valid = t < n;
  const int c0 = part * DPL;
  Chunk8<T> qc[DPL / 8];
  {
    const T* qp = qkv + (valid ? t : 0) * ld + h * HD + c0;
#pragma unroll
    for (int i = 0; i < DPL / 8; ++i) qc[i].load(qp + 8 * i);
  }
  const int span = valid ? min(pos[t] + 1, left) : 1;
  bf16* Rb = (bf16*)Rst;
  float* Rs = (float*)Rst;
  for (int idx = tid; idx < MAXL * HD / 4; idx += NT) {
    const int dist = idx / (HD / 4), c = (idx - dist * (HD / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (dist < left) v = *(const float4*)(R + (int64_t)dist * d + h * HD + c);
    if constexpr (kBf) {
      bf16* dst = &Rb[dist * RROW_B + (c / DPL) * RPART_B + c % DPL];
      dst[0] = (bf16)v.x; dst[1] = (bf16)v.y; dst[2] = (bf16)v.z; dst[3] = (bf16)v.w;
    } else {
      *(float4*)&Rs[dist * RROW + (c / DPL) * RPART + c % DPL] = v;
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NT;
    if (idx < CH) {
      const int rr = idx / (HD / 8), c = (idx - rr * (HD / 8)) * 8;
      kc[it].store(&Ks[rr * LD + c]);
      vc[it].store(&Vs[rr * LD + c]);
    }
  }
  __syncthreads();

  float s[MAXL];
  if constexpr (kBf) {
    const uint32_t* qw = (const uint32_t*)qc;  // 16 packed pairs
#pragma unroll
    for (int dist = 0; dist < MAXL; ++dist) {
      const uint4* kr = (const uint4*)&Ks[(qi + HALO - dist) * LD + c0];
      const uint4* rr = (const uint4*)&Rb[dist * RROW_B + part * RPART_B];
      float ak = 0.f, ar = 0.f;
#pragma unroll
      for (int j = 0; j < DPL / 8; ++j) {
        const uint4 kv = kr[j], rv = rr[j];
        ak = dot2(qw[4 * j], kv.x, ak);
        ak = dot2(qw[4 * j + 1], kv.y, ak);
        ak = dot2(qw[4 * j + 2], kv.z, ak);
        ak = dot2(qw[4 * j + 3], kv.w, ak);
        ar = dot2(qw[4 * j], rv.x, ar);
        ar = dot2(qw[4 * j + 1], rv.y, ar);
        ar = dot2(qw[4 * j + 2], rv.z, ar);
        ar = dot2(qw[4 * j + 3], rv.w, ar);
      }
      s[dist] = ak + ar;
    }
  } else {
    float q[DPL];
#pragma unroll
    for (int i = 0; i < DPL / 8; ++i) {
      const float* qf = (const float*)&qc[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[8 * i + e] = qf[e];
    }
#pragma unroll
    for (int dist = 0; dist < MAXL; ++dist) {
      const T* kr = &Ks[(qi + HALO - dist) * LD + c0];
      const float* rr = &Rs[dist * RROW + part * RPART];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; i += 8) {
        float kv[8];
        load8(kr + i, kv);
        const float4 r0 = *(const float4*)(rr + i), r1 = *(const float4*)(rr + i + 4);
        acc += q[i] * (kv[0] + r0.x) + q[i + 1] * (kv[1] + r0.y) + q[i + 2] * (kv[2] + r0.z) +
               q[i + 3] * (kv[3] + r0.w) + q[i + 4] * (kv[4] + r1.x) + q[i + 5] * (kv[5] + r1.y) +
               q[i + 6] * (kv[6] + r1.z) + q[i + 7] * (kv[7] + r1.w);
      }
      s[dist] = acc;
    }
  }
  // full logits in all four lanes of the token (the quad of lanes)
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) s[dist] = quad_sum(s[dist]);
  // soft cap: cap tanh(s / cap), tanh(x) = 1 - 2 / (e^{2x} + 1) (e^{2x}
  // overflowing to inf gives 1, underflowing to 0 gives -1)
  const float two_over_cap = 2.0f / cap;
  float mx = -INFINITY;
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(s[dist] * two_over_cap) + 1.0f);
    s[dist] = dist < span ? cap * t : -INFINITY;
    mx = fmaxf(mx, s[dist]);
  }
  float den = 0.f;
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    s[dist] = dist < span ? __expf(s[dist] - mx) : 0.f;
    den += s[dist];
  }
  const float rden = __builtin_amdgcn_rcpf(den);
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    const float pd = s[dist] * rden;
    const T* vr = &Vs[(qi + HALO - dist) * LD + c0];
#pragma unroll
    for (int i = 0; i < DPL; i += 8) {
      float vv[8];
      load8(vr + i, vv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i + e] += pd * vv[e];
    }
  }
  if (valid) {
    T* op = o + t * d + h * HD + c0;
#pragma unroll
    for (int i = 0; i < DPL; i += 8) {
      float ov[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = clampf(acc[i + e], lo, hi);
      store8(op + i, ov);
    }
  }
}

}  // namespace

hipError_t launch_attention(ae_dtype dt, const void* qkv, const float* R, const int32_t* pos,
                            int64_t n, int d, int heads, int left, float softcap, float lo,
                            float hi, void* o, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d != heads * HD || left > MAXL || left < 1) return hipErrorInvalidValue;
  // bf16: 128 tokens a block (eight wavefronts, 79.5 KB of LDS, two blocks
  // per CU): 62.2 against 63.6 us for 64-token blocks (halo rows 11 of 139
  // instead of 11 of 75)
  constexpr int QB = 128;
  const dim3 grid((unsigned)((n + QB - 1) / QB), heads);
  if (dt == AE_BF16)
    hipLaunchKernelGGL((k_attn<bf16, QB, 2>), grid, dim3(4 * QB), 0, s, (const bf16*)qkv, R, pos, n,
                       d, left, softcap, lo, hi, (bf16*)o);
  else
    hipLaunchKernelGGL((k_attn<float, 64, 1>), dim3((unsigned)((n + 63) / 64), heads), dim3(256), 0, s, (const float*)qkv, R, pos, n,
                       d, left, softcap, lo, hi, (float*)o);
  return hipGetLastError();
}

}  // namespace ae
