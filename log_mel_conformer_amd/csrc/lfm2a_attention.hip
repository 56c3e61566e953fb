// Self-attention with the Transformer-XL relative-position term over whole
// clips (cera 0.5.3, audio_encoder_gpu.rs: the xl_attention op and the
// attention part of encode_audio_gpu): per head,
//   score(i, j) = ((q_i + u) . k_j + (q_i + v) . p[t_max - 1 - i + j]) / 8,
// softmax over the clip's keys, output sum_j softmax_ij v_j.
//
// The page's kernel holds a whole score row in workgroup memory, which caps
// the clip at 1024 tokens. Here a block takes 128 queries of one clip and
// head (four wavefronts of 32) and walks the keys 32 at a time with an
// online softmax, so the length is unbounded. All three products run on
// v_mfma_f32_32x32x16_bf16 with the query as the lane index of the
// accumulator (lane l: query l % 32; accumulator v: key, table row or
// output dimension (v / 4) * 8 + (l / 32) * 4 + v % 4):
//   S = K (q + u)^T, G = P (q + v)^T, O += V^T softmax^T.
// The position term needs row t_max - 1 - i + j of p for query i and key j,
// a different row per (i, j) diagonal. For the 32 queries of a wavefront
// and a 32-key step those rows span 63 consecutive table rows: the
// wavefront computes G for 32 new table rows per step, keeps the previous
// 32 in a two-slot LDS ring, and each lane reads its 16 (query, key)
// entries out of the ring along the diagonal. The table rows a wavefront
// needs at step s are the ones wavefront w - 1 needed at step s - 1, so
// the block loads one new 32-row tile of p per step into an NW-slot ring.
// A step's K, V and p tiles are fetched into registers during the step
// before it. Softmax probabilities feed the value product straight from
// registers: the key order inside each MFMA k-block is the one the lane
// already holds, and the transposed V tile is read in that same order.
#include <math.h>

#include "lfm2a_launch.h"

namespace ae {
namespace lfm {
namespace {

constexpr int NW = kQueriesPerBlock / 32;  // wavefronts per block
constexpr int KT = 32;   // keys per step
constexpr int KP = 72;   // bf16 pitch of K and p tile rows (144 B: conflict-free 16-byte reads)
constexpr int VP = 40;   // bf16 pitch of the transposed V tile
constexpr int GP = 36;   // float pitch of G rows

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void lds_sync_wave() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ void __launch_bounds__(NW * 64, 2) k_xl_attention(
    const bf16* __restrict__ qkv, const bf16* __restrict__ P, int64_t t_max,
    const float* __restrict__ bias_u, const float* __restrict__ bias_v,
    const int64_t* __restrict__ token_off, const int64_t* __restrict__ qtile_off, int B,
    bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vt[kHd * VP];
  __shared__ __attribute__((aligned(16))) bf16 Ps[NW][32 * KP];
  __shared__ __attribute__((aligned(16))) float Gs[NW][2][32 * GP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ii = lane & 31, hh = lane >> 5;
  const int head = blockIdx.y;
  const int clip = find_clip(qtile_off, B, blockIdx.x);
  const int i0 = (int)(blockIdx.x - qtile_off[clip]) * kQueriesPerBlock;
  const int64_t t0 = token_off[clip];
  const int t = (int)(token_off[clip + 1] - t0);
  const int qi = i0 + 32 * w + ii;
  constexpr int ld = 3 * kD;
  const int64_t p_rows = 2 * t_max - 1;

  // (q + u) and (q + v) fragments of this lane's query: dims 16 s + 8 hh + e
  bf16x8 qu[4], qv[4];
  {
    const bf16* qrow = qkv + (t0 + (qi < t ? qi : t - 1)) * ld + head * kHd;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = 16 * s + 8 * hh;
      const bf16x8 raw = *(const bf16x8*)(qrow + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = (float)raw[e];
        qu[s][e] = (bf16)(q + bias_u[head * kHd + d0 + e]);
        qv[s][e] = (bf16)(q + bias_v[head * kHd + d0 + e]);
      }
    }
  }

  // one 32-row tile of p: rows t_max - i0 + 32 m + r
  auto load_p = [&](int m) {
    const int pr = tid >> 3, pc = (tid & 7) * 8;
    const int64_t rho = t_max - i0 + 32 * (int64_t)m + pr;
    bf16x8 v = {};
    if (rho >= 0 && rho < p_rows) v = *(const bf16x8*)(P + rho * kD + head * kHd + pc);
    *(bf16x8*)(&Ps[(m + NW) % NW][pr * KP + pc]) = v;
  };
  // G[r][query] = p tile m row r . (q + v), into ring slot gslot
  auto compute_g = [&](int m, int gslot) {
    const bf16* pt = Ps[(m + NW) % NW];
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = mfma16(*(const bf16x8*)(pt + ii * KP + 16 * s + 8 * hh), qv[s], acc);
    float* gd = &Gs[w][gslot][ii * GP];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(float4*)(gd + g * 8 + 4 * hh) =
          make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
  };

  // the K, V and p tiles of a step, fetched into registers one step ahead
  // (the loads fly while the previous step computes) and then stored to LDS
  bf16x8 kreg, preg;
  bf16x4 va, vb;
  auto fetch = [&](int s) {
    const int kr = tid >> 3, kc = (tid & 7) * 8;
    const int j = s * KT + kr;
    kreg = bf16x8{};
    if (j < t) kreg = *(const bf16x8*)(qkv + (t0 + j) * ld + kD + head * kHd + kc);
    const int vp = tid >> 4, vd = (tid & 15) * 4;
    const int ja = s * KT + 2 * vp;
    va = bf16x4{};
    vb = bf16x4{};
    if (ja < t) va = *(const bf16x4*)(qkv + (t0 + ja) * ld + 2 * kD + head * kHd + vd);
    if (ja + 1 < t) vb = *(const bf16x4*)(qkv + (t0 + ja + 1) * ld + 2 * kD + head * kHd + vd);
    const int64_t rho = t_max - i0 + 32 * (int64_t)s + kr;
    preg = bf16x8{};
    if (rho >= 0 && rho < p_rows) preg = *(const bf16x8*)(P + rho * kD + head * kHd + kc);
  };
  auto stage = [&](int s) {
    const int kr = tid >> 3, kc = (tid & 7) * 8;
    *(bf16x8*)(&Ks[kr * KP + kc]) = kreg;
    *(bf16x8*)(&Ps[s % NW][kr * KP + kc]) = preg;
    const int vp = tid >> 4, vd = (tid & 15) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 pr = {va[e], vb[e]};
      *(bf16x2*)(&Vt[(vd + e) * VP + 2 * vp]) = pr;
    }
  };

  // prologue: the NW tiles before step 0's; each wavefront's first G slot
#pragma unroll
  for (int m = -NW; m < 0; ++m) load_p(m);
  fetch(0);
  __syncthreads();
  compute_g(-w - 1, 0);

  constexpr float kScaleLog2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[2] = {};
  const int nsteps = (t + KT - 1) / KT;
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();  // every read of the previous K, V and the p slot reused below is done
    stage(s);
    if (s + 1 < nsteps) fetch(s + 1);
    __syncthreads();
    // G for this step's new table tile and S for its keys: two independent
    // MFMA chains, interleaved
    f32x16 gacc = {}, sacc = {};
    {
      const bf16* pt = Ps[(s - w + NW) % NW];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        gacc = mfma16(*(const bf16x8*)(pt + ii * KP + 16 * k + 8 * hh), qv[k], gacc);
        sacc = mfma16(*(const bf16x8*)(&Ks[ii * KP + 16 * k + 8 * hh]), qu[k], sacc);
      }
      float* gd = &Gs[w][(s + 1) & 1][ii * GP];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(gd + g * 8 + 4 * hh) =
            make_float4(gacc[4 * g], gacc[4 * g + 1], gacc[4 * g + 2], gacc[4 * g + 3]);
    }
    lds_sync_wave();
    // this lane's 16 (query, key) entries of G along the diagonal: all
    // addresses are inside the ring, so every read is issued before the
    // key mask is applied
    const float* gA = &Gs[w][s & 1][ii * GP];
    const float* gB = &Gs[w][(s + 1) & 1][ii * GP];
    float g[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int o = (v >> 2) * 8 + 4 * hh + (v & 3) - ii + 31;
      g[v] = *(o < 32 ? gA + o : gB + (o - 32));
    }
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int jj = (v >> 2) * 8 + 4 * hh + (v & 3);
      // the mask as an addend keeps every G value live (no guarded reads)
      x[v] = fmaf(sacc[v] + g[v], kScaleLog2, s * KT + jj < t ? 0.0f : -INFINITY);
      mx = fmaxf(mx, x[v]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      oacc[0][v] *= corr;
      oacc[1][v] *= corr;
    }
    bf16x8 pf[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = exp2f(x[v] - m_new);
      l_run += p;
      pf[v >> 3][v & 7] = (bf16)p;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {  // the two output chains alternate
        const bf16* vr = &Vt[(32 * dt + ii) * VP + 16 * k + 4 * hh];
        const u32x2 lo = *(const u32x2*)vr, hi = *(const u32x2*)(vr + 8);
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
        oacc[dt] = mfma16(__builtin_bit_cast(bf16x8, a), pf[k], oacc[dt]);
      }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qi < t) {
    const float inv = 1.0f / l_tot;
    bf16* orow = out + (t0 + qi) * kD + head * kHd;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x4 v = {(bf16)(oacc[dt][4 * g] * inv), (bf16)(oacc[dt][4 * g + 1] * inv),
                          (bf16)(oacc[dt][4 * g + 2] * inv), (bf16)(oacc[dt][4 * g + 3] * inv)};
        *(bf16x4*)(orow + 32 * dt + g * 8 + 4 * hh) = v;
      }
  }
}

}  // namespace

hipError_t launch_xl_attention(const bf16* qkv, const bf16* p, int64_t t_max, const float* u,
                               const float* v, const int64_t* token_off,
                               const int64_t* qtile_off, int B, int64_t n_qtiles, bf16* o,
                               hipStream_t s) {
  if (n_qtiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_xl_attention, dim3((unsigned)n_qtiles, kHeads), dim3(NW * 64), 0, s, qkv,
                     p, t_max, u, v, token_off, qtile_off, B, o);
  return hipGetLastError();
}

}  // namespace lfm
}  // namespace ae
