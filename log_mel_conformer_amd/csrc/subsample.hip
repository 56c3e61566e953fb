// The subsampler in one pass for bf16 models (egemma2_audio.rs, module
// documentation step 3, AudioTower::subsample and layer_norm_relu): conv0
// (3x3 stride 2 from the log-mel plane to 128 channels, zero padding 1,
// LayerNorm over the channels with gain only, ReLU) and conv1 (3x3 stride 2,
// 128 -> 32 channels, the same LayerNorm and ReLU), flattened per token as
// [frequency][channel].
//
// A token needs conv0 rows 2 t - 1 .. 2 t + 1 of its clip (t its position),
// all 64 frequencies and 128 channels. A block walks `run` consecutive
// tokens in order and keeps those rows in a three-row ring in LDS (row r in slot
// r % 3), so the next token of the same clip computes only its two new
// rows; the 786 MB plane that separate kernels pass through HBM for 32
// clips of 30 s never leaves the CU. Per token:
//  - conv0: each new row is two 32-position units, one per wavefront,
//    each the matrix-core form of the separate conv0 kernel (the nine taps
//    against 128 channels as v_mfma_f32_32x32x16_bf16 with bf16 high and
//    low parts, the taps centred over the channels so the LayerNorm needs
//    only the variance), written into the ring as bf16;
//  - conv1: an implicit GEMM of 32 positions x 32 channels x 1152, each
//    wavefront a quarter of the k-steps with its weight fragments in
//    registers for the whole run and the position fragments gathered from
//    the ring; the four partial tiles meet in LDS, and each wavefront adds
//    them for 8 of the positions, normalises and stores them.
// Rows outside the clip (before it or past its last conv0 row) and
// frequencies outside 0 .. 63 are zero padding: masked where gathered.
#include <atomic>

#include "launch.h"

namespace ae {
namespace {

namespace sf {
constexpr int PB = kF1 * kC0 * 2;       // bytes of one conv0 row: 64 positions x 128 channels
constexpr int KS = kC0 * 9 / 16;        // conv1 k-steps of 16
constexpr int KSW = KS / 4;             // per wavefront
}  // namespace sf

// Byte offset of 8-channel chunk c of position p within a ring row: chunk
// c ^ ((p >> 1) & 15), so the 16 positions 2 f + const that one conv1
// fragment read serves (f consecutive) hit 16 distinct bank groups.
__device__ __forceinline__ int pchunk(int p, int c) { return p * 256 + ((c ^ ((p >> 1) & 15)) << 4); }

__device__ __forceinline__ f32x16 mfma16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ void __launch_bounds__(256, 2) k_subsample(
    const float* __restrict__ mel, const int64_t* __restrict__ frame_off,
    const int64_t* __restrict__ row_off, const int32_t* __restrict__ tok_pos,
    const int32_t* __restrict__ tok_clip, int64_t n_tok, int run, const uint4* __restrict__ frag0,
    const float* __restrict__ g0, const bf16* __restrict__ w1, const float* __restrict__ g1,
    bf16* __restrict__ x1) {
  using namespace sf;
  __shared__ __attribute__((aligned(16))) unsigned char ring[3 * PB];
  __shared__ __attribute__((aligned(16))) float part[4][64][16];
  __shared__ __attribute__((aligned(16))) float gs0[kC0];
  __shared__ __attribute__((aligned(16))) float gs1[kC1];
  __shared__ __attribute__((aligned(16))) uint4 wfs[8 * 64];  // conv0 tap fragments
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = lane & 31, h = lane >> 5;
  for (int i = tid; i < kC0; i += 256) gs0[i] = g0[i];
  if (tid < kC1) gs1[tid] = g1[tid];
  // conv0's first-operand fragments (4 channel tiles x 2 k-steps, lane
  // order) in LDS
  for (int i = tid; i < 8 * 64; i += 256) wfs[i] = frag0[i];
  // this wavefront's conv1 weight fragments (output channel p, k 16 ks +
  // 8 h ..) in registers for the whole run
  uint4 bw[KSW];
#pragma unroll
  for (int i = 0; i < KSW; ++i)
    bw[i] = *(const uint4*)(w1 + (size_t)p * (kC0 * 9) + 16 * (KSW * wave + i) + 8 * h);
  __syncthreads();

  // A token's conv0 work (uniform): its clip, position, the clip's conv0
  // rows and frames, and the rows lo .. lo + n - 1 it adds to the ring
  // (those of 2 tp - 1 .. 2 tp + 1 that exist and are not there yet). Unit
  // u = (row lo + u / 2, half u % 2) goes to wavefront u % 4, at most two
  // units each; a unit's nine log-mel inputs per lane are fetched one token
  // ahead, raw (from clamped addresses), and masked where used.
  struct Work {
    int cl, tp, T0, F, lo, n;
    int64_t fb;
  };
  int have_clip = -1, have_hi = -1;  // the ring holds rows .. have_hi of clip have_clip
  auto plan = [&](int64_t t) {
    Work q;
    q.cl = tok_clip[t];
    q.tp = tok_pos[t];
    const int64_t r0 = row_off[q.cl];
    q.T0 = (int)(row_off[q.cl + 1] - r0);
    q.fb = frame_off[q.cl];
    q.F = (int)(frame_off[q.cl + 1] - q.fb);
    int lo = max(2 * q.tp - 1, 0);
    if (q.cl == have_clip) lo = max(lo, have_hi + 1);
    const int hi = min(2 * q.tp + 1, q.T0 - 1);
    q.lo = lo;
    q.n = hi >= lo ? hi - lo + 1 : 0;
    if (q.n > 0) {
      if (q.cl != have_clip) have_hi = -1;
      have_clip = q.cl;
      have_hi = max(have_hi, hi);
    }
    return q;
  };
  auto fetch = [&](const Work& q, float (&xr)[2][9]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = wave + 4 * k;
      if (u < 2 * q.n) {
        const int row = q.lo + (u >> 1), f = (u & 1) * 32 + p;
#pragma unroll
        for (int dt = 0; dt < 3; ++dt)
#pragma unroll
          for (int df = 0; df < 3; ++df) {
            const int fi = 2 * row + dt - 1, bi = 2 * f + df - 1;
            xr[k][dt * 3 + df] =
                mel[(q.fb + min(max(fi, 0), q.F - 1)) * kMels + min(max(bi, 0), kMels - 1)];
          }
      }
    }
  };
  const int64_t t_first = (int64_t)blockIdx.x * run;
  const int64_t t_end = t_first + run < n_tok ? t_first + run : n_tok;
  float xr[2][9], xn[2][9];
  Work cur = plan(t_first);
  fetch(cur, xr);
  for (int64_t t = t_first; t < t_end; ++t) {
    const int tp = cur.tp, T0 = cur.T0;
    for (int ku = 0; ku < 2; ++ku) {
      const int u = wave + 4 * ku;
      if (u >= 2 * cur.n) break;
      const int row = cur.lo + (u >> 1);
      const int f = (u & 1) * 32 + p;
      // the position's nine log-mel inputs (frames 2 row - 1 .. 2 row + 1,
      // bins 2 f - 1 .. 2 f + 1, zero outside the clip and the bins), split
      // into bf16 high and low parts
      float x[9];
#pragma unroll
      for (int dt = 0; dt < 3; ++dt)
#pragma unroll
        for (int df = 0; df < 3; ++df) {
          const int fi = 2 * row + dt - 1, bi = 2 * f + df - 1;
          const bool ok = fi >= 0 && fi < cur.F && bi >= 0 && bi < kMels;
          x[dt * 3 + df] = ok ? (ku == 0 ? xr[0][dt * 3 + df] : xr[1][dt * 3 + df]) : 0.f;
        }
      bf16 ph[9], pl[9];
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        ph[k] = (bf16)x[k];
        pl[k] = (bf16)(x[k] - (float)ph[k]);
      }
      // slot k of the position operand: high, low, high of the taps, zero
      // from 27 on (the tap fragments hold high, high, low)
      auto slot = [&](int k) -> bf16 {
        if (k >= 27) return (bf16)0.f;
        const int term = k / 9, tap = k - 9 * term;
        return term == 1 ? pl[tap] : ph[tap];
      };
      bf16x8 a0, a1, b0, b1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a0[i] = slot(i);
        b0[i] = slot(8 + i);
        a1[i] = slot(16 + i);
        b1[i] = slot(24 + i);
      }
      const uint4 x0 = __builtin_bit_cast(uint4, h ? b0 : a0);
      const uint4 xk1 = __builtin_bit_cast(uint4, h ? b1 : a1);
      f32x16 acc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[ct] = f32x16{};
        acc[ct] = mfma16(wfs[(ct * 2) * 64 + lane], x0, acc[ct]);
        acc[ct] = mfma16(wfs[(ct * 2 + 1) * 64 + lane], xk1, acc[ct]);
      }
      // acc[ct][v]: centred output of channel 32 ct + 8 (v / 4) + 4 h + v % 4
      float q = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) q += acc[ct][v] * acc[ct][v];
      q += __shfl_xor(q, 32, 64);
      const float inv = rsqrtf(q * (1.0f / kC0) + kEps);
      // the gains are read here, not hoisted next to the accumulators (64
      // more live registers next to the run's conv1 weights would spill)
      asm volatile("" ::: "memory");
      unsigned char* dst = ring + (row % 3) * PB;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ch = ct * 32 + j * 8 + h * 4;
          const float4 g = *(const float4*)&gs0[ch];
          const bf16x4 o = {(bf16)fmaxf(acc[ct][4 * j] * inv * g.x, 0.f),
                            (bf16)fmaxf(acc[ct][4 * j + 1] * inv * g.y, 0.f),
                            (bf16)fmaxf(acc[ct][4 * j + 2] * inv * g.z, 0.f),
                            (bf16)fmaxf(acc[ct][4 * j + 3] * inv * g.w, 0.f)};
          *(bf16x4*)(dst + pchunk(f, ch >> 3) + 8 * h) = o;
        }
    }
    // the next token's inputs are on their way while this one finishes
    Work nxt = cur;
    if (t + 1 < t_end) {
      nxt = plan(t + 1);
      fetch(nxt, xn);
    }
    __syncthreads();  // the token's rows are in the ring

    // conv1, this wavefront's k-steps: k = (dt * 3 + df) * 128 + channel,
    // the position operand gathered from ring rows 2 tp - 1 + dt
    f32x16 acc1 = {};
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      const int ks = KSW * wave + i;
      const int tap = ks >> 3, dt = tap / 3, df = tap - 3 * dt;
      const int row = 2 * tp - 1 + dt, pos = 2 * p + df - 1;
      const bool ok = row >= 0 && row < T0 && pos >= 0;
      const uint4 a = *(const uint4*)(ring + (row < 0 ? 0 : row % 3) * PB +
                                      pchunk(pos < 0 ? 0 : pos, 2 * (ks & 7) + h));
      acc1 = mfma16(bw[i], ok ? a : make_uint4(0u, 0u, 0u, 0u), acc1);
      // at most six gathers in flight: hoisting all eighteen would spill
      if (i % 6 == 5) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(float4*)&part[wave][lane][4 * g] =
          make_float4(acc1[4 * g], acc1[4 * g + 1], acc1[4 * g + 2], acc1[4 * g + 3]);
    __syncthreads();  // the partial tiles are in LDS
    {
      // every wavefront finishes 8 of the 32 positions: lane l takes
      // position 8 wave + l / 8 and channels 4 (l % 8) .. + 3, which a
      // partial tile holds in lane position + 32 ((l / 2) % 2) at elements
      // 4 ((l % 8) / 2) .. + 3; the position's 32 channels are the 8 lanes
      // of its group
      const int pos = 8 * wave + (lane >> 3), cq = lane & 7;
      const int src = pos + 32 * (cq & 1), e0 = 4 * (cq >> 1);
      const float4 a = *(const float4*)&part[0][src][e0];
      const float4 b = *(const float4*)&part[1][src][e0];
      const float4 c = *(const float4*)&part[2][src][e0];
      const float4 e = *(const float4*)&part[3][src][e0];
      const float y[4] = {(a.x + b.x) + (c.x + e.x), (a.y + b.y) + (c.y + e.y),
                          (a.z + b.z) + (c.z + e.z), (a.w + b.w) + (c.w + e.w)};
      float sum = (y[0] + y[1]) + (y[2] + y[3]);
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      sum += __shfl_xor(sum, 4, 64);
      const float mean = sum * (1.0f / kC1);
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) q += (y[i] - mean) * (y[i] - mean);
      q += __shfl_xor(q, 1, 64);
      q += __shfl_xor(q, 2, 64);
      q += __shfl_xor(q, 4, 64);
      const float inv = rsqrtf(q * (1.0f / kC1) + kEps);
      const float4 g = *(const float4*)&gs1[4 * cq];
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 o = {(bf16)fmaxf((y[0] - mean) * inv * g.x, 0.f),
                        (bf16)fmaxf((y[1] - mean) * inv * g.y, 0.f),
                        (bf16)fmaxf((y[2] - mean) * inv * g.z, 0.f),
                        (bf16)fmaxf((y[3] - mean) * inv * g.w, 0.f)};
      *(bf16x4*)(x1 + t * (kF2 * kC1) + pos * kC1 + 4 * cq) = o;
    }
    cur = nxt;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 9; ++i) xr[k][i] = xn[k][i];
  }
}

}  // namespace

hipError_t launch_subsample_fused(const float* mel, const int64_t* frame_off,
                                  const int64_t* row_off, const int32_t* tok_pos,
                                  const int32_t* tok_clip, int64_t n_tok, const void* w0_frag,
                                  const float* g0, const void* w1, const float* g1, void* x1,
                                  hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  // One round of blocks, two per CU, each walking an equal run of tokens:
  // for 24000 tokens 48 a block took 217 us, against 226 for 16, 240 for 8
  // and 257 for 32 (1.5 rounds of the CUs)
  static std::atomic<int> cus[64];  // per device, 0 until first asked
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n_cu = cus[dev].load(std::memory_order_relaxed);
  if (n_cu == 0) {
    int v = 0;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    n_cu = v > 0 ? v : 1;
    cus[dev].store(n_cu, std::memory_order_relaxed);
  }
  const int64_t slots = 2 * (int64_t)n_cu;
  const int run = (int)((n_tok + slots - 1) / slots);
  const unsigned grid = (unsigned)((n_tok + run - 1) / run);
  hipLaunchKernelGGL(k_subsample, dim3(grid), dim3(256), 0, s, mel, frame_off, row_off, tok_pos,
                     tok_clip, n_tok, run, (const uint4*)w0_frag, g0, (const bf16*)w1, g1,
                     (bf16*)x1);
  return hipGetLastError();
}

}  // namespace ae
