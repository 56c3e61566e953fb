// Local attention core (egemma2_audio.rs, module documentation step 4 and
// AudioTower::attention): token t of head h attends to the tokens
// t - d, d < span = min(pos[t] + 1, left), of its own clip; the logit is
// q_t . k_{t-d} + q_t . R[d] (R the relative key of distance d), capped as
// softcap * tanh(logit / softcap), and the output is the softmax-weighted
// sum of v_{t-d}. q and k arrive already scaled by the projection epilogue;
// R arrives in the storage type.
#include "launch.h"
#include "lds_dma.h"

namespace ae {
namespace {

constexpr int HD = 128;         // head dim
constexpr int MAXL = 12;        // largest window these kernels serve
constexpr int HALO = MAXL - 1;

// fp32 storage (the parity path): one block per (64 consecutive tokens,
// head). The K and V rows those tokens can reach (64 + left - 1 of them)
// are staged in LDS (16-byte loads, all issued before the stores; rows
// padded to spread banks), R[0..left) of the head with each 32-dimension
// part padded to a 36-float pitch, so the parts the four lanes of a token
// read start on distinct banks. Four lanes serve one token, 32 of the 128
// dimensions each: a lane forms its partial logits for every distance, two
// cross-lane steps give all four lanes the full logits, each lane runs the
// (identical) softmax, then accumulates its 32 output dimensions. Rows
// before the buffer or past its end are staged as zeros and masked out, so
// no uninitialised value can reach the weighted sum.
namespace f32k {
constexpr int QB = 64;
constexpr int DPL = 32;          // dimensions per lane
constexpr int LD = HD + 4;       // floats per staged K / V row
constexpr int RPART = DPL + 4;   // floats per staged R part
constexpr int RROW = 4 * RPART;
}  // namespace f32k

__global__ void __launch_bounds__(4 * f32k::QB) k_attn_f32(
    const float* __restrict__ qkv, const float* __restrict__ R, const int32_t* __restrict__ pos,
    int64_t n, int d, int left, float cap, float lo, float hi, float* __restrict__ o) {
  using namespace f32k;
  constexpr int NT = 4 * QB;  // threads: four lanes per token
  constexpr int ROWS = QB + HALO;
  __shared__ __attribute__((aligned(16))) float Ks[ROWS * LD];
  __shared__ __attribute__((aligned(16))) float Vs[ROWS * LD];
  __shared__ __attribute__((aligned(16))) float Rs[MAXL * RROW];
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * QB;
  const int tid = threadIdx.x;
  const int64_t ld = 3 * (int64_t)d;
  // stage K and V: rows t0 - HALO .. t0 + QB - 1, 8 floats per chunk; all
  // of a thread's loads are issued before its first LDS store
  constexpr int CH = ROWS * (HD / 8);
  constexpr int IT = (CH + NT - 1) / NT;
  float4 kc[IT][2], vc[IT][2];
  const float4 zf = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NT;
    const int rr = idx / (HD / 8), c = (idx - rr * (HD / 8)) * 8;
    const int64_t t = t0 - HALO + rr;
    if (idx < CH && t >= 0 && t < n) {
      const float* kp = qkv + t * ld + d + h * HD + c;
      const float* vp = qkv + t * ld + 2 * d + h * HD + c;
      kc[it][0] = *(const float4*)kp;
      kc[it][1] = *(const float4*)(kp + 4);
      vc[it][0] = *(const float4*)vp;
      vc[it][1] = *(const float4*)(vp + 4);
    } else {
      kc[it][0] = kc[it][1] = vc[it][0] = vc[it][1] = zf;
    }
  }
  // the token's query part and span: loaded before the staging stores so
  // their latency overlaps them
  const int qi = tid >> 2, part = tid & 3;
  const int64_t t = t0 + qi;
  const bool valid = t < n;
  const int c0 = part * DPL;
  float q[DPL];
  {
    const float* qp = qkv + (valid ? t : 0) * ld + h * HD + c0;
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const float4 v = *(const float4*)(qp + i);
      q[i] = v.x; q[i + 1] = v.y; q[i + 2] = v.z; q[i + 3] = v.w;
    }
  }
  const int span = valid ? min(pos[t] + 1, left) : 1;
  for (int idx = tid; idx < MAXL * HD / 4; idx += NT) {
    const int dist = idx / (HD / 4), c = (idx - dist * (HD / 4)) * 4;
    float4 v = zf;
    if (dist < left) v = *(const float4*)(R + (int64_t)dist * d + h * HD + c);
    *(float4*)&Rs[dist * RROW + (c / DPL) * RPART + c % DPL] = v;
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NT;
    if (idx < CH) {
      const int rr = idx / (HD / 8), c = (idx - rr * (HD / 8)) * 8;
      *(float4*)&Ks[rr * LD + c] = kc[it][0];
      *(float4*)&Ks[rr * LD + c + 4] = kc[it][1];
      *(float4*)&Vs[rr * LD + c] = vc[it][0];
      *(float4*)&Vs[rr * LD + c + 4] = vc[it][1];
    }
  }
  __syncthreads();

  float s[MAXL];
#pragma unroll
  for (int dist = 0; dist < MAXL; ++dist) {
    const float* kr = &Ks[(qi + HALO - dist) * LD + c0];
    const float* rr = &Rs[dist * RROW + part * RPART];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; i += 8) {
      const float4 k0 = *(const float4*)(kr + i), k1 = *(const float4*)(kr + i + 4);
      const float4 r0 = *(const float4*)(rr + i), r1 = *(const float4*)(rr + i + 4);
      acc += q[i] * (k0.x + r0.x) + q[i + 1] * (k0.y + r0.y) + q[i + 2] * (k0.z + r0.z) +
             q[i + 3] * (k0.w + r0.w) + q[i + 4] * (k1.x + r1.x) + q[i + 5] * (k1.y + r1.y) +
             q[i + 6] * (k1.z + r1.z) + q[i + 7] * (k1.w + r1.w);
    }
    s[dist] = acc;
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
    const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(s[dist] * two_over_cap) + 1.0f);
    s[dist] = dist < span ? cap * th : -INFINITY;
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
    const float* vr = &Vs[(qi + HALO - dist) * LD + c0];
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const float4 v = *(const float4*)(vr + i);
      acc[i] += pd * v.x;
      acc[i + 1] += pd * v.y;
      acc[i + 2] += pd * v.z;
      acc[i + 3] += pd * v.w;
    }
  }
  if (valid) {
    float* op = o + t * d + h * HD + c0;
#pragma unroll
    for (int i = 0; i < DPL; i += 4)
      *(float4*)(op + i) = make_float4(clampf(acc[i], lo, hi), clampf(acc[i + 1], lo, hi),
                                       clampf(acc[i + 2], lo, hi), clampf(acc[i + 3], lo, hi));
  }
}

// bf16 storage: the logits on the matrix cores (v_mfma_f32_32x32x16_bf16),
// the weighted sum on the vector units. One block per (128 consecutive
// tokens, head), one wavefront per 32 tokens.
//  - staging: the head's K rows t0 - 16 .. t0 + 143 and R's first 16 rows
//    go into LDS, and each wavefront's 32 Q rows into its own region, by
//    buffer loads that write LDS directly (1 KB = four 256-byte rows per
//    instruction). A row's 16-byte chunk c sits at chunk c ^ (row & 15), so
//    the 16 rows one read serves hit 16 distinct bank groups;
//  - logits: S = K Q^T over keys q0 - 16 .. q0 + 47 (q0 the wavefront's
//    first token) and Srel = R Q^T over the distances. The operand order
//    leaves a lane with one token's values: lane l holds token l % 32 and
//    keys (or distances) 8 (v / 4) + 4 (l / 32) + v % 4 of its accumulator
//    element v;
//  - the band: S goes to LDS and each lane reads back its token's logits at
//    key t - dist for the eight distances its Srel elements hold (lanes
//    32-63 hold distances 4-7 and 12-15, the last four always masked), adds
//    q.R[dist], caps, and takes the softmax together with lane l ^ 32;
//  - output: V rows t0 - 16 .. t0 + 127 replace K in LDS (staged the same
//    way, after every wavefront's logits; loading V into registers at the
//    start instead measured 63 against 43 us a layer). Each lane sums 64
//    dimensions of its token over the distances with packed dot products
//    (two distances each, probabilities rounded to bf16) in a fixed order.
//    A third product P V^T on the matrix cores measured 43.0 against 48.5
//    us a layer, but it groups a token's keys into 16-key steps by the
//    token's place in the block, so a clip's output would change (by
//    rounding) with the clips packed before it; this form keeps every
//    clip's output bit-identical wherever it sits in a batch.
namespace mf {
constexpr int QB = 128;             // tokens per block
constexpr int NWAVE = QB / 32;      // one wavefront per 32 tokens
constexpr int KOFF = 16;            // staged rows start 16 keys before the block
constexpr int KROWS = QB + 32;      // K rows: every wavefront's 64 keys
constexpr int VROWS = QB + KOFF;    // V rows: keys q0 - 11 .. q0 + 31 of every wavefront
constexpr int RB = HD * 2;          // bytes per staged row
constexpr int SP = 68;              // floats per logit row
constexpr int OP = HD + 8;          // bf16 per staged output row
constexpr int WBYTES = 32 * SP * 4; // a wavefront's region: Q, then the logits, then the output
static_assert(32 * RB <= WBYTES && 32 * OP * 2 <= WBYTES, "regions overlay each other");
static_assert(KROWS % 16 == 0 && VROWS % 16 == 0, "four-row groups spread over the wavefronts");
}  // namespace mf

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// a.b over two packed bf16 pairs, plus c (float32 accumulation)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ f32x16 mfma16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// byte offset of 16-byte chunk c of staged row r
__device__ __forceinline__ int srow(int r, int c) { return r * mf::RB + ((c ^ (r & 15)) << 4); }

// Block b takes head b % heads of token block b / heads. Blocks are dealt
// to the eight XCDs in turn, so with eight heads every token block of one
// head runs on one XCD, whose L2 then serves the K and V rows a block
// shares with the block before it (47.5 against 49.3 us a layer with the
// token block as the fast index).
__global__ void __launch_bounds__(256, 2) k_attn_mfma(
    const bf16* __restrict__ qkv, const bf16* __restrict__ Rb, const int32_t* __restrict__ pos,
    int64_t n, int d, int left, float cap, float lo, float hi, bf16* __restrict__ o) {
  using namespace mf;
  __shared__ __attribute__((aligned(1024))) unsigned char X[(KROWS + 16) * RB];
  __shared__ __attribute__((aligned(1024))) unsigned char Wr[NWAVE * WBYTES];
  const int heads = d / HD;
  const int h = (int)(blockIdx.x % (unsigned)heads);
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)heads) * QB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hf = lane >> 5;
  const int64_t ld = 3 * (int64_t)d;
  const int64_t q0 = t0 + 32 * wave;
  const int64_t tq = q0 + r32;
  unsigned char* Ww = Wr + wave * WBYTES;

  // One buffer resource from row max(t0 - 16, 0) to the end of the buffer:
  // rows past n read zeros, rows before 0 take an offset past the range.
  const int64_t base = t0 - KOFF > 0 ? t0 - KOFF : 0;
  const uint64_t bytes = (uint64_t)(n - base) * ld * sizeof(bf16);
  const i32x4 rs = buffer_rsrc(qkv + base * ld, (uint32_t)(bytes < 0x7FFFFFF0ull ? bytes : 0x7FFFFFF0ull));
  // lane l of a four-row group: row l / 16, physical chunk l % 16
  const int gr = lane >> 4, pc = lane & 15;
  auto stage = [&](unsigned char* dst, int64_t row0, int g, int col) {
    const int lr = 4 * g + gr;  // row within the staged image
    const int64_t row = row0 + lr;
    const uint32_t off = row < base ? 0x80000000u
                                    : (uint32_t)((row - base) * ld * (int64_t)sizeof(bf16)) +
                                          (uint32_t)(col * (int)sizeof(bf16)) +
                                          (uint32_t)((pc ^ (lr & 15)) << 4);
    raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + g * 1024), 16, off, 0,
                        0, 0);
  };
#pragma unroll
  for (int i = 0; i < KROWS / 4 / NWAVE; ++i) stage(X, t0 - KOFF, wave + NWAVE * i, d + h * HD);
#pragma unroll
  for (int g = 0; g < 8; ++g) stage(Ww, q0, g, h * HD);
  // R's rows 0 .. 15 after K (rows from `left` on read zeros), one group of
  // four rows per wavefront
  {
    const i32x4 rr = buffer_rsrc(Rb, (uint32_t)(left * d * (int)sizeof(bf16)));
    const int lr = 4 * wave + gr;
    raw_buffer_load_lds(rr, (__attribute__((address_space(3))) void*)(X + KROWS * RB + wave * 1024),
                        16, (uint32_t)((lr * d + h * HD) * (int)sizeof(bf16)) +
                                (uint32_t)((pc ^ (lr & 15)) << 4),
                        0, 0, 0);
  }
  // the token's position, from an index clamped into the buffer (a load
  // whose destination an else branch overwrote would have to complete
  // before the branch)
  const int ptq = pos[tq < n ? tq : n - 1];
  const int span = tq < n ? min(ptq + 1, left) : 1;
  wait_vmcnt<0>();  // K, Q and R staged
  __syncthreads();

  f32x16 s0 = {}, s1 = {}, sr = {};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int c = 2 * ks + hf;
    const uint4 qf = *(const uint4*)(Ww + srow(r32, c));
    const uint4 k0 = *(const uint4*)(X + srow(32 * wave + r32, c));
    const uint4 k1 = *(const uint4*)(X + srow(32 * wave + 32 + r32, c));
    const uint4 rf = *(const uint4*)(X + KROWS * RB + srow(r32 & 15, c));
    s0 = mfma16(k0, qf, s0);
    s1 = mfma16(k1, qf, s1);
    sr = mfma16(rf, qf, sr);
  }
  // logits to the wavefront's region: row = token, column = key - (q0 - 16);
  // the band covers columns 1 .. 47
  float* Sw = (float*)Ww;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    *(float4*)&Sw[r32 * SP + 8 * g + 4 * hf] =
        make_float4(s0[4 * g], s0[4 * g + 1], s0[4 * g + 2], s0[4 * g + 3]);
    if (g < 2)
      *(float4*)&Sw[r32 * SP + 32 + 8 * g + 4 * hf] =
          make_float4(s1[4 * g], s1[4 * g + 1], s1[4 * g + 2], s1[4 * g + 3]);
  }
  wait_lgkmcnt0();
  __builtin_amdgcn_wave_barrier();
  // this lane's eight distances, capped, then the softmax over the token's
  // span with the partner lane
  const float two_over_cap = 2.0f / cap;
  float lg[8];
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int dist = 8 * (v >> 2) + 4 * hf + (v & 3);
    const float x = Sw[r32 * SP + r32 + KOFF - dist] + sr[v];
    const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(x * two_over_cap) + 1.0f);
    lg[v] = dist < span ? cap * th : -INFINITY;
    mx = fmaxf(mx, lg[v]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float den = 0.f;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int dist = 8 * (v >> 2) + 4 * hf + (v & 3);
    lg[v] = dist < span ? __expf(lg[v] - mx) : 0.f;
    den += lg[v];
  }
  den += __shfl_xor(den, 32);
  const float rden = __builtin_amdgcn_rcpf(den);
  // the token's twelve probabilities in both lanes (the partner holds the
  // other half), as bf16 pairs (distance 2j, 2j + 1)
  float own[8], oth[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    own[v] = lg[v] * rden;
    oth[v] = __shfl_xor(own[v], 32);
  }
  uint32_t pp[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    float pa[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int dist = 2 * j + e;  // held by lanes 0-31 as element v, or by lanes 32-63
      const int v = dist < 4 ? dist : dist - 4;
      const bool mine = (dist >> 2) == 1 ? hf == 1 : hf == 0;
      pa[e] = mine ? own[v] : oth[v];
    }
    const bf16x2 pv = {(bf16)pa[0], (bf16)pa[1]};
    pp[j] = __builtin_bit_cast(uint32_t, pv);
  }
  // every wavefront is past its K reads: V takes K's place
  __syncthreads();
#pragma unroll
  for (int i = 0; i < VROWS / 4 / NWAVE; ++i) stage(X, t0 - KOFF, wave + NWAVE * i, 2 * d + h * HD);
  wait_vmcnt<0>();
  __syncthreads();  // V staged

  // o = sum over distances of p_dist v_{t - dist}: this lane's 64 dimensions
  // (half hf of the head), two distances per packed dot product, always in
  // the same order, so a token's output does not depend on where its clip
  // sits in the batch
  float oacc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) oacc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int ra = 32 * wave + KOFF + r32 - 2 * j;  // V row of distance 2j
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 a = *(const uint4*)(X + srow(ra, 8 * hf + c));
      const uint4 b = *(const uint4*)(X + srow(ra - 1, 8 * hf + c));
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oacc[8 * c + 2 * e] = dot2(__builtin_amdgcn_perm(bw[e], aw[e], 0x05040100u), pp[j],
                                   oacc[8 * c + 2 * e]);
        oacc[8 * c + 2 * e + 1] = dot2(__builtin_amdgcn_perm(bw[e], aw[e], 0x07060302u), pp[j],
                                       oacc[8 * c + 2 * e + 1]);
      }
    }
  }
  // clamp, stage rows in the region, store whole rows
  bf16* Ow = (bf16*)Ww;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)clampf(oacc[8 * c + e], lo, hi);
    *(bf16x8*)&Ow[r32 * OP + 64 * hf + 8 * c] = v;
  }
  wait_lgkmcnt0();
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = it * 64 + lane;
    const int row = c >> 4, col = (c & 15) * 8;
    const int64_t t = q0 + row;
    if (t < n) *(uint4*)(o + t * d + h * HD + col) = *(const uint4*)&Ow[row * OP + col];
  }
}

}  // namespace

hipError_t launch_attention(ae_dtype dt, const void* qkv, const void* R, const int32_t* pos,
                            int64_t n, int d, int heads, int left, float softcap, float lo,
                            float hi, void* o, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (d != heads * HD || left > MAXL || left < 1) return hipErrorInvalidValue;
  if (dt == AE_BF16) {
    const int64_t blocks = (n + mf::QB - 1) / mf::QB * heads;
    if (blocks > (int64_t)(UINT32_MAX / 256)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_mfma, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16*)qkv,
                       (const bf16*)R, pos, n, d, left, softcap, lo, hi, (bf16*)o);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)((n + f32k::QB - 1) / f32k::QB), heads),
                     dim3(4 * f32k::QB), 0, s, (const float*)qkv, (const float*)R, pos, n, d, left,
                     softcap, lo, hi, (float*)o);
  return hipGetLastError();
}

}  // namespace ae
