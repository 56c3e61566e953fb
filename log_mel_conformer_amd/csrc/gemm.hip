// Projection GEMMs on CDNA4 matrix cores: C = epilogue(A B^T).
//
// Every projection of the tower is y = x W^T with W stored [out][in]
// (egemma2_audio.rs, ClipLin::apply and the subsampler's conv1 GEMM), so
// both operands are K-contiguous rows. A block stages BMx128-byte and
// BNx128-byte slices of A and B through double-buffered LDS (16-byte chunks,
// XOR-swizzled by row so the fragment reads of a wavefront hit distinct
// banks) and runs 32x32 MFMAs: v_mfma_f32_32x32x16_bf16 for bf16 operands,
// v_mfma_f32_32x32x2f32 for fp32 (four per 16-byte chunk pair). A lane's
// 16-byte fragment holds consecutive k; the two lane halves take
// consecutive chunks, and A and B use the same k assignment, so the sum
// over k is complete whatever order the unit walks it in.
//
// The epilogues fuse what follows each projection on the page: the output
// clamp of a clippable linear, SiLU plus the next projection's input clamp
// (feed-forward), the GLU of the light conv's linear_start, the output
// projection's bias, per-column q/k scaling, and conv1's channel
// LayerNorm + ReLU (the tower's residual adds run in the row kernels); for
// the LFM2A encoder (cera 0.5.3, audio_encoder_gpu.rs), the bias adds with
// ReLU, SiLU or erf GELU, the GLU with its bias, and the scaled residual
// adds of macaron_ffn. Float operands with K = 4096 split K over four
// blocks per tile and add the partial tiles in a second pass.
#include <type_traits>

#include "launch.h"
#include "lds_dma.h"

namespace ae {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int ROWB = 128;  // bytes of one tile row per k-step (8 chunks)

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static __device__ __forceinline__ void run(f32x16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// LDS image of a tile row: chunk c of row r sits at chunk c ^ ((r >> 1) & 7).
// The LDS has 64 four-byte banks (256 bytes), i.e. two 128-byte rows; a
// 16-byte fragment read serves 16 lanes (16 consecutive rows, one chunk
// index) per pass, and this XOR gives those 16 rows 16 distinct 16-byte
// bank groups.
__device__ __forceinline__ int swz(int row, int c) {
  return row * ROWB + ((c ^ ((row >> 1) & 7)) << 4);
}

template <typename TO> __device__ __forceinline__ void store_out(TO* C, size_t idx, float v) {
  C[idx] = from_f32<TO>(v);
}

// Four consecutive outputs of one row, as one 16-byte (float) or 8-byte
// (bf16) store.
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *(bf16x4*)p = v;
}

// The activations of EPI_ACT; GELU in its erf form.
__device__ __forceinline__ float act_apply(int act, float x) {
  if (act == ACT_RELU) return fmaxf(x, 0.0f);
  if (act == ACT_SILU) return x * sigmoidf_(x);
  if (act == ACT_GELU_ERF) return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  return x;
}

// Epilogue of a wavefront's tile at (row0, col0). The MFMAs take the B
// fragment as their first operand, so each 32x32 accumulator holds the
// transposed sub-tile: acc[i][j][v] is C at row row0 + 32 i + lane % 32 and
// column col0 + 32 j + (v / 4) * 8 + (lane / 32) * 4 + v % 4. A lane thus
// owns four runs of four consecutive columns of one row per sub-tile, which
// it writes as vector stores.
template <typename TO, int MT, int NTL, int EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x16 (&acc)[MT][NTL], int row0,
                                         int col0, int seg, int lane) {
  TO* C = (TO*)p.C;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = row0 + i * 32 + r;
    const bool ok = row < p.M;
    TO* crow = C + (size_t)(ok ? row : 0) * p.ldc;
    if (EPI == EPI_GLU) {
      const float lo = p.olo[0], hi = p.ohi[0];
#pragma unroll
      for (int jp = 0; jp < NTL / 2; ++jp)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = col0 / 2 + jp * 32 + g * 8 + h * 4;
          float ba[4] = {0.f, 0.f, 0.f, 0.f}, bb[4] = {0.f, 0.f, 0.f, 0.f};
          if (p.bias) {  // 16-byte loads of the a and b halves' biases
            const float4 va = *(const float4*)(p.bias + col);
            const float4 vb = *(const float4*)(p.bias + p.glu_d + col);
            ba[0] = va.x; ba[1] = va.y; ba[2] = va.z; ba[3] = va.w;
            bb[0] = vb.x; bb[1] = vb.y; bb[2] = vb.z; bb[3] = vb.w;
          }
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float a = clampf(acc[i][2 * jp][4 * g + e], lo, hi);
            float b = clampf(acc[i][2 * jp + 1][4 * g + e], lo, hi);
            if (p.bias) {
              a += ba[e];
              b += bb[e];
            }
            o[e] = a * sigmoidf_(b);
          }
          if (ok) store4(crow + col, o[0], o[1], o[2], o[3]);
        }
    } else if (EPI == EPI_LNRELU) {
      // the row's 32 channels: 16 in this lane, 16 in lane ^ 32
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) sum += acc[i][0][v];
      sum += __shfl_xor(sum, 32, 64);
      const float mean = sum * (1.0f / 32);
      float q = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float dx = acc[i][0][v] - mean;
        q += dx * dx;
      }
      q += __shfl_xor(q, 32, 64);
      const float inv = rsqrtf(q * (1.0f / 32) + kEps);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = g * 8 + h * 4;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = fmaxf((acc[i][0][4 * g + e] - mean) * inv * p.gain[col + e], 0.0f);
        if (ok) store4(crow + col, o[0], o[1], o[2], o[3]);
      }
    } else {
      const float lo = p.olo[seg], hi = p.ohi[seg];
#pragma unroll
      for (int j = 0; j < NTL; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = col0 + j * 32 + g * 8 + h * 4;
          float x[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]};
          if (EPI == EPI_STORE) {
            float4 sc = make_float4(1.f, 1.f, 1.f, 1.f);
            if (p.colscale) sc = *(const float4*)(p.colscale + col);
            if (ok)
              store4(crow + col, clampf(x[0], lo, hi) * sc.x, clampf(x[1], lo, hi) * sc.y,
                     clampf(x[2], lo, hi) * sc.z, clampf(x[3], lo, hi) * sc.w);
          } else if (EPI == EPI_SILU) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float y = clampf(x[e], lo, hi);
              o[e] = clampf(y * sigmoidf_(y), p.nlo, p.nhi);
            }
            if (ok) store4(crow + col, o[0], o[1], o[2], o[3]);
          } else if (EPI == EPI_RESID) {
            float* hp = (float*)crow + col;
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = clampf(x[e], lo, hi);
            if (p.bias) {
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (o[e] + p.bias[col + e]) * p.rscale;
            }
            if (ok) {
              const float4 hv = *(const float4*)hp;
              store4(hp, hv.x + o[0], hv.y + o[1], hv.z + o[2], hv.w + o[3]);
            }
          } else if (EPI == EPI_ACT) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[e] = act_apply(p.act, x[e] + (p.bias ? p.bias[col + e] : 0.0f));
            if (ok) store4(crow + col, o[0], o[1], o[2], o[3]);
          } else if (EPI == EPI_BIAS) {
            const float4 bv = *(const float4*)(p.bias + col);
            if (ok) store4((float*)crow + col, x[0] + bv.x, x[1] + bv.y, x[2] + bv.z, x[3] + bv.w);
          }
        }
    }
  }
}

// Four values to or from LDS as one access (8 bytes of bf16, 16 of float).
__device__ __forceinline__ void put4(unsigned char* p, const float* o) {
  *(float4*)p = make_float4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ void put4_bf16(unsigned char* p, const float* o) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v = {(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
  *(bf16x4*)p = v;
}
template <typename TS> __device__ __forceinline__ void put4s(unsigned char* p, const float* o) {
  if (std::is_same<TS, float>::value) put4(p, o);
  else put4_bf16(p, o);
}
template <typename TS> __device__ __forceinline__ void get4s(const unsigned char* p, float* o) {
  if (std::is_same<TS, float>::value) {
    const float4 v = *(const float4*)p;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (float)v[e];
  }
}

// LDS bytes of one 32-row slab per wavefront row in the staged epilogue; a
// kernel whose stage ring is smaller than that gets the larger LDS array.
template <typename TO, int EPI, int BN, int WM>
constexpr int staged_slab_bytes() {
  constexpr int es = EPI == EPI_RESID ? 4 : (int)sizeof(TO);
  constexpr int outn = EPI == EPI_GLU ? BN / 2 : BN;
  return WM * 32 * (outn * es + 4 * es);
}

constexpr int staged_slabs(int mt, int slab, int ldsb) {
  int best = 1;
  for (int s = 1; s <= mt; ++s)
    if (mt % s == 0 && s * slab <= ldsb) best = s;
  return best;
}

// Epilogue of a k_gemm_dl tile, staged through the (then idle) LDS. From
// the accumulators a lane owns four consecutive columns of 32 different
// rows per store, which reaches the L2 as partial-line writes from every CU
// at once. Instead, every wavefront writes its epilogue values into a
// row-major LDS image of SPI 32-row slabs (pitch padded by one access, so
// the 32 rows of a write land in distinct banks), and after a barrier the
// block stores whole rows, consecutive lanes on consecutive bytes. The
// light conv's residual add happens in that second phase, so the residual
// is read with the same row-contiguous pattern. Values match the direct
// epilogue exactly (same arithmetic, same rounding points).
template <typename TO, int BM, int BN, int WM, int WN, int EPI, int LDSB>
__device__ __forceinline__ void epilogue_staged(const GemmParams& p,
                                                f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                                                unsigned char* smem, int m0, int n0, int wm,
                                                int wn, int seg, int wave, int lane) {
  constexpr int NW = WM * WN, WTM = BM / WM, WTN = BN / WN, MT = WTM / 32, NTL = WTN / 32;
  constexpr bool GLU = EPI == EPI_GLU;
  constexpr int OUTN = GLU ? BN / 2 : BN, WOUT = OUTN / WN;
  using TS = typename std::conditional<EPI == EPI_RESID, float, TO>::type;
  constexpr int ES = sizeof(TS), VB = 4 * ES;
  constexpr int PITCH = OUTN * ES + VB;
  constexpr int SLAB = WM * 32 * PITCH;
  static_assert(SLAB <= LDSB, "one slab must fit the staging space");
  constexpr int SPI = staged_slabs(MT, SLAB, LDSB);
  constexpr int R = WM * SPI * 32;  // staged rows per pass
  constexpr int LPR = OUTN / 4;     // lanes per staged row
  static_assert(64 % LPR == 0, "whole rows per wavefront access");
  constexpr int RPI = 64 / LPR;     // rows per wavefront access
  static_assert((R / RPI) % NW == 0, "row groups spread evenly over wavefronts");
  static_assert(EPI != EPI_LNRELU, "conv1's epilogue is not staged");

  const int r = lane & 31, h = lane >> 5;
  const float lo = p.olo[GLU ? 0 : seg], hi = p.ohi[GLU ? 0 : seg];
  const int ocol0 = GLU ? n0 / 2 : n0;
  TO* C = (TO*)p.C;
  // every wavefront is past its last fragment read, and the main loop's
  // final (unused) refill has landed, before the stage buffers are reused
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < MT / SPI; ++pass) {
    if (pass > 0) __syncthreads();
#pragma unroll
    for (int s = 0; s < SPI; ++s) {
      const int i = pass * SPI + s;
      unsigned char* srow = smem + (wm * SPI * 32 + s * 32 + r) * PITCH;
      if (GLU) {
#pragma unroll
        for (int jp = 0; jp < NTL / 2; ++jp)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wn * WOUT + jp * 32 + g * 8 + h * 4;
            float ba[4] = {0.f, 0.f, 0.f, 0.f}, bb[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.bias) {  // 16-byte loads of the a and b halves' biases
              const float4 va = *(const float4*)(p.bias + ocol0 + c);
              const float4 vb = *(const float4*)(p.bias + p.glu_d + ocol0 + c);
              ba[0] = va.x; ba[1] = va.y; ba[2] = va.z; ba[3] = va.w;
              bb[0] = vb.x; bb[1] = vb.y; bb[2] = vb.z; bb[3] = vb.w;
            }
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float a = clampf(acc[i][2 * jp][4 * g + e], lo, hi);
              float b = clampf(acc[i][2 * jp + 1][4 * g + e], lo, hi);
              if (p.bias) {
                a += ba[e];
                b += bb[e];
              }
              o[e] = a * sigmoidf_(b);
            }
            put4s<TS>(srow + c * ES, o);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wn * WOUT + j * 32 + g * 8 + h * 4;
            const int col = ocol0 + c;
            float o[4];
            if (EPI == EPI_STORE) {
              float4 sc = make_float4(1.f, 1.f, 1.f, 1.f);
              if (p.colscale) sc = *(const float4*)(p.colscale + col);
              const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = clampf(acc[i][j][4 * g + e], lo, hi) * scv[e];
            } else if (EPI == EPI_SILU) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float y = clampf(acc[i][j][4 * g + e], lo, hi);
                o[e] = clampf(y * sigmoidf_(y), p.nlo, p.nhi);
              }
            } else if (EPI == EPI_RESID) {
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = clampf(acc[i][j][4 * g + e], lo, hi);
              if (p.bias) {
                const float4 bv = *(const float4*)(p.bias + col);
                const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (o[e] + bb[e]) * p.rscale;
              }
            } else if (EPI == EPI_ACT) {
              // one 16-byte bias load per four columns, and the activation
              // chosen once per group rather than per value
              const float4 bv =
                  p.bias ? *(const float4*)(p.bias + col) : make_float4(0.f, 0.f, 0.f, 0.f);
              const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
              if (p.act == ACT_SILU) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float y = acc[i][j][4 * g + e] + bb[e];
                  o[e] = y * sigmoidf_(y);
                }
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = act_apply(p.act, acc[i][j][4 * g + e] + bb[e]);
              }
            } else {  // EPI_BIAS
              const float4 bv = *(const float4*)(p.bias + col);
              o[0] = acc[i][j][4 * g] + bv.x;
              o[1] = acc[i][j][4 * g + 1] + bv.y;
              o[2] = acc[i][j][4 * g + 2] + bv.z;
              o[3] = acc[i][j][4 * g + 3] + bv.w;
            }
            put4s<TS>(srow + c * ES, o);
          }
      }
    }
    __syncthreads();
    if constexpr (EPI != EPI_RESID) {
      // the staged values are already in the output type: copy raw 16-byte
      // chunks, consecutive lanes on consecutive bytes of a row (against
      // 8-byte pieces widened to float and narrowed again: FFN W1 190 ->
      // 187 us, q|k|v 143.8 -> 141.3, step 15.84 -> 15.72 ms on one box)
      constexpr int L16 = OUTN * ES / 16;  // lanes per staged row
      static_assert(64 % L16 == 0, "whole rows per wavefront access");
      constexpr int RP16 = 64 / L16;
      static_assert((R / RP16) % NW == 0, "row groups spread evenly over wavefronts");
#pragma unroll
      for (int t = 0; t < R / RP16 / NW; ++t) {
        const int sr = (t * NW + wave) * RP16 + lane / L16;
        const int cb = (lane % L16) * 16;
        const int wr = sr / (SPI * 32), w = sr - wr * (SPI * 32);
        const int grow = m0 + wr * WTM + (pass * SPI + w / 32) * 32 + (w & 31);
        if (grow < p.M) {
          // rows sit at an 8-byte pitch offset: two 8-byte LDS reads
          const uint2 lo2 = *(const uint2*)(smem + sr * PITCH + cb);
          const uint2 hi2 = *(const uint2*)(smem + sr * PITCH + cb + 8);
          const uint4 v = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
          *(uint4*)((unsigned char*)(C + (size_t)grow * p.ldc + ocol0) + cb) = v;
        }
      }
      continue;
    }
#pragma unroll
    for (int t = 0; t < R / RPI / NW; ++t) {
      const int sr = (t * NW + wave) * RPI + lane / LPR;
      const int c = (lane % LPR) * 4;
      const int wr = sr / (SPI * 32), w = sr - wr * (SPI * 32);
      const int grow = m0 + wr * WTM + (pass * SPI + w / 32) * 32 + (w & 31);
      if (grow < p.M) {
        float o[4];
        get4s<TS>(smem + sr * PITCH + c * ES, o);
        TO* dst = C + (size_t)grow * p.ldc + ocol0 + c;
        if (EPI == EPI_RESID) {
          const float4 hv = *(const float4*)dst;
          o[0] += hv.x; o[1] += hv.y; o[2] += hv.z; o[3] += hv.w;
        }
        store4(dst, o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <typename T, typename TO, int BM, int BN, int WM, int WN, int AL, int EPI>
__global__ void __launch_bounds__(WM * WN * 64) k_gemm(GemmParams p) {
  constexpr int NTH = WM * WN * 64;
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int BK = ROWB / sizeof(T);     // k per step
  constexpr int A_PT = BM * 8 / NTH;       // A chunks per thread per step
  constexpr int B_PT = BN * 8 / NTH;
  static_assert(A_PT * NTH == BM * 8 && B_PT * NTH == BN * 8, "tile/thread mismatch");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NTL = WTN / 32;
  static_assert(MT * 32 == WTM && NTL * 32 == WTN, "wave tile must be 32-aligned");
  static_assert(EPI != EPI_GLU || (WTN % 64) == 0, "GLU pairs need 64-column wave tiles");
  constexpr int STAGE = (BM + BN) * ROWB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN;
  // a K split: block b takes tile b % tiles and the split-th share of the
  // k-steps, and leaves its partial tile for k_gemm_reduce
  const int splits = p.splits > 1 ? p.splits : 1;
  const int tiles = ((p.M + BM - 1) / BM) * tiles_n;
  const int tile = (int)blockIdx.x % tiles, split = (int)blockIdx.x / tiles;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  int seg = 0, nloc = n0;
  if (EPI != EPI_GLU && EPI != EPI_LNRELU) {
    seg = n0 / p.seg_n;
    nloc = n0 - seg * p.seg_n;
  }
  const T* Ab = (const T*)p.A[seg];
  const T* Bb = (const T*)p.Bm[seg];

  // ---- per-thread sources of the chunks this thread stages
  const T* a_src[A_PT];
  bool a_ok[A_PT];
  int c_base[A_PT], c_lo[A_PT], c_hi[A_PT], c_f[A_PT];
#pragma unroll
  for (int i = 0; i < A_PT; ++i) {
    const int q = tid + i * NTH, row = q >> 3, c = q & 7;
    const int gm = m0 + row;
    if (AL == A_PLAIN) {
      a_ok[i] = gm < p.M;
      a_src[i] = Ab + (size_t)(a_ok[i] ? gm : 0) * p.lda + c * EPC;
    } else {
      // conv1 im2col: row = token * 32 + f; k = (dt*3 + df)*128 + ci
      const int g = gm >> 5;
      c_f[i] = gm & 31;
      if (g < p.n_tok) {
        const int t = p.tok_pos[g], cl = p.tok_clip[g];
        const int64_t r0 = p.row_off[cl];
        const int t1n = (int)(p.row_off[cl + 1] - r0);
        c_base[i] = (int)r0 + 2 * t - 1;
        c_lo[i] = (2 * t - 1 >= 0) ? 0 : 1;
        c_hi[i] = min(2, t1n - (2 * t - 1) - 1);
      } else {
        c_base[i] = 0;
        c_lo[i] = 3;
        c_hi[i] = -1;
      }
      a_ok[i] = true;
      a_src[i] = nullptr;
    }
  }
  const T* b_src[B_PT];
#pragma unroll
  for (int i = 0; i < B_PT; ++i) {
    const int q = tid + i * NTH, row = q >> 3, c = q & 7;
    int wrow;
    if (EPI == EPI_GLU) {
      const int vr = n0 + row;  // virtual row: 32 'a' rows, then 32 'b' rows
      wrow = ((vr >> 5) & 1) * p.glu_d + (vr >> 6) * 32 + (vr & 31);
    } else {
      wrow = nloc + row;
    }
    b_src[i] = Bb + (size_t)wrow * p.ldb + c * EPC;
  }

  u32x4 ra[A_PT], rb[B_PT];
  auto load_global = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      if (AL == A_PLAIN) {
        ra[i] = a_ok[i] ? *(const u32x4*)(a_src[i] + (size_t)kt * BK) : u32x4{0, 0, 0, 0};
      } else {
        const int c = (tid + i * NTH) & 7;
        const int kidx = kt * BK + c * EPC;
        const int tap = kidx >> 7, ci = kidx & 127;
        const int dt = tap / 3, df = tap - 3 * (tap / 3);
        const int f1 = 2 * c_f[i] - 1 + df;
        const bool ok = dt >= c_lo[i] && dt <= c_hi[i] && f1 >= 0 && f1 < kF1;
        const T* y0 = (const T*)p.y0;
        ra[i] = ok ? *(const u32x4*)(y0 + ((size_t)(c_base[i] + dt) * kF1 + f1) * kC0 + ci)
                   : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) rb[i] = *(const u32x4*)(b_src[i] + (size_t)kt * BK);
  };
  auto store_lds = [&](int buf) {
    unsigned char* s = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int q = tid + i * NTH;
      *(u32x4*)(s + swz(q >> 3, q & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int q = tid + i * NTH;
      *(u32x4*)(s + BM * ROWB + swz(q >> 3, q & 7)) = rb[i];
    }
  };

  f32x16 acc[MT][NTL];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = p.K / BK / splits, k0 = split * nk;
  load_global(k0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global(k0 + kt + 1);
    const unsigned char* s = smem + cur * STAGE;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int c = 2 * st + (lane >> 5);
      u32x4 fa[MT], fb[NTL];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        fa[i] = *(const u32x4*)(s + swz(wm * WTM + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < NTL; ++j)
        fb[j] = *(const u32x4*)(s + BM * ROWB + swz(wn * WTN + j * 32 + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j) Mma<T>::run(acc[i][j], fb[j], fa[i]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  if (splits > 1) {
    float4* dst = (float4*)p.part +
                  ((size_t)(split * tiles + tile) * (WM * WN) + wave) * (MT * NTL * 4 * 64) + lane;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTL; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          dst[((i * NTL + j) * 4 + v4) * 64] =
              make_float4(acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                          acc[i][j][4 * v4 + 3]);
    return;
  }
  epilogue<TO, MT, NTL, EPI>(p, acc, m0 + wm * WTM, n0 + wn * WTN, seg, lane);
}

// The second pass of a K split: each wavefront adds its accumulators' shares
// from the p.splits partial tiles in split order (a fixed order, so the
// result does not depend on which split finished first) and runs the
// epilogue the one-pass kernel would have.
template <typename TO, int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM * WN * 64) k_gemm_reduce(GemmParams p) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NTL = WTN / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN;
  const int tiles = ((p.M + BM - 1) / BM) * tiles_n;
  const int tile = blockIdx.x;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int seg = (EPI != EPI_GLU && EPI != EPI_LNRELU) ? n0 / p.seg_n : 0;
  f32x16 acc[MT][NTL];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int sp = 0; sp < p.splits; ++sp) {
    const float4* src = (const float4*)p.part +
                        ((size_t)(sp * tiles + tile) * (WM * WN) + wave) * (MT * NTL * 4 * 64) +
                        lane;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTL; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 v = src[((i * NTL + j) * 4 + v4) * 64];
          acc[i][j][4 * v4] += v.x;
          acc[i][j][4 * v4 + 1] += v.y;
          acc[i][j][4 * v4 + 2] += v.z;
          acc[i][j][4 * v4 + 3] += v.w;
        }
  }
  epilogue<TO, MT, NTL, EPI>(p, acc, m0 + wm * WTM, n0 + wn * WTN, seg, lane);
}

// Map the hardware block index to a tile. The dispatcher deals blocks to
// the 8 XCDs round-robin; the blocks of one XCD get one contiguous range of
// tile numbers, and tile numbers walk column-major through bands of GM row
// tiles, so the ~32 blocks an XCD runs at once cover a GM x (32/GM) window
// whose A and B slices are shared through that XCD's L2.
template <int GM>
__device__ __forceinline__ void tile_of(int b, int nblk, int tiles_m, int tiles_n, int& tm,
                                        int& tn) {
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = b & 7, local = b >> 3;
  const int t = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int band = t / (GM * tiles_n);
  const int m_lo = band * GM;
  const int gm = min(GM, tiles_m - m_lo);
  const int r = t - band * GM * tiles_n;
  tn = r / gm;
  tm = m_lo + (r - tn * gm);
}

// Workgroup barrier without the memory fence __syncthreads() adds (which
// would wait for every outstanding global load); the asm statements keep
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS image of a tile row of RB bytes: chunk c of row r sits at chunk
// c ^ f(r), f chosen so that the 16 rows one fragment-read pass serves (16
// consecutive rows, one chunk index) land in 16 distinct 16-byte groups of
// the 64 four-byte banks: with 128-byte rows two rows share the 256-byte
// bank space, with 64-byte rows four do.
template <int RB>
__device__ __forceinline__ int swz_rb(int row, int c) {
  if (RB == 128) return row * 128 + ((c ^ ((row >> 1) & 7)) << 4);
  return row * 64 + ((c ^ ((row >> 2) & 3)) << 4);
}

// Plain-operand GEMM with direct global->LDS loads and a STAGES-deep ring
// of LDS stages (each BM + BN rows of RB bytes, i.e. RB / sizeof(T) of k).
// Every 1-KB group of rows is filled by one buffer_load_dwordx4 ... lds of
// one wavefront, lane l landing at byte 16 l of the group; the XOR swizzle is
// applied on the source side (lane l fetches the logical chunk that belongs
// at its physical slot), so the LDS image is the swizzled layout the
// fragment reads expect. Loads run STAGES - 1 stages ahead of the MFMAs;
// each wavefront waits only for its own loads of the stage it is about to
// read (exact vmcnt), then a bare barrier publishes the stage. Rows past M
// read zeros (their results are never stored).
//
// FB is the number of register sets for the MFMA fragments. With two, the
// reads of the next substep are in flight under the MFMAs of the current
// one; with one, each substep reads its fragments and then multiplies,
// which saves (MT + NTL) * 4 registers a lane. That fits a 96x128
// wavefront tile in 256 registers (accumulators included), so each SIMD
// runs two such wavefronts that hide each other's waits: eight of them in
// one 384x256 block, or four in each of two 192x256 blocks that share a CU
// (two 64-byte stages, 56 KB of LDS each).
template <typename T, typename TO, int BM, int BN, int WM, int WN, int RB, int STAGES, int EPI,
          int OCC, int GM, int FB>
__global__ void __launch_bounds__(WM * WN * 64, OCC) k_gemm_dl(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int BK = RB / sizeof(T);
  constexpr int CPR = RB / 16;                 // chunks per row
  constexpr int RPG = 1024 / RB;               // rows per 1-KB group
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NTL = WTN / 32;
  static_assert(MT * 32 == WTM && NTL * 32 == WTN, "wave tile must be 32-aligned");
  static_assert(EPI != EPI_GLU || (WTN % 64) == 0, "GLU pairs need 64-column wave tiles");
  static_assert(BM % RPG == 0 && BN % RPG == 0, "whole groups");
  constexpr int GROUPS = (BM + BN) / RPG;
  static_assert(GROUPS % NW == 0, "groups spread evenly over wavefronts");
  constexpr int GPW = GROUPS / NW;             // loads per wavefront per stage
  static_assert(GPW * (STAGES - 2) < 64, "vmcnt range");
  static_assert(FB == 1 || FB == 2, "one or two fragment sets");
  constexpr int STAGE = (BM + BN) * RB;
  constexpr int SLAB0 = staged_slab_bytes<TO, EPI, BN, WM>();
  constexpr int SMEM = STAGES * STAGE > SLAB0 ? STAGES * STAGE : SLAB0;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  // wavefront index as a scalar: LDS destinations (m0) then need no
  // per-load readfirstlane
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN, tiles_m = (p.M + BM - 1) / BM;
  int tm, tn;
  tile_of<GM>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  int seg = 0, nloc = n0;
  if (EPI != EPI_GLU) {
    seg = n0 / p.seg_n;
    nloc = n0 - seg * p.seg_n;
  }
  const T* Ab = (const T*)p.A[seg];
  const T* Bb = (const T*)p.Bm[seg];

  // Loads are buffer loads straight to LDS with a buffer resource per
  // operand: A based at the tile's first row and sized to the rows below M,
  // B at the weight matrix. The range check covers only the per-lane
  // offset, so an A group's row offset is folded into it (one register per
  // group) and A rows past M read zeros (their results are never stored);
  // B groups share one per-lane offset and keep their row offset in a
  // scalar register. The k advance is a scalar offset.
  static_assert(NW % 2 == 0, "groups of one wavefront share the swizzle parity");
  const int l = lane / CPR, pc = lane % CPR;
  // the swizzle of row g * RPG + l: with 128-byte rows it depends on g's
  // parity, which equals the wavefront's (NW is even)
  const int sw = RB == 128 ? (((wave & 1) * 4 + (l >> 1)) & 7) : ((l >> 2) & 3);
  const int c = pc ^ sw;
  const uint32_t lane_a = (uint32_t)((l * p.lda + c * EPC) * (int)sizeof(T));
  const uint32_t lane_b = (uint32_t)((l * p.ldb + c * EPC) * (int)sizeof(T));
  const size_t a_bytes = (size_t)(p.M - m0) * p.lda * sizeof(T);
  const i32x4 rs_a = buffer_rsrc(Ab + (size_t)m0 * p.lda,
                                 (uint32_t)(a_bytes < 0xFFFFFFFFull ? a_bytes : 0xFFFFFFFFull));
  const i32x4 rs_b = buffer_rsrc(Bb, 0xFFFFFFFFu);
  uint32_t voff[GPW], soff[GPW];
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int r0 = (wave + i * NW) * RPG;
    if (r0 < BM) {
      voff[i] = lane_a + (uint32_t)(r0 * p.lda * (int)sizeof(T));
      soff[i] = 0;
    } else {
      const int br0 = r0 - BM;
      int wrow0;
      if (EPI == EPI_GLU) {
        // 32 'a' rows, then 32 'b' rows: a group's rows stay in one run
        const int vr = n0 + br0;
        wrow0 = ((vr >> 5) & 1) * p.glu_d + (vr >> 6) * 32 + (vr & 31);
      } else {
        wrow0 = nloc + br0;
      }
      voff[i] = lane_b;
      // uniform by construction; say so, or the compiler may keep it in a
      // vector register and loop over its distinct values
      soff[i] = __builtin_amdgcn_readfirstlane((uint32_t)((size_t)wrow0 * p.ldb * sizeof(T)));
    }
  }
  auto issue_one = [&](int i, int buf, int kt) {
    const int g = wave + i * NW;
    raw_buffer_load_lds(g * RPG < BM ? rs_a : rs_b,
                        (__attribute__((address_space(3))) void*)(smem + buf * STAGE + g * 1024),
                        16, voff[i], soff[i] + (uint32_t)(kt * RB), 0, 0);
  };
  auto issue = [&](int buf, int kt) {
#pragma unroll
    for (int i = 0; i < GPW; ++i) issue_one(i, buf, kt);
  };

  f32x16 acc[MT][NTL];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTL; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // With FB == 2, fragments are double-buffered in registers: the reads of
  // substep st + 1 (or of the next stage's substep 0) are issued before the
  // MFMAs of substep st, and sched_barrier keeps the scheduler from sinking
  // them back next to their use.
  constexpr int NSUB = CPR / 2;
  u32x4 fa[FB][MT], fb[FB][NTL];
  auto load_frags = [&](int sel, const unsigned char* sb, int st) {
    const int c = 2 * st + (lane >> 5);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      fa[sel][i] = *(const u32x4*)(sb + swz_rb<RB>(wm * WTM + i * 32 + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < NTL; ++j)
      fb[sel][j] = *(const u32x4*)(sb + BM * RB + swz_rb<RB>(wn * WTN + j * 32 + (lane & 31), c));
  };

  const int nk = p.K / BK;
  // prologue: stages 0 .. STAGES-2 in flight, publish stage 0, queue the next
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, st);
  if (STAGES - 2 < nk) wait_vmcnt<GPW * (STAGES - 2)>();
  else wait_vmcnt<0>();
  bare_barrier();
  if (STAGES - 1 < nk) issue(STAGES - 1, STAGES - 1);
  if constexpr (FB == 2) load_frags(0, smem, 0);

  // One substep: the MFMAs on fragment set `cur`, with the operations the
  // caller emitted just before threaded between them: after each of the
  // first MFMAs one fragment read (for the next substep) and, in the
  // publishing substep, one global->LDS load of a later stage. Issuing the
  // loads back to back would stall the wavefront's issue for their whole
  // duration; spread out, they hide under the MFMAs.
  constexpr int NMFMA = MT * NTL, NLOAD = MT + NTL;
  static_assert(FB == 1 || NLOAD <= NMFMA, "interleave needs an MFMA per read");
  // A wavefront runs its MFMA run at raised priority, so the SIMD's other
  // wavefront, reading fragments or waiting, does not take issue slots from
  // it (FFN W2 170.1 -> 167.0 us, the LFM2A step 8.16 -> 8.10 ms).
  // s_setprio is a scheduling boundary: a caller that emits fragment reads
  // or loads to be threaded between the MFMAs raises the priority before
  // emitting them (raise = false here), or they could not move past it.
  auto mfmas = [&](int cur, int nreads, int nloads, bool raise = true) {
    if (raise) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTL; ++j) Mma<T>::run(acc[i][j], fb[cur][j], fa[cur][i]);
    // reads and loads cannot pass each other (the compiler keeps LDS reads
    // ahead of the LDS-writing loads), so: MFMA+read pairs, then MFMA+load
    // pairs, then the remaining MFMAs (loads beyond the MFMA count go last)
#pragma unroll
    for (int q = 0; q < NMFMA; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (q < nreads) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      } else if (q < nreads + nloads) {
        __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);  // scalar setup
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global->LDS load
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Every iteration but the last publishes the next stage before its last
  // substep; the last iteration is peeled so the loop body has no branch.
  if constexpr (FB == 1) {
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const unsigned char* sb = smem + (kt % STAGES) * STAGE;
#pragma unroll
      for (int st = 0; st < NSUB; ++st) {
        load_frags(0, sb, st);
        if (st + 1 < NSUB) {
          mfmas(0, 0, 0);
          continue;
        }
        // the last substep's fragments have landed: publish stage kt + 1
        // and refill stage kt's buffer (the same rules as below), with the
        // loads threaded between this substep's MFMAs
        wait_lgkmcnt0();
        if (kt + STAGES - 1 < nk) wait_vmcnt<GPW * (STAGES - 2)>();
        else wait_vmcnt<0>();
        bare_barrier();
        // the loads one by one between the MFMAs, in program order (the
        // scheduler, left to itself, bunches them ahead of the MFMAs)
        __builtin_amdgcn_s_setprio(1);
        const int rb = kt % STAGES, rk = min(kt + STAGES, nk - 1);
#pragma unroll
        for (int q = 0; q < NMFMA; ++q) {
          Mma<T>::run(acc[q / NTL][q % NTL], fb[0][q % NTL], fa[0][q / NTL]);
          if (q < GPW) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(q, rb, rk);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int i = NMFMA; i < GPW; ++i) issue_one(i, rb, rk);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    const unsigned char* sb = smem + ((nk - 1) % STAGES) * STAGE;
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
      load_frags(0, sb, st);
      mfmas(0, 0, 0);
    }
  } else {
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const unsigned char* sb = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
      const int cur = st & 1;
      if (st + 1 < NSUB) {
        __builtin_amdgcn_s_setprio(1);
        load_frags(cur ^ 1, sb, st + 1);
      } else {
        // Publish stage kt + 1 (this wave's loads of it have landed and its
        // reads of stage kt have returned), start reading it, and refill
        // stage kt's buffer with stage kt + STAGES. Near the end there is no
        // such stage; the buffer then gets the last stage again (valid
        // addresses, never read: the stages still to come live in the other
        // buffers), which keeps this substep free of branches so its loads
        // can interleave with the MFMAs. The reads go first: the compiler
        // cannot tell the two buffers apart and would keep them in order.
        if (kt + STAGES - 1 < nk) wait_vmcnt<GPW * (STAGES - 2)>();
        else wait_vmcnt<0>();
        wait_lgkmcnt0();
        bare_barrier();
        __builtin_amdgcn_s_setprio(1);
        load_frags(cur ^ 1, smem + ((kt + 1) % STAGES) * STAGE, 0);
        issue(kt % STAGES, min(kt + STAGES, nk - 1));
        mfmas(cur, NLOAD, GPW, false);
        continue;
      }
      mfmas(cur, NLOAD, 0, false);
    }
  }
  {
    const unsigned char* sb = smem + ((nk - 1) % STAGES) * STAGE;
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
      const int cur = st & 1;
      __builtin_amdgcn_s_setprio(1);
      if (st + 1 < NSUB) load_frags(cur ^ 1, sb, st + 1);
      mfmas(cur, st + 1 < NSUB ? NLOAD : 0, 0, false);
    }
  }
  }
  // Every epilogue is staged through LDS, SiLU and GLU included: with the
  // 384x256 tiles that took FFN W1 from 218 to 208.5 us and the GLU
  // projection from 101.7 to 98.2 against storing them straight from
  // registers (which the 256x256 tiles had preferred).
  epilogue_staged<TO, BM, BN, WM, WN, EPI, SMEM>(p, acc, smem, m0, n0, wm, wn, seg, wave, lane);
}

template <typename T, typename TO, int BM, int BN, int WM, int WN, int RB, int STAGES, int EPI,
          int OCC = 1, int GM = 4, int FB = 2>
hipError_t run_dl(const GemmParams& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
  hipLaunchKernelGGL((k_gemm_dl<T, TO, BM, BN, WM, WN, RB, STAGES, EPI, OCC, GM, FB>), dim3(tiles),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <typename T, typename TO, int BM, int BN, int WM, int WN, int AL, int EPI>
hipError_t run(const GemmParams& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
  hipLaunchKernelGGL((k_gemm<T, TO, BM, BN, WM, WN, AL, EPI>), dim3(tiles), dim3(WM * WN * 64), 0,
                     s, p);
  return hipGetLastError();
}

// The float path's K split. A split count that followed the row count
// would change each output's summation order between a clip run alone and
// the same clip packed with others, so it follows K alone: the 4096-deep
// FFN W2 (in a 30 s clip 192 64x64 tiles with 4096-deep k-loops, 768
// wavefronts for 1024 SIMDs) runs as four splits of 1024, every other
// projection (K of 1024 to 1536) whole. Each split leaves its partial tile
// in p.part, and k_gemm_reduce adds them in split order and runs the
// epilogue. The caller's area must hold splits x (M rounded up to the row
// tile) x N floats; a smaller one is an error, not a silent unsplit run.
// Measured on a 30 s clip: FFN W2 102.6 us whole, 83.7 in two splits, 66.7
// in four (step 6.74 -> 6.21 -> 5.78 ms); on a 1 s clip 100.8, 55.0 and
// 32.9 us. For large batches four splits add 32 bytes of partial traffic a
// row and column pair (about 7% on a 24000-row W2).
constexpr int kSplitK4096 = 4;
int f32_splits(int K) { return K >= 4096 && K % 4096 == 0 ? kSplitK4096 * (K / 4096) : 1; }

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t run_f32(const GemmParams& p0, hipStream_t s) {
  if (p0.M <= 0) return hipSuccess;
  GemmParams p = p0;
  const int S = f32_splits(p.K);
  p.splits = S;
  if (S == 1) return run<float, float, BM, BN, WM, WN, A_PLAIN, EPI>(p, s);
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
  if (!p.part || (size_t)S * tiles * BM * BN * sizeof(float) > p.part_bytes)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm<float, float, BM, BN, WM, WN, A_PLAIN, EPI>), dim3(tiles * S),
                     dim3(WM * WN * 64), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_reduce<float, BM, BN, WM, WN, EPI>), dim3(tiles), dim3(WM * WN * 64),
                     0, s, p);
  return hipGetLastError();
}

// fp32 operands (the parity path): register-staged 128x128 tiles, or for
// fewer than 4096 rows (a 30 s clip has 750 tokens, where 128x128 tiles
// give a 1024-column output 48 blocks for 256 CUs) 64x64 tiles of four
// 32x32 wavefronts (64x128 for the GLU, whose column pairs need 64-column
// wavefront tiles). Every tile shape accumulates an output over k in the
// same order, so the shape, which follows the row count, changes no bit.
hipError_t dispatch_f32(int epi, int aload, const GemmParams& p, hipStream_t s) {
  if (aload == A_CONV1) return run<float, float, 128, 32, 4, 1, A_CONV1, EPI_LNRELU>(p, s);
  if (p.M < 4096) {
    switch (epi) {
      case EPI_STORE: return run_f32<64, 64, 2, 2, EPI_STORE>(p, s);
      case EPI_SILU: return run_f32<64, 64, 2, 2, EPI_SILU>(p, s);
      case EPI_GLU: return run_f32<64, 128, 2, 2, EPI_GLU>(p, s);
      case EPI_RESID: return run_f32<64, 64, 2, 2, EPI_RESID>(p, s);
      case EPI_BIAS: return run_f32<64, 64, 2, 2, EPI_BIAS>(p, s);
      case EPI_ACT: return run_f32<64, 64, 2, 2, EPI_ACT>(p, s);
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_STORE: return run_f32<128, 128, 2, 2, EPI_STORE>(p, s);
    case EPI_SILU: return run_f32<128, 128, 2, 2, EPI_SILU>(p, s);
    case EPI_GLU: return run_f32<128, 128, 2, 2, EPI_GLU>(p, s);
    case EPI_RESID: return run_f32<128, 128, 2, 2, EPI_RESID>(p, s);
    case EPI_BIAS: return run_f32<128, 128, 2, 2, EPI_BIAS>(p, s);
    case EPI_ACT: return run_f32<128, 128, 2, 2, EPI_ACT>(p, s);
  }
  return hipErrorInvalidValue;
}

// bf16 operands: direct-to-LDS pipelined kernels; the tile shape follows
// the row count, the output width (tiles per wave of 256 CUs) and the
// epilogue.
//  N a multiple of 1024, no residual add: 384x256, 8 wavefronts of 96x128
//         with one fragment set, two 128-byte stages (the whole 160 KB of LDS)
//  other N % 256 == 0, no residual add: 192x128 blocks, 4 wavefronts of
//         96x64 with one fragment set, two 64-byte stages, three blocks per CU
//  otherwise (the fp32 residual add): 256x128, 8 wavefronts of 64x64, two
//         blocks per CU
template <int EPI, typename TO>
hipError_t run_bf16(const GemmParams& p, hipStream_t s) {
  // fewer rows (the LFM2A encoder's 12032 tokens): the shapes below leave
  // CUs idle (a 512-column output in 192x256 tiles is 126 tiles for 256
  // CUs), and a 512-column output in 128x128 tiles is still only 376 tiles.
  // Those run latency-bound, so each tile gets eight 32x64 wavefronts with
  // one fragment set (three blocks per CU): measured inside that encoder
  // against four 64x64 wavefronts (and 256x128 blocks for 2048 columns),
  // the step went from 8.34 to 7.67-7.84 ms (feed-forward down 52.6 -> 46.7
  // us, the attention projections 28.4 -> 23.5, the convolution module's
  // 27.8 -> 23.8)
  if (p.M < 16384) return run_dl<bf16, TO, 128, 128, 4, 2, 64, 3, EPI, 3, 4, 1>(p, s);
  // measured inside the encoder (24000 rows), against the shapes before:
  // - 384x256 tiles (in bands of 4 row tiles) against 256x256 tiles of
  //   eight 128x64 wavefronts: q|k|v 165 -> 156 us (752 tiles in 2.9 rounds
  //   of the CUs instead of 1128 in 4.4), the GLU projection 103.5 -> 100.7,
  //   FFN W1 the same; against paired 192x256 blocks: FFN W2 180 -> 170.6,
  //   the attention post projection 56.3 -> 54.2;
  // - paired 192x256 blocks against one 192x256 block per CU with two
  //   fragment sets and three stages: FFN W2 208 -> 184, post 67 -> 58, the
  //   head's projections 85 -> 75 on average; for the head's 512- and
  //   1536-column outputs 384x256 tiles leave CUs idle (126 and 378 tiles);
  // - linear_end's fp32 residual add measured 98.7 us in 256x128 blocks,
  //   101.4 in 384x256 tiles and 103 in paired 192x256 blocks.
  // - bands of 8 row tiles for the 4096-deep FFN W2 (167 -> 164 us against
  //   bands of 4; the others are 1-2% slower that way).
  if (p.N % 1024 == 0 && EPI != EPI_RESID) {
    if (p.K >= 2048) return run_dl<bf16, TO, 384, 256, 4, 2, 128, 2, EPI, 1, 8, 1>(p, s);
    return run_dl<bf16, TO, 384, 256, 4, 2, 128, 2, EPI, 1, 4, 1>(p, s);
  }
  // outputs not a multiple of 1024 wide (the head's 1536 and 512, the
  // LFM2A stem's 256): 192x128 blocks of four 96x64 wavefronts, three per
  // CU. Against paired 192x256 blocks the head's projections went from
  // 75.9 to 72.4 us on average and the LFM2A stem GEMMs from 166.0 to 128.5
  // (out_proj's 1536 columns make 1500 such tiles, 1.95 rounds of the CUs'
  // 768 slots, against 750 paired blocks in 1.46 rounds of 512)
  if (p.N % 256 == 0 && EPI != EPI_RESID)
    return run_dl<bf16, TO, 192, 128, 2, 2, 64, 2, EPI, 3, 4, 1>(p, s);
  return run_dl<bf16, TO, 256, 128, 4, 2, 64, 3, EPI, 2, 2>(p, s);
}

hipError_t dispatch_bf16(int epi, int aload, bool out_bf16, const GemmParams& p, hipStream_t s) {
  if (aload == A_CONV1) return hipErrorInvalidValue;  // bf16: launch_subsample_fused
  if (p.N % 128 != 0) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE:
      return out_bf16 ? run_bf16<EPI_STORE, bf16>(p, s) : run_bf16<EPI_STORE, float>(p, s);
    case EPI_SILU:
      return out_bf16 ? run_bf16<EPI_SILU, bf16>(p, s) : run_bf16<EPI_SILU, float>(p, s);
    case EPI_GLU:
      return out_bf16 ? run_bf16<EPI_GLU, bf16>(p, s) : run_bf16<EPI_GLU, float>(p, s);
    case EPI_RESID: return run_bf16<EPI_RESID, float>(p, s);
    case EPI_BIAS: return run_bf16<EPI_BIAS, float>(p, s);
    case EPI_ACT:
      return out_bf16 ? run_bf16<EPI_ACT, bf16>(p, s) : run_bf16<EPI_ACT, float>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t gemm_f32_part_bytes(int64_t M, int N, int K) {
  const int S = f32_splits(K);
  if (S == 1 || M <= 0) return 0;
  return (size_t)S * (size_t)((M + 127) / 128 * 128) * (size_t)N * sizeof(float);
}

hipError_t launch_gemm(ae_dtype dt, int epi, int aload, bool out_bf16, const GemmParams& p,
                       hipStream_t s) {
  if (dt == AE_BF16) return dispatch_bf16(epi, aload, out_bf16, p, s);
  return dispatch_f32(epi, aload, p, s);
}

}  // namespace ae
