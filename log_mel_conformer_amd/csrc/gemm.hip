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
// (feed-forward), the GLU of the light conv's linear_start, the light conv's
// residual add, the output projection's bias, per-column q/k scaling, and
// conv1's channel LayerNorm + ReLU.
#include <type_traits>

#include "launch.h"

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

__device__ __forceinline__ int swz(int row, int c) { return row * ROWB + ((c ^ (row & 7)) << 4); }

template <typename TO> __device__ __forceinline__ void store_out(TO* C, size_t idx, float v) {
  C[idx] = from_f32<TO>(v);
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
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
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

  const int nk = p.K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
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
        for (int j = 0; j < NTL; ++j) Mma<T>::run(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue. acc[i][j][v] sits at row (v/4)*8 + (lane/32)*4 + v%4 and
  // column lane%32 of the 32x32 sub-tile (i, j).
  TO* C = (TO*)p.C;
  const int rbase = m0 + wm * WTM + (lane >> 5) * 4;
  const int cl = lane & 31;
  if (EPI == EPI_GLU) {
    const float lo = p.olo[0], hi = p.ohi[0];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int jp = 0; jp < NTL / 2; ++jp) {
        const int col = (n0 + wn * WTN) / 2 + jp * 32 + cl;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
          const float a = clampf(acc[i][2 * jp][v], lo, hi);
          const float b = clampf(acc[i][2 * jp + 1][v], lo, hi);
          if (row < p.M) store_out(C, (size_t)row * p.ldc + col, a * sigmoidf_(b));
        }
      }
  } else if (EPI == EPI_LNRELU) {
    const float g = p.gain[cl];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
        const float x = acc[i][0][v];
        float s = x;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        const float mean = s * (1.0f / 32);
        const float dx = x - mean;
        float q = dx * dx;
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) q += __shfl_xor(q, o, 64);
        const float y = fmaxf(dx * rsqrtf(q * (1.0f / 32) + kEps) * g, 0.0f);
        if (row < p.M) store_out(C, (size_t)row * p.ldc + cl, y);
      }
  } else {
    const float lo = p.olo[seg], hi = p.ohi[seg];
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
      const int col = n0 + wn * WTN + j * 32 + cl;
      const float sc = (EPI == EPI_STORE && p.colscale) ? p.colscale[col] : 1.0f;
      const float bias = (EPI == EPI_BIAS) ? p.bias[col] : 0.0f;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
          if (row >= p.M) continue;
          const size_t idx = (size_t)row * p.ldc + col;
          const float x = acc[i][j][v];
          if (EPI == EPI_STORE) {
            store_out(C, idx, clampf(x, lo, hi) * sc);
          } else if (EPI == EPI_SILU) {
            const float y = clampf(x, lo, hi);
            store_out(C, idx, clampf(y * sigmoidf_(y), p.nlo, p.nhi));
          } else if (EPI == EPI_RESID) {
            float* H = (float*)p.C;
            H[idx] += clampf(x, lo, hi);
          } else if (EPI == EPI_BIAS) {
            ((float*)p.C)[idx] = x + bias;
          }
        }
    }
  }
}

template <typename T, typename TO, int BM, int BN, int WM, int WN, int AL, int EPI>
hipError_t run(const GemmParams& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
  hipLaunchKernelGGL((k_gemm<T, TO, BM, BN, WM, WN, AL, EPI>), dim3(tiles), dim3(WM * WN * 64), 0,
                     s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(int epi, int aload, bool out_bf16, const GemmParams& p, hipStream_t s) {
  typedef typename std::conditional<std::is_same<T, float>::value, float, bf16>::type TB;
  if (aload == A_CONV1) {
    if (out_bf16) return run<T, TB, 128, 32, 4, 1, A_CONV1, EPI_LNRELU>(p, s);
    return run<T, float, 128, 32, 4, 1, A_CONV1, EPI_LNRELU>(p, s);
  }
  switch (epi) {
    case EPI_STORE:
      if (out_bf16) return run<T, TB, 128, 128, 2, 2, A_PLAIN, EPI_STORE>(p, s);
      return run<T, float, 128, 128, 2, 2, A_PLAIN, EPI_STORE>(p, s);
    case EPI_SILU:
      if (out_bf16) return run<T, TB, 128, 128, 2, 2, A_PLAIN, EPI_SILU>(p, s);
      return run<T, float, 128, 128, 2, 2, A_PLAIN, EPI_SILU>(p, s);
    case EPI_GLU:
      if (out_bf16) return run<T, TB, 128, 128, 2, 2, A_PLAIN, EPI_GLU>(p, s);
      return run<T, float, 128, 128, 2, 2, A_PLAIN, EPI_GLU>(p, s);
    case EPI_RESID: return run<T, float, 128, 128, 2, 2, A_PLAIN, EPI_RESID>(p, s);
    case EPI_BIAS: return run<T, float, 128, 128, 2, 2, A_PLAIN, EPI_BIAS>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(ae_dtype dt, int epi, int aload, bool out_bf16, const GemmParams& p,
                       hipStream_t s) {
  if (dt == AE_BF16) return dispatch<bf16>(epi, aload, out_bf16, p, s);
  return dispatch<float>(epi, aload, false, p, s);
}

}  // namespace ae
