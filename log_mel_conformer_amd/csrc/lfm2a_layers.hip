// LFM2A stem, row and convolution kernels (cera 0.5.3, audio_encoder_gpu.rs:
// conv_stem_gpu with STEM_LAYER_MODES / STEM_RELU_AFTER, the layernorm op,
// the convolution module of encode_audio_gpu, and the relative-position
// table it uploads per chunk).
//
// Layout: the stem keeps its planes channels-last, [time][freq][256], so
// that the two pointwise layers are plain GEMMs over (time, freq) rows and
// the depthwise layers read 16 contiguous bytes of channels per lane; the
// flatten ahead of pre_encode_out then is the row itself, in (freq,
// channel) order, and the model permutes that matrix's columns once to
// match (the page flattens channel-major).
#include <math.h>

#include "lfm2a_launch.h"

namespace ae {
namespace lfm {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------ stem layers 0 and 1
// Layer 0 (3x3 stride 2, 1 -> 256 channels, ReLU) feeds only layer 1
// (depthwise 3x3 stride 2), so one kernel makes layer 1's output straight
// from the features and layer 0's 1.5 GB plane (at 32 x 30 s) never
// reaches memory. One block per layer-1 output row r (time step): the
// seven feature rows 4r - 3 .. 4r + 3 that layer 0's rows 2r - 1 .. 2r + 1
// read sit in LDS with the zero border; lane = 4 channels, wavefront = 8
// of the 32 output frequencies. A lane computes its channels' layer-0
// values column by column (float32, kept in registers: column 2f + 1 of
// one output is column 2(f + 1) - 1 of the next) and applies layer 1's
// taps. Layer 0 values outside its plane are layer 1's zero padding.
__global__ void __launch_bounds__(256) k_stem01(const float* __restrict__ feat,
                                                const int64_t* __restrict__ frame_off,
                                                const int64_t* __restrict__ row1_off,
                                                const int64_t* __restrict__ row2_off, int B,
                                                const float* __restrict__ w0,
                                                const float* __restrict__ b0,
                                                const float* __restrict__ wt1,
                                                const float* __restrict__ b1,
                                                bf16* __restrict__ y2) {
  __shared__ float in[7][kMel + 2];
  const int64_t r = blockIdx.x;
  const int c = find_clip(row2_off, B, r);
  const int64_t rl = r - row2_off[c];
  const int64_t F = frame_off[c + 1] - frame_off[c];
  const int64_t H1 = row1_off[c + 1] - row1_off[c];
  const float* fc = feat + frame_off[c] * kMel;
  for (int i = threadIdx.x; i < 7 * (kMel + 2); i += 256) {
    const int a = i / (kMel + 2), col = i % (kMel + 2) - 1;
    const int64_t fr = 4 * rl - 3 + a;
    in[a][col + 1] = (fr >= 0 && fr < F && col >= 0 && col < kMel) ? fc[fr * kMel + col] : 0.f;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ch = 4 * lane;
  float w[4][9], b[4], wd[4][9], bd[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    b[k] = b0[ch + k];
    bd[k] = b1[ch + k];
#pragma unroll
    for (int t = 0; t < 9; ++t) {
      w[k][t] = w0[(ch + k) * 9 + t];
      wd[k][t] = wt1[t * kStemCh + ch + k];
    }
  }
  // which of layer 0's rows 2r - 1, 2r, 2r + 1 exist in this clip
  bool rok[3];
#pragma unroll
  for (int dy = 0; dy < 3; ++dy) {
    const int64_t rho = 2 * rl - 1 + dy;
    rok[dy] = rho >= 0 && rho < H1;
  }
  __syncthreads();
  // layer-0 column f1 >= 0 (rows dy = 0..2, 4 channels); rows outside the
  // plane are 0
  auto column = [&](int f1, float (&v)[3][4]) {
#pragma unroll
    for (int dy = 0; dy < 3; ++dy) {
      float x[9];
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int bb = 0; bb < 3; ++bb) x[a * 3 + bb] = in[2 * dy + a][2 * f1 + bb];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float acc = b[k];
#pragma unroll
        for (int t = 0; t < 9; ++t) acc += w[k][t] * x[t];
        v[dy][k] = rok[dy] ? fmaxf(acc, 0.f) : 0.f;
      }
    }
  };
  const int f_lo = wv * 8;
  float cprev[3][4], c0[3][4], c1[3][4];
  if (f_lo > 0) {
    column(2 * f_lo - 1, cprev);
  } else {  // column -1: layer 1's zero padding
#pragma unroll
    for (int dy = 0; dy < 3; ++dy)
#pragma unroll
      for (int k = 0; k < 4; ++k) cprev[dy][k] = 0.f;
  }
  bf16* out = y2 + (r * kF2) * kStemCh + ch;
  for (int f = f_lo; f < f_lo + 8; ++f) {
    column(2 * f, c0);
    column(2 * f + 1, c1);
    float o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float acc = bd[k];
#pragma unroll
      for (int dy = 0; dy < 3; ++dy)
        acc += wd[k][dy * 3] * cprev[dy][k] + wd[k][dy * 3 + 1] * c0[dy][k] +
               wd[k][dy * 3 + 2] * c1[dy][k];
      o[k] = acc;
    }
    const bf16x4 v = {(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
    *(bf16x4*)(out + (size_t)f * kStemCh) = v;
#pragma unroll
    for (int dy = 0; dy < 3; ++dy)
#pragma unroll
      for (int k = 0; k < 4; ++k) cprev[dy][k] = c1[dy][k];
  }
}

// -------------------------------------------------- depthwise 3x3 stride 2
// Thread = 8 channels of one output position; 32 threads per position,
// kPosPerBlock positions per block (the taps stay in registers). The clip
// offsets are staged in LDS: a position's clip is a binary search over
// them, which through global memory is a chain of dependent loads.
constexpr int kPosPerBlock = 64;
constexpr int kMaxClipsLds = 512;

__global__ void __launch_bounds__(256) k_dw3s2(const bf16* __restrict__ y,
                                               const int64_t* __restrict__ in_off,
                                               const int64_t* __restrict__ out_off, int B,
                                               int64_t total_pos, int w_in,
                                               const float* __restrict__ wt,
                                               const float* __restrict__ bias,
                                               bf16* __restrict__ z) {
  __shared__ int64_t soff[kMaxClipsLds + 1], doff[kMaxClipsLds + 1];
  const bool lds_off = B <= kMaxClipsLds;
  if (lds_off)
    for (int i = threadIdx.x; i <= B; i += 256) {
      soff[i] = in_off[i];
      doff[i] = out_off[i];
    }
  const int c8 = (threadIdx.x & 31) * 8;
  const int w_out = w_in / 2;
  float w[9][8], b[8];
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const float4 a = *(const float4*)(wt + t * kStemCh + c8);
    const float4 d = *(const float4*)(wt + t * kStemCh + c8 + 4);
    w[t][0] = a.x; w[t][1] = a.y; w[t][2] = a.z; w[t][3] = a.w;
    w[t][4] = d.x; w[t][5] = d.y; w[t][6] = d.z; w[t][7] = d.w;
  }
  {
    const float4 a = *(const float4*)(bias + c8), d = *(const float4*)(bias + c8 + 4);
    b[0] = a.x; b[1] = a.y; b[2] = a.z; b[3] = a.w; b[4] = d.x; b[5] = d.y; b[6] = d.z; b[7] = d.w;
  }
  __syncthreads();
  for (int i = 0; i < kPosPerBlock / 8; ++i) {
    const int64_t pos = (int64_t)blockIdx.x * kPosPerBlock + i * 8 + (threadIdx.x >> 5);
    if (pos >= total_pos) break;
    const int64_t ro = pos / w_out;
    const int fo = (int)(pos - ro * w_out);
    const int64_t* io = lds_off ? soff : in_off;
    const int64_t* oo = lds_off ? doff : out_off;
    const int c = find_clip(oo, B, ro);
    const int64_t rl = ro - oo[c];
    const int64_t hin = io[c + 1] - io[c];
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = b[e];
#pragma unroll
    for (int dy = 0; dy < 3; ++dy) {
      const int64_t ri = 2 * rl + dy - 1;
      if (ri < 0 || ri >= hin) continue;
      const bf16* row = y + ((io[c] + ri) * w_in) * kStemCh + c8;
#pragma unroll
      for (int dz = 0; dz < 3; ++dz) {
        const int fi = 2 * fo + dz - 1;
        if (fi < 0 || fi >= w_in) continue;
        const bf16x8 v = *(const bf16x8*)(row + (size_t)fi * kStemCh);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w[dy * 3 + dz][e] * (float)v[e];
      }
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[e];
    *(bf16x8*)(z + pos * kStemCh + c8) = o;
  }
}

// ------------------------------------------------------------- LayerNorm
// A wavefront takes kLnRows 512-wide rows, loads them all (8 values per
// lane and row, two float4), then normalises them one by one; float32
// statistics: mean, then the mean square deviation from it.
__device__ __forceinline__ void ln8(const float* v, const float* w, const float* b, float eps,
                                    int lane, float* y) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  const float mean = wave_sum(s) * (1.0f / kD);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = v[i] - mean;
    q += d * d;
  }
  const float inv = rsqrtf(wave_sum(q) * (1.0f / kD) + eps);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 wv = *(const float4*)(w + h * 256 + lane * 4);
    const float4 bv = *(const float4*)(b + h * 256 + lane * 4);
    y[4 * h + 0] = (v[4 * h + 0] - mean) * inv * wv.x + bv.x;
    y[4 * h + 1] = (v[4 * h + 1] - mean) * inv * wv.y + bv.y;
    y[4 * h + 2] = (v[4 * h + 2] - mean) * inv * wv.z + bv.z;
    y[4 * h + 3] = (v[4 * h + 3] - mean) * inv * wv.w + bv.w;
  }
}

constexpr int kLnRows = 4;  // rows per wavefront, loaded together

__global__ void __launch_bounds__(256) k_layernorm(LnParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kLnRows;
  if (row0 >= p.n) return;
  float v[kLnRows][8];
#pragma unroll
  for (int q = 0; q < kLnRows; ++q) {
    const int64_t row = row0 + q < p.n ? row0 + q : p.n - 1;
    const float* xr = p.x + row * kD;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 a = *(const float4*)(xr + h * 256 + lane * 4);
      v[q][4 * h] = a.x; v[q][4 * h + 1] = a.y; v[q][4 * h + 2] = a.z; v[q][4 * h + 3] = a.w;
    }
  }
#pragma unroll
  for (int q = 0; q < kLnRows; ++q) {
    const int64_t row = row0 + q;
    if (row >= p.n) break;
    float* xr = p.x + row * kD;
    float y[8];
    ln8(v[q], p.w1, p.b1, p.eps, lane, y);
    if (p.write_x) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *(float4*)(xr + h * 256 + lane * 4) =
            make_float4(y[4 * h], y[4 * h + 1], y[4 * h + 2], y[4 * h + 3]);
    }
    if (p.w2) {
      float z[8];
      ln8(y, p.w2, p.b2, p.eps, lane, z);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = z[i];
    }
    if (p.a) {
      bf16* ar = p.a + row * kD;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x4 o = {(bf16)y[4 * h], (bf16)y[4 * h + 1], (bf16)y[4 * h + 2],
                          (bf16)y[4 * h + 3]};
        *(bf16x4*)(ar + h * 256 + lane * 4) = o;
      }
    }
  }
}

// ------------------------------------------------ depthwise conv1d + SiLU
// Thread = 4 channels; 128 threads cover a row, a block two groups of kRW
// consecutive rows. A group loads its kRW + K - 1 input rows into registers
// up front (one memory latency, not one per row); taps come transposed
// ([K][512], a float4 per tap), and a tap reaching past its own clip's ends
// (rows of a clip are consecutive) is 0. Four rows a group: 12032 rows
// then make 1504 blocks, enough wavefronts per CU to hide the loads (16 rows
// a group, 376 blocks, measured 19.7 against 15.8 us; 8 rows 16.2 us).
constexpr int kRW = 4;
constexpr int kMaxKern = 9;

__global__ void __launch_bounds__(256) k_dwconv(const bf16* __restrict__ g,
                                                const int32_t* __restrict__ tok_pos,
                                                const int32_t* __restrict__ tok_clip,
                                                const int64_t* __restrict__ token_off, int64_t n,
                                                const float* __restrict__ wt, int K,
                                                const float* __restrict__ bias,
                                                const float* __restrict__ aw,
                                                const float* __restrict__ ab,
                                                bf16* __restrict__ out) {
  const int grp = threadIdx.x >> 7;
  const int ch = (threadIdx.x & 127) * 4;
  const int64_t r0 = ((int64_t)blockIdx.x * 2 + grp) * kRW;
  if (r0 >= n) return;
  const int lo = (K - 1) / 2;
  float tw[kMaxKern][4];
#pragma unroll
  for (int j = 0; j < kMaxKern; ++j) {
    const float4 v = j < K ? *(const float4*)(wt + (size_t)j * kD + ch) : make_float4(0.f, 0.f, 0.f, 0.f);
    tw[j][0] = v.x; tw[j][1] = v.y; tw[j][2] = v.z; tw[j][3] = v.w;
  }
  const float4 bv = *(const float4*)(bias + ch), av = *(const float4*)(aw + ch),
               cv = *(const float4*)(ab + ch);
  const float bb[4] = {bv.x, bv.y, bv.z, bv.w}, aa[4] = {av.x, av.y, av.z, av.w},
              cc[4] = {cv.x, cv.y, cv.z, cv.w};
  // the group's rows: position in the clip and the clip's length, and the
  // kRW + K - 1 input rows (bf16, two registers a row), all fetched before
  // the first row is computed
  int pos_q[kRW], len_q[kRW];
#pragma unroll
  for (int q = 0; q < kRW; ++q) {
    const int64_t r = r0 + q < n ? r0 + q : n - 1;
    pos_q[q] = tok_pos[r];
    len_q[q] = tok_clip[r];
  }
  bf16x4 raw[kRW + kMaxKern - 1];
#pragma unroll
  for (int i = 0; i < kRW + kMaxKern - 1; ++i) {
    int64_t rr = r0 - lo + i;
    rr = rr < 0 ? 0 : (rr >= n ? n - 1 : rr);
    raw[i] = *(const bf16x4*)(g + rr * kD + ch);
  }
#pragma unroll
  for (int q = 0; q < kRW; ++q)
    len_q[q] = (int)(token_off[len_q[q] + 1] - token_off[len_q[q]]);
#pragma unroll
  for (int q = 0; q < kRW; ++q) {
    const int64_t r = r0 + q;
    if (r >= n) break;
    const int pos = pos_q[q];
    const int len = len_q[q];
    float acc[4] = {bb[0], bb[1], bb[2], bb[3]};
#pragma unroll
    for (int j = 0; j < kMaxKern; ++j) {
      const int src = pos + j - lo;
      if (j < K && src >= 0 && src < len) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += tw[j][e] * (float)raw[q + j][e];
      }
    }
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float y = acc[e] * aa[e] + cc[e];
      o[e] = y * sigmoidf_(y);
    }
    const bf16x4 v = {(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
    *(bf16x4*)(out + r * kD + ch) = v;
  }
}

// ----------------------------------------------------- relative positions
// Row r holds position t_max - 1 - r: (sin, cos)(p * 10000^(-2i / dim)),
// evaluated in float64 and rounded once.
__global__ void k_pos_table(int64_t t_max, int dim, bf16* __restrict__ pe) {
  const int64_t r = blockIdx.x;
  const double p = (double)(t_max - 1 - r);
  for (int i = threadIdx.x; i < dim / 2; i += blockDim.x) {
    const double w = exp(-(2.0 * i / dim) * log(10000.0));
    double sv, cv;
    sincos(p * w, &sv, &cv);
    pe[r * dim + 2 * i] = (bf16)(float)sv;
    pe[r * dim + 2 * i + 1] = (bf16)(float)cv;
  }
}

// ------------------------------------------------------------ model prep
__global__ void k_f32_to_bf16(const float* __restrict__ src, bf16* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (bf16)src[i];
}

__global__ void k_flatten_permute(const bf16* __restrict__ src, int rows, int C, int F,
                                  bf16* __restrict__ dst) {
  const int64_t total = (int64_t)rows * C * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t o = i / ((int64_t)C * F);
    const int k = (int)(i - o * C * F);  // destination column f * C + c
    const int f = k / C, c = k - f * C;
    dst[i] = src[o * C * F + (int64_t)c * F + f];
  }
}

__global__ void k_transpose_f32(const float* __restrict__ src, int C, int K,
                                float* __restrict__ dst) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < C * K; i += gridDim.x * blockDim.x) {
    const int j = i / C, c = i - j * C;
    dst[i] = src[c * K + j];
  }
}

__global__ void k_concat3(const float* a, const float* b, const float* c, int n, float* dst) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < 3 * n; i += gridDim.x * blockDim.x)
    dst[i] = i < n ? a[i] : (i < 2 * n ? b[i - n] : c[i - 2 * n]);
}

unsigned grid_for(int64_t n, int per_block, unsigned cap = 65536) {
  const int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_stem01(const float* feat, const int64_t* frame_off, const int64_t* row1_off,
                         const int64_t* row2_off, int B, int64_t rows2, const float* w0,
                         const float* b0, const float* wt1, const float* b1, bf16* y2,
                         hipStream_t s) {
  if (rows2 <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stem01, dim3((unsigned)rows2), dim3(256), 0, s, feat, frame_off, row1_off,
                     row2_off, B, w0, b0, wt1, b1, y2);
  return hipGetLastError();
}

hipError_t launch_dw3s2(const bf16* y, const int64_t* in_off, const int64_t* out_off, int B,
                        int64_t rows_out, int w_in, const float* wt, const float* b, bf16* z,
                        hipStream_t s) {
  const int64_t total = rows_out * (w_in / 2);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dw3s2, dim3((unsigned)((total + kPosPerBlock - 1) / kPosPerBlock)),
                     dim3(256), 0, s, y, in_off, out_off, B, total, w_in, wt, b, z);
  return hipGetLastError();
}

hipError_t launch_layernorm(const LnParams& p, hipStream_t s) {
  if (p.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_layernorm, dim3((unsigned)((p.n + 4 * kLnRows - 1) / (4 * kLnRows))),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dwconv(const bf16* g, const int32_t* tok_pos, const int32_t* tok_clip,
                         const int64_t* token_off, int64_t n, const float* wt, int k,
                         const float* b, const float* aw, const float* ab, bf16* c,
                         hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (k < 1 || k > kMaxKern) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dwconv, dim3((unsigned)((n + 2 * kRW - 1) / (2 * kRW))), dim3(256), 0, s, g,
                     tok_pos, tok_clip, token_off, n, wt, k, b, aw, ab, c);
  return hipGetLastError();
}

hipError_t launch_pos_table(int64_t t_max, int dim, bf16* pe, hipStream_t s) {
  if (t_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pos_table, dim3((unsigned)(2 * t_max - 1)), dim3(256), 0, s, t_max, dim,
                     pe);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, bf16* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_f32_to_bf16, dim3(grid_for(n, 256)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_flatten_permute(const bf16* src, int rows, int C, int F, bf16* dst,
                                  hipStream_t s) {
  hipLaunchKernelGGL(k_flatten_permute, dim3(grid_for((int64_t)rows * C * F, 256)), dim3(256), 0,
                     s, src, rows, C, F, dst);
  return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* src, int C, int K, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_f32, dim3(grid_for((int64_t)C * K, 256)), dim3(256), 0, s, src,
                     C, K, dst);
  return hipGetLastError();
}

hipError_t launch_concat3(const float* a, const float* b, const float* c, int n, float* dst,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_concat3, dim3(grid_for(3 * (int64_t)n, 256)), dim3(256), 0, s, a, b, c, n,
                     dst);
  return hipGetLastError();
}

}  // namespace lfm
}  // namespace ae
