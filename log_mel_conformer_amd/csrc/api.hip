// The C ABI of libae.so: argument validation, packing plans, workspace
// layout, model tables and the launch sequence of the encoder forward
// (egemma2_audio.rs: num_frames, num_tokens, AudioTower::load,
// soft_tokens, encode_locked).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

using namespace ae;

struct ae_model {
  ae_config cfg;
  ae_dtype dt;
  int device;
  ae_weights w;
  std::vector<ae_layer_weights> layers;
  int head_dim, left, n_dist;
  float q_scale, k_scale;
  void* R = nullptr;          // [layers][n_dist][hidden], storage type
  float* colscale = nullptr;  // [layers][3 hidden]
  void* conv1r = nullptr;     // [32][9 * 128], model dtype
  void* conv0f = nullptr;     // bf16 models: conv0's centred taps as matrix-core fragments
  float* dwt = nullptr;       // [layers][conv_kernel][hidden]: light-conv taps transposed
  std::vector<int> attn_nout;  // distinct input clamps among q, k, v (1..3)
  bool q8 = false;             // int8 projections, widened per forward
  std::vector<ae_layer_scales> scales;
};

namespace ae {

static thread_local std::string g_err;

ae_status set_error(ae_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// ------------------------------------------------------------- timing
namespace {
struct Timing {
  std::mutex mu;
  int cls = -1;
  std::vector<hipEvent_t> ev;  // pairs
  size_t used = 0;
  bool open = false;
};
Timing g_tm;
constexpr size_t kMaxTimed = 4096;
}  // namespace

void timing_begin(int cls, hipStream_t s) {
  if (cls != g_tm.cls) return;
  std::lock_guard<std::mutex> lk(g_tm.mu);
  if (g_tm.used >= kMaxTimed) return;
  if (g_tm.ev.size() < 2 * (g_tm.used + 1)) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) { hipEventDestroy(a); return; }
    g_tm.ev.push_back(a);
    g_tm.ev.push_back(b);
  }
  hipEventRecord(g_tm.ev[2 * g_tm.used], s);
  g_tm.open = true;
}

void timing_end(int cls, hipStream_t s) {
  if (cls != g_tm.cls) return;
  std::lock_guard<std::mutex> lk(g_tm.mu);
  if (!g_tm.open) return;
  hipEventRecord(g_tm.ev[2 * g_tm.used + 1], s);
  g_tm.used++;
  g_tm.open = false;
}

// ------------------------------------------------------ small kernels
namespace {

// Host tables ride in the kernel arguments (captured at launch, so the
// host array may be reused at once and no pinned staging is needed); 256
// values a launch keeps a 256-clip plan's four tables to five launches.
constexpr int kI64Chunk = 256;
struct I64Chunk {
  int64_t v[kI64Chunk];
};

__global__ void k_write_i64(int64_t* dst, I64Chunk c, int count) {
  const int i = threadIdx.x;
  if (i < count) dst[i] = c.v[i];
}

__global__ void k_token_index(const int64_t* token_off, int B, int64_t n, int32_t* tok_pos,
                              int32_t* tok_clip) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n) return;
  const int c = find_clip(token_off, B, g);
  tok_pos[g] = (int32_t)(g - token_off[c]);
  tok_clip[g] = c;
}

// R[dist][j] = sum_i PE[dist][i] rel_k[j][i]; PE row dist = [sin(dist inv_i),
// cos(dist inv_i)], inv_i = exp(-i ln(10000) / (d/2 - 1)). One wavefront per
// output, double accumulation (a one-off table), stored in the model's
// storage type (bf16 models round it).
template <typename T>
__global__ void k_relative_keys(const T* __restrict__ W, int d, int n_dist, T* __restrict__ R) {
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (int64_t)n_dist * d) return;
  const int dist = (int)(wid / d), j = (int)(wid - (int64_t)dist * d);
  const int nts = d / 2;
  const double incr = log(10000.0) / (double)(nts > 2 ? nts - 1 : 1);
  double acc = 0.0;
  for (int i = lane; i < d; i += 64) {
    const int f = i < nts ? i : i - nts;
    const double ang = (double)dist * exp(-(double)f * incr);
    const double pe = i < nts ? sin(ang) : cos(ang);
    acc += pe * (double)to_f32(W[(int64_t)j * d + i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) R[wid] = from_f32<T>((float)acc);
}

// q columns: q_scale * softplus(per_dim_scale[j % head_dim]) (torch's
// softplus: x above 20 passes through); k columns: k_scale; v columns: 1.
__global__ void k_qkv_scale(const float* pds, int d, int hd, float q_scale, float k_scale,
                            float* colscale) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= 3 * d) return;
  float v = 1.0f;
  if (j < d) {
    const float x = pds[j % hd];
    const float sp = x > 20.0f ? x : (float)log1p(exp((double)x));
    v = q_scale * sp;
  } else if (j < 2 * d) {
    v = k_scale;
  }
  colscale[j] = v;
}

// [32][128][3][3] -> [32][(dt*3 + df)*128 + ci]
template <typename T>
__global__ void k_conv1_reorder(const T* __restrict__ w, T* __restrict__ wr) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= kC1 * kC0 * 9) return;
  const int co = i / (kC0 * 9), rem = i - co * kC0 * 9;
  const int ci = rem / 9, tap = rem - ci * 9;
  wr[co * kC0 * 9 + tap * kC0 + ci] = w[i];
}

// Widening of int8 projections: out[r][c] = bf16(float(q[r][c]) * s[r]),
// for up to 10 matrices in one launch. A block covers 4096 consecutive
// values of one matrix (16 a thread); its matrix comes from the block index
// through a uniform scan of the prefix of block counts, and each thread's
// row from one 32-bit division.
struct DqJobs {
  const int8_t* q[10];
  const float* s[10];
  bf16* out[10];
  int cols[10];
  int64_t first[11];  // prefix of the jobs' 16-value chunk counts
  int bfirst[11];     // prefix of the jobs' block counts
};

constexpr int kDqBlockValues = 4096;

__global__ void __launch_bounds__(256) k_dequant(DqJobs j) {
  const int b = blockIdx.x;
  int k = 0;
  while (b >= j.bfirst[k + 1]) ++k;  // uniform
  const uint32_t n = (uint32_t)((j.first[k + 1] - j.first[k]) * 16);
  const uint32_t e = (uint32_t)(b - j.bfirst[k]) * kDqBlockValues + threadIdx.x * 16u;
  if (e >= n) return;
  const uint32_t r = e / (uint32_t)j.cols[k];
  const float sc = j.s[k][r];
  const int4 v = *(const int4*)(j.q[k] + e);
  const int words[4] = {v.x, v.y, v.z, v.w};
  bf16x8 o0, o1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o0[i] = (bf16)((float)(int8_t)(words[i / 4] >> (8 * (i & 3))) * sc);
    o1[i] = (bf16)((float)(int8_t)(words[2 + i / 4] >> (8 * (i & 3))) * sc);
  }
  *(bf16x8*)(j.out[k] + e) = o0;
  *(bf16x8*)(j.out[k] + e + 8) = o1;
}

__global__ void k_transpose_taps(const float* w, int d, int K, float* wt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d * K) return;
  const int c = i / K, k = i - c * K;
  wt[k * d + c] = w[i];
}

}  // namespace

hipError_t launch_transpose_taps(const float* w, int d, int K, float* wt, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_taps, dim3((d * K + 255) / 256), dim3(256), 0, s, w, d, K, wt);
  return hipGetLastError();
}

hipError_t launch_dequant(const DqJobs& jobs, hipStream_t s) {
  if (jobs.first[10] == 0) return hipSuccess;
  DqJobs j = jobs;
  j.bfirst[0] = 0;
  for (int k = 0; k < 10; ++k) {
    const int64_t vals = (j.first[k + 1] - j.first[k]) * 16;
    if (vals > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
    j.bfirst[k + 1] = j.bfirst[k] + (int)((vals + kDqBlockValues - 1) / kDqBlockValues);
  }
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)j.bfirst[10]), dim3(256), 0, s, j);
  return hipGetLastError();
}

hipError_t launch_write_i64(int64_t* dst, const int64_t* vals, int count, hipStream_t s) {
  for (int off = 0; off < count; off += kI64Chunk) {
    I64Chunk c;
    const int k = count - off < kI64Chunk ? count - off : kI64Chunk;
    memcpy(c.v, vals + off, sizeof(int64_t) * k);
    hipLaunchKernelGGL(k_write_i64, dim3(1), dim3(kI64Chunk), 0, s, dst + off, c, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_token_index(const int64_t* token_off, int B, int64_t n, int32_t* tok_pos,
                              int32_t* tok_clip, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_token_index, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, token_off,
                     B, n, tok_pos, tok_clip);
  return hipGetLastError();
}

hipError_t launch_relative_keys(ae_dtype dt, const void* rel_k, int d, int n_dist, void* R,
                                hipStream_t s) {
  const unsigned grid = (unsigned)(((int64_t)n_dist * d + 3) / 4);
  if (dt == AE_BF16)
    hipLaunchKernelGGL(k_relative_keys<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)rel_k, d,
                       n_dist, (bf16*)R);
  else
    hipLaunchKernelGGL(k_relative_keys<float>, dim3(grid), dim3(256), 0, s, (const float*)rel_k,
                       d, n_dist, (float*)R);
  return hipGetLastError();
}

hipError_t launch_qkv_scale(const float* pds, int d, int hd, float q_scale, float k_scale,
                            float* colscale, hipStream_t s) {
  hipLaunchKernelGGL(k_qkv_scale, dim3((3 * d + 255) / 256), dim3(256), 0, s, pds, d, hd, q_scale,
                     k_scale, colscale);
  return hipGetLastError();
}

hipError_t launch_conv1_reorder(ae_dtype dt, const void* w1, void* w1r, hipStream_t s) {
  const int n = kC1 * kC0 * 9;
  if (dt == AE_BF16)
    hipLaunchKernelGGL(k_conv1_reorder<bf16>, dim3((n + 255) / 256), dim3(256), 0, s,
                       (const bf16*)w1, (bf16*)w1r);
  else
    hipLaunchKernelGGL(k_conv1_reorder<float>, dim3((n + 255) / 256), dim3(256), 0, s,
                       (const float*)w1, (float*)w1r);
  return hipGetLastError();
}

}  // namespace ae

// =================================================================== host

namespace {

int64_t frames_of(int64_t n) {
  if (n > kMaxSamples) n = kMaxSamples;
  return n <= kHop ? 0 : (n - kHop + kHop - 1) / kHop;
}
int64_t half_up(int64_t x) { return (x + 1) / 2; }

struct Plan {
  int B = 0;
  std::vector<int64_t> sample_off, frame_off, row_off, token_off;
  int64_t frames() const { return frame_off[B]; }
  int64_t rows() const { return row_off[B]; }
  int64_t tokens() const { return token_off[B]; }
};

void plan_from_frames(Plan& p) {
  p.row_off.assign(p.B + 1, 0);
  p.token_off.assign(p.B + 1, 0);
  for (int i = 0; i < p.B; ++i) {
    const int64_t F = p.frame_off[i + 1] - p.frame_off[i];
    const int64_t T1 = half_up(F);
    p.row_off[i + 1] = p.row_off[i] + T1;
    p.token_off[i + 1] = p.token_off[i] + half_up(T1);
  }
}

ae_status plan_from_samples(const int64_t* sample_off, int B, Plan& p) {
  if (B < 0) return set_error(AE_ERR_INVALID, "B must be >= 0");
  if (B > 0 && !sample_off) return set_error(AE_ERR_INVALID, "sample_off is NULL");
  p.B = B;
  if (sample_off) p.sample_off.assign(sample_off, sample_off + B + 1);
  else p.sample_off.assign(1, 0);
  if (B > 0 && p.sample_off[0] < 0) return set_error(AE_ERR_INVALID, "sample_off[0] < 0");
  p.frame_off.assign(B + 1, 0);
  for (int i = 0; i < B; ++i) {
    const int64_t n = p.sample_off[i + 1] - p.sample_off[i];
    if (n < 0) return set_error(AE_ERR_INVALID, "sample_off must be non-decreasing");
    p.frame_off[i + 1] = p.frame_off[i] + frames_of(n);
  }
  plan_from_frames(p);
  return AE_OK;
}

ae_status plan_from_frame_off(const int64_t* frame_off, int B, Plan& p) {
  if (B < 0) return set_error(AE_ERR_INVALID, "B must be >= 0");
  if (B > 0 && !frame_off) return set_error(AE_ERR_INVALID, "frame_off is NULL");
  p.B = B;
  if (frame_off) p.frame_off.assign(frame_off, frame_off + B + 1);
  else p.frame_off.assign(1, 0);
  if (B > 0 && p.frame_off[0] != 0) return set_error(AE_ERR_INVALID, "frame_off[0] must be 0");
  for (int i = 0; i < B; ++i) {
    const int64_t F = p.frame_off[i + 1] - p.frame_off[i];
    if (F < 0) return set_error(AE_ERR_INVALID, "frame_off must be non-decreasing");
    if (F > frames_of(kMaxSamples))
      return set_error(AE_ERR_SHAPE, "a clip has more than 2999 frames (30 s)");
  }
  p.sample_off.assign(B + 1, 0);
  plan_from_frames(p);
  return AE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Ws {
  int64_t* tab = nullptr;  // [4][B+1]: samples, frames, conv0 rows, tokens
  int32_t *tok_pos = nullptr, *tok_clip = nullptr;
  float* mel = nullptr;
  void* y0 = nullptr;
  void* x1 = nullptr;
  float* h = nullptr;
  void* a[3] = {nullptr, nullptr, nullptr};
  void* u = nullptr;
  void* y = nullptr;  // GEMM outputs feeding a post-norm, model dtype
  void* y2 = nullptr;  // bf16 models: the second output of a row-kernel pair
  void* qkv = nullptr;
  void* o = nullptr;
  void* g = nullptr;
  void* c = nullptr;
  float* o1 = nullptr;
  void* on = nullptr;
  void* dq = nullptr;  // int8 models: one layer's projections widened to bf16
  float* part = nullptr;  // float models: partial tiles of FFN W2's K split
  size_t part_bytes = 0;
  size_t total = 0;
};

// Offsets of every buffer for B clips, F frames and T tokens (conv0 rows
// bounded by (F + B) / 2 + 1). With base == nullptr only `total` is meaningful.
Ws ws_layout(const ae_model* m, int B, int64_t F, int64_t T, char* base) {
  Ws w;
  const size_t es = m->dt == AE_BF16 ? 2 : 4;
  const size_t d = m->cfg.hidden;
  const int64_t T1 = (F + B) / 2 + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.tab = (int64_t*)take(sizeof(int64_t) * 4 * (size_t)(B + 1));
  w.tok_pos = (int32_t*)take(sizeof(int32_t) * (size_t)T);
  w.tok_clip = (int32_t*)take(sizeof(int32_t) * (size_t)T);
  w.mel = (float*)take(sizeof(float) * (size_t)F * kMels);
  // the conv0 plane: fp32 models only (bf16 models keep it on chip)
  w.y0 = m->dt == AE_BF16 ? nullptr : take(es * (size_t)T1 * kF1 * kC0);
  w.x1 = take(es * (size_t)T * kC1 * kF2);
  w.h = (float*)take(sizeof(float) * (size_t)T * d);
  for (int i = 0; i < 3; ++i) w.a[i] = take(es * (size_t)T * d);
  w.u = take(es * (size_t)T * m->cfg.ff);
  w.y = take(es * (size_t)T * d);
  if (m->dt == AE_BF16) w.y2 = take(es * (size_t)T * d);
  w.qkv = take(es * (size_t)T * 3 * d);
  w.o = take(es * (size_t)T * d);
  w.g = take(es * (size_t)T * d);
  w.c = take(es * (size_t)T * d);
  w.o1 = (float*)take(sizeof(float) * (size_t)T * m->cfg.out_hidden);
  w.on = take(es * (size_t)T * m->cfg.out_hidden);
  if (m->q8) w.dq = take(2 * (4 * (size_t)m->cfg.ff * d + 7 * d * d));
  if (m->dt != AE_BF16) {
    // the K-split area of the float projections: the largest any of them
    // needs (with the tower's sizes only FFN W2, K = ff, splits)
    const int di = (int)d, ff = m->cfg.ff, oh = m->cfg.out_hidden, od = m->cfg.out_dim;
    const int shapes[8][2] = {{ff, di}, {di, ff}, {3 * di, di}, {2 * di, di},
                              {di, di}, {di, kC1 * kF2}, {oh, di}, {od, oh}};  // {N, K}
    for (const auto& nk : shapes)
      w.part_bytes = std::max(w.part_bytes, gemm_f32_part_bytes(T, nk[0], nk[1]));
    if (w.part_bytes) w.part = (float*)take(w.part_bytes);
  }
  w.total = off;
  return w;
}

#define AE_LAUNCH(cls, stream, expr)                                                   \
  do {                                                                                 \
    timing_begin((cls), (stream));                                                     \
    hipError_t e_ = (expr);                                                            \
    timing_end((cls), (stream));                                                       \
    if (e_ != hipSuccess)                                                              \
      return set_error(AE_ERR_HIP, std::string("launch failed: ") + #expr + ": " +     \
                                       hipGetErrorString(e_));                         \
  } while (0)

const float kInf = INFINITY;

// w: the call's workspace, whose K-split area (float models) the GEMM may use
GemmParams gemm_params(const Ws& w, int M, int N, int K, const void* A, int lda, const void* B,
                       int ldb, void* C, int ldc) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.part = w.part;
  p.part_bytes = w.part_bytes;
  p.M = M; p.N = N; p.K = K;
  p.A[0] = p.A[1] = p.A[2] = A;
  p.lda = lda;
  p.Bm[0] = p.Bm[1] = p.Bm[2] = B;
  p.seg_n = N;
  p.ldb = ldb;
  p.C = C;
  p.ldc = ldc;
  for (int i = 0; i < 3; ++i) { p.olo[i] = -kInf; p.ohi[i] = kInf; }
  p.nlo = -kInf; p.nhi = kInf;
  p.rscale = 1.0f;
  return p;
}

void set_out_clip(GemmParams& p, const ae_clip& c) {
  for (int i = 0; i < 3; ++i) { p.olo[i] = c.out_lo; p.ohi[i] = c.out_hi; }
}

RowNormParams rn_params(int64_t n, int d, float* h) {
  RowNormParams r;
  memset(&r, 0, sizeof(r));
  r.n = n; r.d = d; r.h = h; r.scale = 1.0f;
  for (int i = 0; i < 3; ++i) { r.lo[i] = -kInf; r.hi[i] = kInf; }
  return r;
}

ae_status check_clip(const ae_clip& c, const char* name) {
  if (!(c.in_lo <= c.in_hi) || !(c.out_lo <= c.out_hi))
    return set_error(AE_ERR_INVALID, std::string("clamp bounds of ") + name +
                                         " must satisfy lo <= hi (and not be NaN)");
  return AE_OK;
}

bool same_in(const ae_clip& a, const ae_clip& b) { return a.in_lo == b.in_lo && a.in_hi == b.in_hi; }

// Subsampler + input projection over the plan `pl` (tables already on the
// device in w.tab). Output x: [tokens][hidden] float.
ae_status subsample_impl(const ae_model* m, const float* mel, const Plan& pl, const Ws& w,
                         float* x, hipStream_t s) {
  const int B = pl.B;
  const int64_t* d_frame = w.tab + (B + 1);
  const int64_t* d_row = w.tab + 2 * (B + 1);
  const int64_t* d_tok = w.tab + 3 * (B + 1);
  const int64_t T = pl.tokens();
  if (T == 0) return AE_OK;
  AE_HIP_TRY(launch_token_index(d_tok, B, T, w.tok_pos, w.tok_clip, s));
  if (m->dt == AE_BF16) {
    // both convolutions in one pass, the conv0 plane kept on chip
    AE_LAUNCH(AE_K_CONV1, s, launch_subsample_fused(mel, d_frame, d_row, w.tok_pos, w.tok_clip, T,
                                                    m->conv0f, m->w.ln0, m->conv1r, m->w.ln1,
                                                    w.x1, s));
  } else {
    AE_LAUNCH(AE_K_CONV0, s, launch_conv0(m->dt, mel, d_frame, d_row, B, pl.rows(), m->w.conv0,
                                          m->w.ln0, w.y0, s));
    GemmParams p = gemm_params(w, (int)(T * 32), kC1, kC0 * 9, nullptr, 0, m->conv1r, kC0 * 9,
                               w.x1, kC1);
    p.y0 = w.y0;
    p.row_off = d_row;
    p.tok_pos = w.tok_pos;
    p.tok_clip = w.tok_clip;
    p.n_tok = (int)T;
    p.gain = m->w.ln1;
    AE_LAUNCH(AE_K_CONV1, s, launch_gemm(m->dt, EPI_LNRELU, A_CONV1, true, p, s));
  }
  const int d = m->cfg.hidden;
  GemmParams q =
      gemm_params(w, (int)T, d, kC1 * kF2, w.x1, kC1 * kF2, m->w.in_proj, kC1 * kF2, x, d);
  AE_LAUNCH(AE_K_GEMM_HEAD, s, launch_gemm(m->dt, EPI_STORE, A_PLAIN, false, q, s));
  return AE_OK;
}

// One Conformer layer on h [n][d]. If `pre_done`, w.a[0] already holds
// clamp(rms(h) * ff1_pre); if `next` is given, the layer's last row kernel
// also writes the next layer's first input that way.
ae_status layer_impl(const ae_model* m, int l, float* h, const int32_t* pos, int64_t n,
                     const Ws& w, hipStream_t s, bool pre_done, const ae_layer_weights* next,
                     void* h_copy) {
  const int d = m->cfg.hidden, ff = m->cfg.ff;
  const int M = (int)n;
  const ae_dtype dt = m->dt;
  const bool lowp = dt == AE_BF16;
  const size_t es = lowp ? 2 : 4;
  if (n == 0) return AE_OK;
  // int8 models: widen this layer's ten projections into the workspace and
  // run the layer on the widened copies
  ae_layer_weights Lq = m->layers[l];
  if (m->q8) {
    const ae_layer_weights& L0 = m->layers[l];
    const ae_layer_scales& S = m->scales[l];
    const void* qs[10] = {L0.ff1_w1, L0.ff1_w2, L0.q, L0.k, L0.v, L0.post, L0.lc_start, L0.lc_end,
                          L0.ff2_w1, L0.ff2_w2};
    const float* ss[10] = {S.ff1_w1, S.ff1_w2, S.q, S.k, S.v, S.post, S.lc_start, S.lc_end,
                           S.ff2_w1, S.ff2_w2};
    const int rows[10] = {ff, d, d, d, d, d, 2 * d, d, ff, d};
    const int cols[10] = {d, ff, d, d, d, d, d, d, d, ff};
    const void** dst[10] = {&Lq.ff1_w1, &Lq.ff1_w2, &Lq.q, &Lq.k, &Lq.v, &Lq.post, &Lq.lc_start,
                            &Lq.lc_end, &Lq.ff2_w1, &Lq.ff2_w2};
    DqJobs j;
    bf16* o = (bf16*)w.dq;
    j.first[0] = 0;
    for (int i = 0; i < 10; ++i) {
      j.q[i] = (const int8_t*)qs[i];
      j.s[i] = ss[i];
      j.out[i] = o;
      j.cols[i] = cols[i];
      j.first[i + 1] = j.first[i] + (int64_t)rows[i] * cols[i] / 16;
      *dst[i] = o;
      o += (size_t)rows[i] * cols[i];
    }
    AE_LAUNCH(AE_K_DEQUANT, s, launch_dequant(j, s));
  }
  const ae_layer_weights& L = Lq;

  auto ffn = [&](const float* pre, const void* w1, const ae_clip& c1, const void* w2,
                 const ae_clip& c2, bool done, void* yout) -> ae_status {
    if (!done) {
      RowNormParams r = rn_params(n, d, h);
      r.w_next = pre; r.n_out = 1; r.a[0] = w.a[0]; r.lo[0] = c1.in_lo; r.hi[0] = c1.in_hi;
      AE_LAUNCH(AE_K_ROWNORM, s, launch_rownorm(dt, r, s));
    }
    GemmParams p1 = gemm_params(w, M, ff, d, w.a[0], d, w1, d, w.u, ff);
    set_out_clip(p1, c1);
    p1.nlo = c2.in_lo; p1.nhi = c2.in_hi;
    AE_LAUNCH(AE_K_GEMM_FFN1, s, launch_gemm(dt, EPI_SILU, A_PLAIN, lowp, p1, s));
    GemmParams p2 = gemm_params(w, M, d, ff, w.u, ff, w2, ff, yout, d);
    set_out_clip(p2, c2);
    AE_LAUNCH(AE_K_GEMM_FFN2, s, launch_gemm(dt, EPI_STORE, A_PLAIN, lowp, p2, s));
    return AE_OK;
  };

  // In bf16 models the row kernels run in pairs (after FFN 1 and after the
  // attention; after the light conv and after FFN 2): the first of a pair
  // leaves h unwritten and the second applies both residual updates, its
  // own GEMM output in y2 and the first's still in y.
  void* y_second = lowp ? w.y2 : w.y;
  // ---- FFN 1
  ae_status st =
      ffn(L.ff1_pre, L.ff1_w1, L.ff1_w1_clip, L.ff1_w2, L.ff1_w2_clip, pre_done, w.y);
  if (st != AE_OK) return st;
  // residual + attention pre-norm (q, k, v inputs; distinct clamps only if needed)
  {
    RowNormParams r = rn_params(n, d, h);
    r.y = w.y; r.scale = m->cfg.residual_weight; r.w_post = L.ff1_post;
    r.skip_h = lowp;
    r.w_next = L.attn_pre;
    const ae_clip* cl[3] = {&L.q_clip, &L.k_clip, &L.v_clip};
    r.n_out = m->attn_nout[l];
    for (int i = 0; i < 3; ++i) {
      const int src = (r.n_out == 1) ? 0 : i;
      r.a[i] = w.a[i];
      r.lo[i] = cl[src]->in_lo;
      r.hi[i] = cl[src]->in_hi;
    }
    AE_LAUNCH(AE_K_ROWNORM, s, launch_rownorm(dt, r, s));
  }
  // ---- attention: fused q|k|v projection with per-column q/k scaling
  {
    GemmParams p = gemm_params(w, M, 3 * d, d, w.a[0], d, L.q, d, w.qkv, 3 * d);
    const int nout = m->attn_nout[l];
    p.A[1] = nout == 1 ? w.a[0] : w.a[1];
    p.A[2] = nout == 1 ? w.a[0] : w.a[2];
    p.Bm[1] = L.k;
    p.Bm[2] = L.v;
    p.seg_n = d;
    const ae_clip* cl[3] = {&L.q_clip, &L.k_clip, &L.v_clip};
    for (int i = 0; i < 3; ++i) { p.olo[i] = cl[i]->out_lo; p.ohi[i] = cl[i]->out_hi; }
    p.colscale = m->colscale + (size_t)l * 3 * d;
    AE_LAUNCH(AE_K_GEMM_QKV, s, launch_gemm(dt, EPI_STORE, A_PLAIN, lowp, p, s));
  }
  AE_LAUNCH(AE_K_ATTN, s,
            launch_attention(dt, w.qkv, (const char*)m->R + es * l * m->n_dist * d, pos, n, d,
                             m->cfg.heads, m->left, m->cfg.softcap, L.post_clip.in_lo,
                             L.post_clip.in_hi, w.o, s));
  {
    GemmParams p = gemm_params(w, M, d, d, w.o, d, L.post, d, y_second, d);
    set_out_clip(p, L.post_clip);
    AE_LAUNCH(AE_K_GEMM_POST, s, launch_gemm(dt, EPI_STORE, A_PLAIN, lowp, p, s));
  }
  {
    RowNormParams r = rn_params(n, d, h);
    if (lowp) {
      r.y0 = w.y; r.scale0 = m->cfg.residual_weight; r.w_post0 = L.ff1_post;
    }
    r.y = y_second; r.scale = 1.0f; r.w_post = L.attn_post;
    r.w_next = L.lc_pre; r.n_out = 1; r.a[0] = w.a[0];
    r.lo[0] = L.lc_start_clip.in_lo; r.hi[0] = L.lc_start_clip.in_hi;
    AE_LAUNCH(AE_K_ROWNORM, s, launch_rownorm(dt, r, s));
  }
  // ---- light conv
  {
    GemmParams p = gemm_params(w, M, 2 * d, d, w.a[0], d, L.lc_start, d, w.g, d);
    set_out_clip(p, L.lc_start_clip);
    p.glu_d = d;
    AE_LAUNCH(AE_K_GEMM_LCSTART, s, launch_gemm(dt, EPI_GLU, A_PLAIN, lowp, p, s));
  }
  AE_LAUNCH(AE_K_LCONV, s,
            launch_lconv(dt, w.g, m->dwt + (size_t)l * m->cfg.conv_kernel * d, m->cfg.conv_kernel,
                         L.lc_norm, pos, n, d,
                         L.lc_end_clip.in_lo, L.lc_end_clip.in_hi, w.c, s));
  // linear_end stores its clamped output; FFN 2's pre-norm row kernel adds
  // it to h (the light conv's residual has no norm) while the row is in
  // registers, so the GEMM's epilogue does not wait on reading h
  {
    GemmParams p = gemm_params(w, M, d, d, w.c, d, L.lc_end, d, w.y, d);
    set_out_clip(p, L.lc_end_clip);
    AE_LAUNCH(AE_K_GEMM_LCEND, s, launch_gemm(dt, EPI_STORE, A_PLAIN, lowp, p, s));
  }
  {
    RowNormParams r = rn_params(n, d, h);
    r.y = w.y; r.scale = 1.0f;
    r.skip_h = lowp;
    r.w_next = L.ff2_pre; r.n_out = 1; r.a[0] = w.a[0];
    r.lo[0] = L.ff2_w1_clip.in_lo; r.hi[0] = L.ff2_w1_clip.in_hi;
    AE_LAUNCH(AE_K_ROWNORM, s, launch_rownorm(dt, r, s));
  }
  // ---- FFN 2
  st = ffn(L.ff2_pre, L.ff2_w1, L.ff2_w1_clip, L.ff2_w2, L.ff2_w2_clip, true, y_second);
  if (st != AE_OK) return st;
  {
    RowNormParams r = rn_params(n, d, h);
    if (lowp) {
      r.y0 = w.y; r.scale0 = 1.0f;  // the light conv's plain residual add
    }
    r.y = y_second; r.scale = m->cfg.residual_weight; r.w_post = L.ff2_post;
    r.w_out = L.norm_out;
    r.h_copy = h_copy;
    if (next) {
      r.w_next = next->ff1_pre; r.n_out = 1; r.a[0] = w.a[0];
      r.lo[0] = next->ff1_w1_clip.in_lo; r.hi[0] = next->ff1_w1_clip.in_hi;
    }
    AE_LAUNCH(AE_K_ROWNORM, s, launch_rownorm(dt, r, s));
  }
  return AE_OK;
}

ae_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need > ws_bytes)
    return set_error(AE_ERR_CAPACITY, "workspace of " + std::to_string(ws_bytes) +
                                          " bytes is smaller than the " + std::to_string(need) +
                                          " bytes needed");
  if (need > 0 && !ws) return set_error(AE_ERR_INVALID, "workspace is NULL");
  if (((uintptr_t)ws & 255) != 0) return set_error(AE_ERR_INVALID, "workspace must be 256-byte aligned");
  return AE_OK;
}

ae_status check_sizes(const ae_model* m, int64_t T, int64_t F) {
  if (T * 32 + 256 > (int64_t)INT32_MAX || F * kMels > (int64_t)INT32_MAX * 8)
    return set_error(AE_ERR_CAPACITY, "batch too large for 32-bit row indices");
  (void)m;
  return AE_OK;
}

ae_status write_tab(const Plan& pl, const Ws& w, hipStream_t s) {
  std::vector<int64_t> tab;
  tab.insert(tab.end(), pl.sample_off.begin(), pl.sample_off.end());
  tab.insert(tab.end(), pl.frame_off.begin(), pl.frame_off.end());
  tab.insert(tab.end(), pl.row_off.begin(), pl.row_off.end());
  tab.insert(tab.end(), pl.token_off.begin(), pl.token_off.end());
  AE_HIP_TRY(launch_write_i64(w.tab, tab.data(), (int)tab.size(), s));
  return AE_OK;
}

ae_status encode_impl(const ae_model* m, const float* wave, const Plan& pl, float* out,
                      float* const* trace, const Ws& w, hipStream_t s);

}  // namespace

// Scratch memory of ae_encode_static, for callers that cannot allocate: one
// copy per device, held until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in
// symbol); it takes the device address from hipGetSymbolAddress, once per
// device, and uses that.
static __device__ __align__(256) unsigned char scratch[AE_STATIC_SCRATCH_BYTES];

namespace {

constexpr size_t kStaticScratchBytes = AE_STATIC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on device `dev` (the current device).
ae_status static_scratch(int dev, char** out) {
  if (dev < 0 || dev >= kMaxScratchDevices)
    return set_error(AE_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(AE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                       hipGetErrorString(e));
    if (((uintptr_t)p & 255) != 0)
      return set_error(AE_ERR_HIP, "static scratch is not 256-byte aligned");
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return AE_OK;
}

}  // namespace

// ================================================================ C ABI
extern "C" {

const char* ae_last_error(void) { return g_err.c_str(); }

void ae_config_default(ae_config* c) {
  if (!c) return;
  c->hidden = 1024;
  c->heads = 8;
  c->layers = 12;
  c->ff = 4096;
  c->conv_kernel = 5;
  c->chunk = 12;
  c->ctx_left = 13;
  c->ctx_right = 0;
  c->softcap = 50.0f;
  c->residual_weight = 0.5f;
  c->out_hidden = 1536;
  c->out_dim = 512;
}

int64_t ae_num_frames(int64_t n) { return n < 0 ? 0 : frames_of(n); }
int64_t ae_num_tokens(int64_t n) { return half_up(half_up(ae_num_frames(n))); }

ae_status ae_plan(const int64_t* n_samples, int32_t B, int64_t* sample_off, int64_t* frame_off,
                  int64_t* row_off, int64_t* token_off) {
  if (B < 0) return set_error(AE_ERR_INVALID, "B must be >= 0");
  if (B > 0 && !n_samples) return set_error(AE_ERR_INVALID, "n_samples is NULL");
  int64_t so = 0, fo = 0, ro = 0, to = 0;
  for (int i = 0; i <= B; ++i) {
    if (sample_off) sample_off[i] = so;
    if (frame_off) frame_off[i] = fo;
    if (row_off) row_off[i] = ro;
    if (token_off) token_off[i] = to;
    if (i == B) break;
    const int64_t n = n_samples[i];
    if (n < 0) return set_error(AE_ERR_INVALID, "negative clip length");
    const int64_t F = frames_of(n), T1 = half_up(F);
    so += n < kMaxSamples ? n : kMaxSamples;
    fo += F;
    ro += T1;
    to += half_up(T1);
  }
  return AE_OK;
}

ae_status ae_plan_frames(const int64_t* frame_off, int32_t B, int64_t* row_off,
                         int64_t* token_off) {
  Plan pl;
  ae_status st = plan_from_frame_off(frame_off, B, pl);
  if (st != AE_OK) return st;
  for (int i = 0; i <= B; ++i) {
    if (row_off) row_off[i] = pl.row_off[i];
    if (token_off) token_off[i] = pl.token_off[i];
  }
  return AE_OK;
}

ae_status ae_timing_enable(int32_t cls) {
  if (cls < -1 || cls >= AE_K_COUNT) return set_error(AE_ERR_INVALID, "unknown kernel class");
  std::lock_guard<std::mutex> lk(g_tm.mu);
  g_tm.cls = cls;
  g_tm.used = 0;
  g_tm.open = false;
  return AE_OK;
}

ae_status ae_timing_read(int64_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_tm.mu);
  double sum = 0.0;
  for (size_t i = 0; i < g_tm.used; ++i) {
    AE_HIP_TRY(hipEventSynchronize(g_tm.ev[2 * i + 1]));
    float ms = 0.f;
    AE_HIP_TRY(hipEventElapsedTime(&ms, g_tm.ev[2 * i], g_tm.ev[2 * i + 1]));
    sum += ms;
  }
  if (launches) *launches = (int64_t)g_tm.used;
  if (total_ms) *total_ms = sum;
  g_tm.used = 0;
  return AE_OK;
}

static ae_status model_create_impl(const ae_config* cfg, const ae_weights* w, ae_dtype dt,
                                   const ae_layer_scales* scales, ae_stream stream,
                                   ae_model** out) {
  if (!out) return set_error(AE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!cfg || !w) return set_error(AE_ERR_INVALID, "cfg and weights must not be NULL");
  if (dt != AE_F32 && dt != AE_BF16) return set_error(AE_ERR_INVALID, "unknown dtype");
  const ae_config& c = *cfg;
  if (scales) {
    if (dt != AE_BF16) return set_error(AE_ERR_UNSUPPORTED, "int8 projections need AE_BF16");
    if (c.layers < 1 || c.layers > 256) return set_error(AE_ERR_INVALID, "layers must be in 1..256");
    const char* sn[] = {"ff1_w1", "ff1_w2", "q", "k", "v", "post", "lc_start", "lc_end",
                        "ff2_w1", "ff2_w2"};
    for (int l = 0; l < c.layers; ++l) {
      const ae_layer_scales& S = scales[l];
      const float* sp[] = {S.ff1_w1, S.ff1_w2, S.q, S.k, S.v, S.post, S.lc_start, S.lc_end,
                           S.ff2_w1, S.ff2_w2};
      for (int i = 0; i < 10; ++i)
        if (!sp[i] || ((uintptr_t)sp[i] & 3) != 0)
          return set_error(AE_ERR_INVALID, "layer " + std::to_string(l) + ": scale of " + sn[i] +
                                               " is NULL or misaligned");
    }
  }
  if (c.ctx_right != 0)
    return set_error(AE_ERR_UNSUPPORTED, "attention_context_right " + std::to_string(c.ctx_right) +
                                             " is not supported (only 0)");
  if (c.hidden != 1024 || c.heads <= 0 || c.hidden % c.heads != 0 || c.hidden / c.heads != 128)
    return set_error(AE_ERR_UNSUPPORTED, "only hidden 1024 with 128-wide heads is implemented");
  if (c.layers < 1 || c.layers > 256) return set_error(AE_ERR_INVALID, "layers must be in 1..256");
  if (c.ff < 128 || c.ff % 128 != 0) return set_error(AE_ERR_UNSUPPORTED, "ff must be a multiple of 128");
  if (c.conv_kernel < 1 || c.conv_kernel > 16)
    return set_error(AE_ERR_UNSUPPORTED, "conv_kernel must be in 1..16");
  if (c.out_hidden != 1024 && c.out_hidden != 1536 && c.out_hidden != 2048)
    return set_error(AE_ERR_UNSUPPORTED, "out_hidden must be 1024, 1536 or 2048");
  if (c.out_dim < 128 || c.out_dim % 128 != 0)
    return set_error(AE_ERR_UNSUPPORTED, "out_dim must be a multiple of 128");
  const int left = c.ctx_left - 1 > 1 ? c.ctx_left - 1 : 1;
  const int n_dist = (c.chunk + c.ctx_left - 1 + c.ctx_right) / 2 + 1;
  if (n_dist < left)
    return set_error(AE_ERR_SHAPE, "relative position table shorter than the attention span");
  if (left > 12) return set_error(AE_ERR_UNSUPPORTED, "attention windows above 12 keys are not built");
  if (!(c.softcap > 0.f)) return set_error(AE_ERR_INVALID, "softcap must be positive");
  // pointers
  const void* top[] = {w->conv0, w->ln0, w->conv1, w->ln1, w->in_proj, w->out_proj, w->out_bias, w->embed};
  const char* top_n[] = {"conv0", "ln0", "conv1", "ln1", "in_proj", "out_proj", "out_bias", "embed"};
  for (int i = 0; i < 8; ++i)
    if (!top[i]) return set_error(AE_ERR_INVALID, std::string("weight ") + top_n[i] + " is NULL");
  if (!w->layers) return set_error(AE_ERR_INVALID, "weights.layers is NULL");
  for (int l = 0; l < c.layers; ++l) {
    const ae_layer_weights& L = w->layers[l];
    const void* ps[] = {L.ff1_pre, L.ff1_w1, L.ff1_w2, L.ff1_post, L.attn_pre, L.q, L.k, L.v,
                        L.post, L.attn_post, L.per_dim_scale, L.rel_k, L.lc_pre, L.lc_start,
                        L.lc_dw, L.lc_norm, L.lc_end, L.ff2_pre, L.ff2_w1, L.ff2_w2, L.ff2_post,
                        L.norm_out};
    const char* pn[] = {"ff1_pre", "ff1_w1", "ff1_w2", "ff1_post", "attn_pre", "q", "k", "v",
                        "post", "attn_post", "per_dim_scale", "rel_k", "lc_pre", "lc_start",
                        "lc_dw", "lc_norm", "lc_end", "ff2_pre", "ff2_w1", "ff2_w2", "ff2_post",
                        "norm_out"};
    for (int i = 0; i < 22; ++i) {
      if (!ps[i])
        return set_error(AE_ERR_INVALID, "layer " + std::to_string(l) + ": weight " + pn[i] + " is NULL");
      if (((uintptr_t)ps[i] & 15) != 0)
        return set_error(AE_ERR_INVALID, "layer " + std::to_string(l) + ": weight " + pn[i] +
                                             " is not 16-byte aligned");
    }
    const ae_clip* cs[] = {&L.ff1_w1_clip, &L.ff1_w2_clip, &L.q_clip, &L.k_clip, &L.v_clip,
                           &L.post_clip, &L.lc_start_clip, &L.lc_end_clip, &L.ff2_w1_clip, &L.ff2_w2_clip};
    const char* cn[] = {"ff1_w1", "ff1_w2", "q", "k", "v", "post", "lc_start", "lc_end", "ff2_w1", "ff2_w2"};
    for (int i = 0; i < 10; ++i) {
      ae_status st = check_clip(*cs[i], cn[i]);
      if (st != AE_OK) return st;
    }
  }
  for (int i = 0; i < 8; ++i)
    if (((uintptr_t)top[i] & 15) != 0)
      return set_error(AE_ERR_INVALID, std::string("weight ") + top_n[i] + " is not 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  AE_HIP_TRY(mel_tables_init());
  ae_model* m = new ae_model();
  m->cfg = c;
  m->dt = dt;
  if (scales) {
    m->q8 = true;
    m->scales.assign(scales, scales + c.layers);
  }
  hipGetDevice(&m->device);
  m->w = *w;
  m->layers.assign(w->layers, w->layers + c.layers);
  m->w.layers = nullptr;
  m->head_dim = c.hidden / c.heads;
  m->left = left;
  m->n_dist = n_dist;
  m->q_scale = (float)(pow((double)m->head_dim, -0.5) / M_LN2);
  m->k_scale = (float)(log(1.0 + M_E) / M_LN2);
  for (int l = 0; l < c.layers; ++l) {
    const ae_layer_weights& L = m->layers[l];
    int nout = 1;
    if (!same_in(L.q_clip, L.k_clip) || !same_in(L.q_clip, L.v_clip)) nout = 3;
    m->attn_nout.push_back(nout);
  }
  const size_t es = dt == AE_BF16 ? 2 : 4;
  auto fail = [&](hipError_t e, const char* what) {
    ae_model_destroy(m);
    return set_error(AE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  };
  hipError_t e;
  if ((e = hipMalloc(&m->R, es * c.layers * n_dist * c.hidden)) != hipSuccess)
    return fail(e, "hipMalloc(R)");
  if ((e = hipMalloc((void**)&m->colscale, sizeof(float) * (size_t)c.layers * 3 * c.hidden)) != hipSuccess)
    return fail(e, "hipMalloc(colscale)");
  if ((e = hipMalloc(&m->conv1r, es * kC1 * kC0 * 9)) != hipSuccess) return fail(e, "hipMalloc(conv1)");
  if ((e = hipMalloc((void**)&m->dwt, sizeof(float) * (size_t)c.layers * c.conv_kernel * c.hidden)) !=
      hipSuccess)
    return fail(e, "hipMalloc(taps)");
  for (int l = 0; l < c.layers; ++l) {
    const ae_layer_weights& L = m->layers[l];
    if ((e = launch_relative_keys(dt, L.rel_k, c.hidden, n_dist,
                                  (char*)m->R + es * l * n_dist * c.hidden, s)) != hipSuccess)
      return fail(e, "relative keys");
    if ((e = launch_transpose_taps(L.lc_dw, c.hidden, c.conv_kernel,
                                   m->dwt + (size_t)l * c.conv_kernel * c.hidden, s)) != hipSuccess)
      return fail(e, "light-conv taps");
    if ((e = launch_qkv_scale(L.per_dim_scale, c.hidden, m->head_dim, m->q_scale, m->k_scale,
                              m->colscale + (size_t)l * 3 * c.hidden, s)) != hipSuccess)
      return fail(e, "qkv scale");
  }
  if ((e = launch_conv1_reorder(dt, w->conv1, m->conv1r, s)) != hipSuccess) return fail(e, "conv1 reorder");
  if (dt == AE_BF16) {
    if ((e = hipMalloc(&m->conv0f, kConv0FragBytes)) != hipSuccess) return fail(e, "hipMalloc(conv0)");
    if ((e = launch_conv0_pack(w->conv0, m->conv0f, s)) != hipSuccess) return fail(e, "conv0 taps");
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail(e, "model tables");
  *out = m;
  return AE_OK;
}

ae_status ae_model_create(const ae_config* cfg, const ae_weights* w, ae_dtype dt,
                          ae_stream stream, ae_model** out) {
  return model_create_impl(cfg, w, dt, nullptr, stream, out);
}

ae_status ae_model_create_q8(const ae_config* cfg, const ae_weights* w,
                             const ae_layer_scales* scales, ae_stream stream, ae_model** out) {
  if (!scales) {
    if (out) *out = nullptr;
    return set_error(AE_ERR_INVALID, "scales must not be NULL");
  }
  return model_create_impl(cfg, w, AE_BF16, scales, stream, out);
}

void ae_model_destroy(ae_model* m) {
  if (!m) return;
  if (m->R) hipFree(m->R);
  if (m->colscale) hipFree(m->colscale);
  if (m->conv1r) hipFree(m->conv1r);
  if (m->conv0f) hipFree(m->conv0f);
  if (m->dwt) hipFree(m->dwt);
  delete m;
}

size_t ae_workspace_bytes(const ae_model* m, int32_t B, int64_t total_frames, int64_t total_tokens) {
  if (!m || B < 0 || total_frames < 0 || total_tokens < 0) return 0;
  return ws_layout(m, B, total_frames, total_tokens, nullptr).total;
}

size_t ae_logmel_workspace_bytes(int32_t B) {
  if (B < 0) return 0;
  return align256(sizeof(int64_t) * 4 * (size_t)(B + 1));
}

ae_status ae_logmel(const float* wave, const int64_t* sample_off, int32_t B, float* mel, void* ws,
                    size_t ws_bytes, ae_stream stream) {
  Plan pl;
  ae_status st = plan_from_samples(sample_off, B, pl);
  if (st != AE_OK) return st;
  if (pl.frames() == 0) return AE_OK;
  if (!wave || !mel) return set_error(AE_ERR_INVALID, "wave and mel must not be NULL");
  st = check_ws(ws, ws_bytes, ae_logmel_workspace_bytes(B));
  if (st != AE_OK) return st;
  if (pl.frames() * kMels > (int64_t)INT32_MAX * 64)
    return set_error(AE_ERR_CAPACITY, "too many frames");
  hipStream_t s = (hipStream_t)stream;
  AE_HIP_TRY(mel_tables_init());
  Ws w;
  w.tab = (int64_t*)ws;
  st = write_tab(pl, w, s);
  if (st != AE_OK) return st;
  AE_LAUNCH(AE_K_LOGMEL, s, launch_logmel(wave, w.tab, w.tab + (B + 1), B, pl.frames(), mel, s));
  return AE_OK;
}

ae_status ae_subsample(const ae_model* m, const float* mel, const int64_t* frame_off, int32_t B,
                       float* x, void* ws, size_t ws_bytes, ae_stream stream) {
  if (!m) return set_error(AE_ERR_INVALID, "model is NULL");
  Plan pl;
  ae_status st = plan_from_frame_off(frame_off, B, pl);
  if (st != AE_OK) return st;
  if (pl.tokens() == 0) return AE_OK;
  if (!mel || !x) return set_error(AE_ERR_INVALID, "mel and x must not be NULL");
  if ((st = check_sizes(m, pl.tokens(), pl.frames())) != AE_OK) return st;
  Ws w = ws_layout(m, B, pl.frames(), pl.tokens(), (char*)ws);
  if ((st = check_ws(ws, ws_bytes, w.total)) != AE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = write_tab(pl, w, s)) != AE_OK) return st;
  return subsample_impl(m, mel, pl, w, x, s);
}

ae_status ae_conformer_layer(const ae_model* m, int32_t layer, float* h, const int32_t* pos,
                             int64_t n, void* ws, size_t ws_bytes, ae_stream stream) {
  if (!m) return set_error(AE_ERR_INVALID, "model is NULL");
  if (layer < 0 || layer >= m->cfg.layers)
    return set_error(AE_ERR_INVALID, "layer index " + std::to_string(layer) + " out of range");
  if (n < 0) return set_error(AE_ERR_INVALID, "n must be >= 0");
  if (n == 0) return AE_OK;
  if (!h || !pos) return set_error(AE_ERR_INVALID, "h and pos must not be NULL");
  ae_status st;
  if ((st = check_sizes(m, n, 0)) != AE_OK) return st;
  Ws w = ws_layout(m, 1, 0, n, (char*)ws);
  if ((st = check_ws(ws, ws_bytes, w.total)) != AE_OK) return st;
  return layer_impl(m, layer, h, pos, n, w, (hipStream_t)stream, false, nullptr, nullptr);
}

ae_status ae_encode(const ae_model* m, const float* wave, const int64_t* sample_off, int32_t B,
                    float* out, float* const* trace, void* ws, size_t ws_bytes, ae_stream stream) {
  if (!m) return set_error(AE_ERR_INVALID, "model is NULL");
  Plan pl;
  ae_status st = plan_from_samples(sample_off, B, pl);
  if (st != AE_OK) return st;
  const int64_t T = pl.tokens();
  if (T == 0) return AE_OK;
  if (!wave || !out) return set_error(AE_ERR_INVALID, "wave and out must not be NULL");
  if ((st = check_sizes(m, T, pl.frames())) != AE_OK) return st;
  Ws w = ws_layout(m, B, pl.frames(), T, (char*)ws);
  if ((st = check_ws(ws, ws_bytes, w.total)) != AE_OK) return st;
  return encode_impl(m, wave, pl, out, trace, w, (hipStream_t)stream);
}

ae_status ae_encode_static(const ae_model* m, const float* wave, const int64_t* sample_off,
                           int32_t B, float* out, ae_stream stream) {
  if (!m) return set_error(AE_ERR_INVALID, "model is NULL");
  Plan pl;
  ae_status st = plan_from_samples(sample_off, B, pl);
  if (st != AE_OK) return st;
  const int64_t T = pl.tokens();
  if (T == 0) return AE_OK;
  if (!wave || !out) return set_error(AE_ERR_INVALID, "wave and out must not be NULL");
  if ((st = check_sizes(m, T, pl.frames())) != AE_OK) return st;
  const size_t need = ws_layout(m, B, pl.frames(), T, nullptr).total;
  if (need > kStaticScratchBytes)
    return set_error(AE_ERR_CAPACITY,
                     "batch needs " + std::to_string(need) + " bytes of scratch; the static "
                     "scratch holds " + std::to_string(kStaticScratchBytes) +
                     " (use ae_encode with a workspace)");
  int dev = -1;
  AE_HIP_TRY(hipGetDevice(&dev));
  if (dev != m->device)
    return set_error(AE_ERR_INVALID, "the current device (" + std::to_string(dev) +
                                         ") is not the model's (" + std::to_string(m->device) + ")");
  char* base = nullptr;
  if ((st = static_scratch(dev, &base)) != AE_OK) return st;
  Ws w = ws_layout(m, B, pl.frames(), T, base);
  return encode_impl(m, wave, pl, out, nullptr, w, (hipStream_t)stream);
}

}  // extern "C"

namespace {

ae_status encode_impl(const ae_model* m, const float* wave, const Plan& pl, float* out,
                      float* const* trace, const Ws& w, hipStream_t s) {
  ae_status st;
  const int B = pl.B;
  const int64_t T = pl.tokens();
  AE_HIP_TRY(mel_tables_init());
  if ((st = write_tab(pl, w, s)) != AE_OK) return st;
  AE_LAUNCH(AE_K_LOGMEL, s, launch_logmel(wave, w.tab, w.tab + (B + 1), B, pl.frames(), w.mel, s));
  if ((st = subsample_impl(m, w.mel, pl, w, w.h, s)) != AE_OK) return st;
  const int d = m->cfg.hidden;
  const size_t hbytes = sizeof(float) * (size_t)T * d;
  if (trace && trace[0]) AE_HIP_TRY(hipMemcpyAsync(trace[0], w.h, hbytes, hipMemcpyDeviceToDevice, s));
  const int L = m->cfg.layers;
  for (int l = 0; l < L; ++l) {
    const ae_layer_weights* next = (l + 1 < L) ? &m->layers[l + 1] : nullptr;
    // in bf16 the head's GEMM reads a bf16 copy of the final residual stream
    void* hc = (l + 1 == L && m->dt == AE_BF16) ? w.a[0] : nullptr;
    if ((st = layer_impl(m, l, w.h, w.tok_pos, T, w, s, l > 0, next, hc)) != AE_OK) return st;
    if (trace && trace[1 + l])
      AE_HIP_TRY(hipMemcpyAsync(trace[1 + l], w.h, hbytes, hipMemcpyDeviceToDevice, s));
  }
  // head: output_proj + bias, weightless RMS norm, embed_audio
  const int oh = m->cfg.out_hidden, od = m->cfg.out_dim;
  {
    const void* hin = m->dt == AE_BF16 ? w.a[0] : (const void*)w.h;
    GemmParams p = gemm_params(w, (int)T, oh, d, hin, d, m->w.out_proj, d, w.o1, oh);
    p.bias = m->w.out_bias;
    AE_LAUNCH(AE_K_GEMM_HEAD, s, launch_gemm(m->dt, EPI_BIAS, A_PLAIN, false, p, s));
  }
  if (trace && trace[L + 1])
    AE_HIP_TRY(hipMemcpyAsync(trace[L + 1], w.o1, sizeof(float) * (size_t)T * oh,
                              hipMemcpyDeviceToDevice, s));
  {
    RowNormParams r = rn_params(T, oh, w.o1);
    r.plain_next = true; r.n_out = 1; r.a[0] = w.on;
    AE_LAUNCH(AE_K_ROWNORM, s, launch_rownorm(m->dt, r, s));
  }
  {
    GemmParams p = gemm_params(w, (int)T, od, oh, w.on, oh, m->w.embed, oh, out, od);
    AE_LAUNCH(AE_K_GEMM_HEAD, s, launch_gemm(m->dt, EPI_STORE, A_PLAIN, false, p, s));
  }
  return AE_OK;
}

}  // namespace
