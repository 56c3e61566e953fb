// LFM2A front end (cera 0.5.3, audio_encoder_gpu.rs: log_mel_spectrogram_gpu
// and the stft_frames, power_spec, mel_project and mel_norm ops): framing
// with center padding, pre-emphasis and the zero-flanked Hann window,
// |DFT|^2 on 257 bins, 128 Slaney mel bands, ln(band + 2^-24), then a
// per-band normalisation over each clip's statistics frames.
//
// The page evaluates the DFT as a direct sum per bin (a GPU without an
// FFT); here the 512-point real transform is one 256-point complex FFT of
// z[n] = y[2n] + i y[2n+1] per frame, sixteen lanes per frame, split as
// 16 x 16 with the second pass after a wavefront-local LDS transpose and
// the real spectrum recovered from Z[k] and Z[256 - k]. The pre-emphasised
// sample y[s] = x[s] - 0.97 x[s - 1] (y[0] = x[0]) is formed in the gather.
// The statistics are accumulated in float64: a shifted sum and sum of
// squares per (clip, band, slice of frames), then one pass combining the
// slices.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "fft16.h"
#include "lfm2a_launch.h"

namespace ae {
namespace lfm {
namespace {

constexpr int kMaxBandW = 1024;
constexpr int kGroups = kMel / 16;  // band groups: bands 16 i .. 16 i + 15
constexpr int FPB = 16;        // frames per block (4 per wavefront)
constexpr int TLD = 17;        // transpose row stride (float2)
constexpr int MAXB_LDS = 512;  // clips whose offsets are staged in LDS

struct Tables {
  float win[kNFft];          // periodic Hann of 400 points centred in 512
  float2 tw256[256];         // exp(-2 pi i m / 256)
  float2 tw512[256];         // exp(-2 pi i m / 512), m < 256
  int band_start[kMel];      // first bin a band reads (its padded list stays below bin 257)
  int group_len[kGroups];    // bins read per band of the group (its widest band's count)
  int group_woff[kGroups];   // group's weights: [q][16 bands] from here
  float band_w[kMaxBandW];   // a quarter of the filter weights, zero padded
};

__constant__ Tables g_tab;

double hz_to_mel(double f) {
  return f < 1000.0 ? f * 3.0 / 200.0 : 15.0 + log(f / 1000.0) * 27.0 / log(6.4);
}
double mel_to_hz(double m) {
  return m < 15.0 ? m * 200.0 / 3.0 : 1000.0 * exp((m - 15.0) * log(6.4) / 27.0);
}

bool build_tables(Tables* t) {
  for (int n = 0; n < kNFft; ++n) t->win[n] = 0.f;
  const int left = (kNFft - kWin) / 2;
  for (int n = 0; n < kWin; ++n)
    t->win[left + n] = (float)(0.5 - 0.5 * cos(2.0 * M_PI * n / kWin));
  for (int m = 0; m < 256; ++m) {
    const double a = -2.0 * M_PI * m / 256.0, b = -2.0 * M_PI * m / 512.0;
    t->tw256[m] = make_float2((float)cos(a), (float)sin(a));
    t->tw512[m] = make_float2((float)cos(b), (float)sin(b));
  }
  // Slaney bands: 130 edges evenly spaced in mel over 0..8 kHz, triangles
  // on the bin frequencies k * 16000 / 512, each scaled to unit area
  const double top = hz_to_mel(8000.0);
  std::vector<double> edge(kMel + 2);
  for (int i = 0; i < kMel + 2; ++i) edge[i] = mel_to_hz(top * i / (kMel + 1));
  std::vector<int> start(kMel, 0), count(kMel, 0);
  std::vector<std::vector<double>> wts(kMel);
  for (int m = 0; m < kMel; ++m) {
    const double lo = edge[m], c = edge[m + 1], hi = edge[m + 2];
    int st = -1;
    for (int k = 0; k < kBins; ++k) {
      const double f = k * 16000.0 / kNFft;
      const double w = fmax(0.0, fmin((f - lo) / (c - lo), (hi - f) / (hi - c))) * 2.0 / (hi - lo);
      if (w > 0.0) {
        if (st < 0) st = k;
        if (k != st + (int)wts[m].size()) return false;  // support must be contiguous
        wts[m].push_back(w);
      }
    }
    start[m] = st < 0 ? 0 : st;
    count[m] = (int)wts[m].size();
  }
  // groups of sixteen bands read a common number of bins; a band whose
  // padded list would run past the last bin starts earlier, its weights
  // shifted to the end of the list. The kernel sums four times the power
  // (twice the spectrum, the split's halves left out), so the weights are
  // quartered here (exact).
  int woff = 0;
  for (int i = 0; i < kGroups; ++i) {
    int q_len = 0;
    for (int j = 0; j < 16; ++j) q_len = std::max(q_len, count[16 * i + j]);
    if (woff + 16 * q_len > kMaxBandW) return false;
    t->group_len[i] = q_len;
    t->group_woff[i] = woff;
    for (int j = 0; j < 16; ++j) {
      const int b = 16 * i + j;
      const int s0 = std::min(start[b], kBins - q_len);
      const int shift = start[b] - s0;
      t->band_start[b] = s0;
      for (int q = 0; q < q_len; ++q) {
        const int e = q - shift;
        t->band_w[woff + 16 * q + j] =
            (e >= 0 && e < count[b]) ? (float)(0.25 * wts[b][e]) : 0.0f;
      }
    }
    woff += 16 * q_len;
  }
  return true;
}

__device__ __forceinline__ int find_clip_lds(const int64_t* off, int B, int64_t r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(256) k_lfm_logmel(const float* __restrict__ wave,
                                                    const int64_t* __restrict__ sample_off,
                                                    const int64_t* __restrict__ frame_off, int B,
                                                    int64_t total, float* __restrict__ mel) {
  __shared__ float2 tw256[256];
  __shared__ float2 tw512[256];
  __shared__ float win[kNFft];
  __shared__ int bstart[kMel];
  __shared__ float bw[kMaxBandW];
  __shared__ int64_t soff[MAXB_LDS + 1], foff[MAXB_LDS + 1];
  __shared__ __attribute__((aligned(16))) float2 xbuf[FPB][16 * TLD];
  for (int i = threadIdx.x; i < 256; i += 256) {
    tw256[i] = g_tab.tw256[i];
    tw512[i] = g_tab.tw512[i];
  }
  for (int i = threadIdx.x; i < kNFft; i += 256) win[i] = g_tab.win[i];
  for (int i = threadIdx.x; i < kMel; i += 256) bstart[i] = g_tab.band_start[i];
  for (int i = threadIdx.x; i < kMaxBandW; i += 256) bw[i] = g_tab.band_w[i];
  const bool lds_off = B <= MAXB_LDS;
  if (lds_off)
    for (int i = threadIdx.x; i <= B; i += 256) {
      soff[i] = sample_off[i];
      foff[i] = frame_off[i];
    }
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int fl = wv * 4 + (lane >> 4);  // frame slot in the block
  const int j = lane & 15;
  float2* T = xbuf[fl];
  float* M = (float*)xbuf[fl];
  // windowed pre-emphasised samples of the frame the block handles next
  // (register double buffer): lane j holds samples n = 2 (16 m + j) + e.
  // Each sample is loaded once: y[s] = x[s] - 0.97 x[s - 1] takes x[s - 1]
  // of an odd n from the same lane and of an even n from lane j - 1 of the
  // frame's 16 (a DPP rotation within the row; lane 0 takes lane 15's
  // previous m, and for n = 0 loads the sample before the frame itself).
  float yw[32];
  // this lane's window weights (samples 2 (16 m + j) + e), for every frame
  float wj[32];
#pragma unroll
  for (int m = 0; m < 16; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) wj[2 * m + e] = win[2 * (16 * m + j) + e];
  auto fetch = [&](int64_t g0) {
    const int64_t g = g0 + fl;
    const bool active = g < total;
    int64_t start = 0, len = 0, base = 0;
    if (active) {
      const int c = lds_off ? find_clip_lds(foff, B, g) : find_clip(frame_off, B, g);
      start = lds_off ? soff[c] : sample_off[c];
      len = (lds_off ? soff[c + 1] : sample_off[c + 1]) - start;
      base = (g - (lds_off ? foff[c] : frame_off[c])) * kHop - kCenterPad;
    }
    // A frame whose 512 samples and the one before them lie inside the clip
    // (all but the first two and last two of a clip) reads through one
    // pointer with immediate offsets and needs no checks. The window is zero
    // on samples 0..55 and 456..511, so groups m = 0 and 15 are not read;
    // the one predecessor that would come from them (lane 0, m = 1) meets
    // a zero window as well.
    if (active && base >= 1 && base + kNFft <= len) {
      const float* p = wave + start + base + 2 * j;
      float x0[16], x1[16];
      x0[0] = x1[0] = x0[15] = x1[15] = 0.f;
#pragma unroll
      for (int m = 1; m < 15; ++m) {
        x0[m] = p[32 * m];
        x1[m] = p[32 * m + 1];
      }
      float rot_prev = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float rot = dpp_mov<0x121>(x1[m]);  // row_ror:1, lane j <- lane j - 1
        const float prev0 = j == 0 ? rot_prev : rot;
        rot_prev = rot;
        yw[2 * m] = (x0[m] - kPreemph * prev0) * wj[2 * m];
        yw[2 * m + 1] = (x1[m] - kPreemph * x0[m]) * wj[2 * m + 1];
      }
      return;
    }
    auto in_clip = [&](int64_t s) { return active && s >= 0 && s < len; };
    float x0[16], x1[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int64_t s0 = base + 2 * (16 * m + j);
      x0[m] = in_clip(s0) ? wave[start + s0] : 0.f;
      x1[m] = in_clip(s0 + 1) ? wave[start + s0 + 1] : 0.f;
    }
    const float before = (j == 0 && in_clip(base - 1)) ? wave[start + base - 1] : 0.f;
    float rot_prev = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float rot = dpp_mov<0x121>(x1[m]);  // row_ror:1, lane j <- lane j - 1
      const float prev0 = j == 0 ? (m == 0 ? before : rot_prev) : rot;
      rot_prev = rot;
      const int n0 = 2 * (16 * m + j);
      const int64_t s0 = base + n0;
      const float y0 = in_clip(s0) ? (s0 > 0 ? x0[m] - kPreemph * prev0 : x0[m]) : 0.f;
      const float y1 = in_clip(s0 + 1) ? (s0 + 1 > 0 ? x1[m] - kPreemph * x0[m] : x1[m]) : 0.f;
      yw[2 * m] = y0 * wj[2 * m];
      yw[2 * m + 1] = y1 * wj[2 * m + 1];
    }
  };
  int64_t g0 = (int64_t)blockIdx.x * FPB;
  if (g0 < total) fetch(g0);
  for (; g0 < total; g0 += (int64_t)gridDim.x * FPB) {
    const int64_t g = g0 + fl;
    const bool active = g < total;
    // pass 1: lane j = n2, DFT over m of z[16 m + j]
    float2 x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) x[m] = make_float2(yw[2 * m], yw[2 * m + 1]);
    const int64_t g1 = g0 + (int64_t)gridDim.x * FPB;
    if (g1 < total) fetch(g1);
    dft16(x);
#pragma unroll
    for (int k1 = 0; k1 < 16; ++k1) {
      const float2 t = k1 == 0 ? x[0] : cmul(x[k1], tw256[(j * k1) & 255]);
      T[k1 * TLD + j] = t;
    }
    wave_sync();
    // pass 2: lane j = k1, DFT over n2
#pragma unroll
    for (int n2 = 0; n2 < 16; ++n2) x[n2] = T[j * TLD + n2];
    dft16(x);  // x[k2] = Z[j + 16 k2]
    wave_sync();
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) T[j + 16 * k2] = x[k2];
    wave_sync();
    // real split: four times the powers of bins j + 16 k2 (and 256 on lane 0)
    float pw[16];
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) {
      const int k = j + 16 * k2;
      const float2 zk = x[k2], zn = T[(256 - k) & 255];
      const float ex = zk.x + zn.x, ey = zk.y - zn.y;  // 2 E[k]
      const float ox = zk.y + zn.y, oy = zn.x - zk.x;  // 2 O[k]
      const float2 w = tw512[k];
      const float xx = fmaf(w.x, ox, fmaf(-w.y, oy, ex));
      const float xy = fmaf(w.x, oy, fmaf(w.y, ox, ey));
      pw[k2] = fmaf(xx, xx, xy * xy);
    }
    const float nyq = 2.0f * (x[0].x - x[0].y);
    const float p256 = nyq * nyq;
    wave_sync();
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) M[j + 16 * k2] = pw[k2];
    if (j == 0) M[256] = p256;
    wave_sync();
    // mel bands j, j + 16, ..., then the log
    // (uniform trip counts per group of sixteen bands; v_log_f32 is log2)
    float out[8];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const float* mp = M + bstart[j + 16 * i];
      const float* wp = bw + g_tab.group_woff[i] + j;
      const int q_len = g_tab.group_len[i];
      float acc = 0.f;
      for (int q = 0; q < q_len; ++q) acc = fmaf(mp[q], wp[16 * q], acc);
      out[i] = __builtin_amdgcn_logf(acc + kLogEps) * 0.69314718055994530942f;
    }
    wave_sync();
    float* O = M + 260;
#pragma unroll
    for (int i = 0; i < 8; ++i) O[j + 16 * i] = out[i];
    wave_sync();
    if (active) {
      const float4 a = *(const float4*)(O + 8 * j), c = *(const float4*)(O + 8 * j + 4);
      float* dst = mel + g * kMel + 8 * j;
      *(float4*)dst = a;
      *(float4*)(dst + 4) = c;
    }
    wave_sync();
  }
}

// One block per (clip, slice of its statistics frames): thread (band,
// half) sums x - K and (x - K)^2 in float64 over every other frame of the
// slice, K the band's value in the clip's first frame.
__global__ void __launch_bounds__(256) k_lfm_mel_stats(const float* __restrict__ mel,
                                                       const int64_t* __restrict__ sample_off,
                                                       const int64_t* __restrict__ frame_off,
                                                       double* __restrict__ part) {
  __shared__ double sh[kMel][2];
  const int c = blockIdx.x, sl = blockIdx.y;
  const int64_t f0 = frame_off[c];
  const int64_t neff = (sample_off[c + 1] - sample_off[c]) / kHop;
  const int band = threadIdx.x & (kMel - 1), half = threadIdx.x >> 7;
  const int64_t lo = neff * sl / kStatSlices, hi = neff * (sl + 1) / kStatSlices;
  double s1 = 0.0, s2 = 0.0;
  if (neff > 0) {
    const double K = mel[f0 * kMel + band];
    for (int64_t f = lo + half; f < hi; f += 2) {
      const double v = (double)mel[(f0 + f) * kMel + band] - K;
      s1 += v;
      s2 += v * v;
    }
  }
  if (half) {
    sh[band][0] = s1;
    sh[band][1] = s2;
  }
  __syncthreads();
  if (!half) {
    double* dst = part + (((int64_t)c * kStatSlices + sl) * kMel + band) * 2;
    dst[0] = s1 + sh[band][0];
    dst[1] = s2 + sh[band][1];
  }
}

__global__ void __launch_bounds__(kMel) k_lfm_mel_final(const float* __restrict__ mel,
                                                        const int64_t* __restrict__ sample_off,
                                                        const int64_t* __restrict__ frame_off,
                                                        const double* __restrict__ part,
                                                        float* __restrict__ stats) {
  const int c = blockIdx.x, band = threadIdx.x;
  const int64_t neff = (sample_off[c + 1] - sample_off[c]) / kHop;
  float* dst = stats + ((int64_t)c * kMel + band) * 2;
  if (neff < 2) {  // no statistics frames worth the name: the host refuses such clips
    dst[0] = 0.f;
    dst[1] = 0.f;
    return;
  }
  double s1 = 0.0, s2 = 0.0;
  for (int sl = 0; sl < kStatSlices; ++sl) {
    const double* p = part + (((int64_t)c * kStatSlices + sl) * kMel + band) * 2;
    s1 += p[0];
    s2 += p[1];
  }
  const double n = (double)neff;
  const double K = mel[frame_off[c] * kMel + band];
  const double var = fmax((s2 - s1 * s1 / n) / (n - 1.0), 0.0);
  dst[0] = (float)(K + s1 / n);
  dst[1] = (float)(1.0 / (sqrt(var) + (double)kNormEps));
}

// Eight rows per block, a float4 per thread.
__global__ void __launch_bounds__(256) k_lfm_mel_norm(float* __restrict__ mel,
                                                      const int64_t* __restrict__ sample_off,
                                                      const int64_t* __restrict__ frame_off,
                                                      int B, int64_t total,
                                                      const float* __restrict__ stats) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= total) return;
  const int q = (threadIdx.x & 31) * 4;
  const int c = find_clip(frame_off, B, row);
  const int64_t local = row - frame_off[c];
  const int64_t neff = (sample_off[c + 1] - sample_off[c]) / kHop;
  float4* p = (float4*)(mel + row * kMel + q);
  if (local >= neff) {
    *p = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float* st = stats + ((int64_t)c * kMel + q) * 2;
  float4 v = *p;
  v.x = (v.x - st[0]) * st[1];
  v.y = (v.y - st[2]) * st[3];
  v.z = (v.z - st[4]) * st[5];
  v.w = (v.w - st[6]) * st[7];
  *p = v;
}

std::mutex g_init_mu;
bool g_init_done[64];

}  // namespace

hipError_t frontend_init() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_init_mu);
  if (g_init_done[dev]) return hipSuccess;
  static Tables host;
  static bool built = false;
  if (!built) {
    if (!build_tables(&host)) return hipErrorInvalidValue;
    built = true;
  }
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_tab), &host, sizeof(Tables), 0, hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  g_init_done[dev] = true;
  return hipSuccess;
}

hipError_t launch_logmel_raw(const float* wave, const int64_t* sample_off,
                             const int64_t* frame_off, int B, int64_t total_frames, float* mel,
                             hipStream_t s) {
  if (total_frames <= 0) return hipSuccess;
  const int64_t blocks = (total_frames + FPB - 1) / FPB;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(k_lfm_logmel, dim3(grid), dim3(256), 0, s, wave, sample_off, frame_off, B,
                     total_frames, mel);
  return hipGetLastError();
}

hipError_t launch_mel_stats(const float* mel, const int64_t* sample_off,
                            const int64_t* frame_off, int B, double* part, float* stats,
                            hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lfm_mel_stats, dim3(B, kStatSlices), dim3(256), 0, s, mel, sample_off,
                     frame_off, part);
  hipLaunchKernelGGL(k_lfm_mel_final, dim3(B), dim3(kMel), 0, s, mel, sample_off, frame_off, part,
                     stats);
  return hipGetLastError();
}

hipError_t launch_mel_norm(float* mel, const int64_t* sample_off, const int64_t* frame_off, int B,
                           int64_t total_frames, const float* stats, hipStream_t s) {
  if (total_frames <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lfm_mel_norm, dim3((unsigned)((total_frames + 7) / 8)), dim3(256), 0, s,
                     mel, sample_off, frame_off, B, total_frames, stats);
  return hipGetLastError();
}

}  // namespace lfm
}  // namespace ae
