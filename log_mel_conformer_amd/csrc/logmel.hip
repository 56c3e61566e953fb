// Log-mel front end: framing, periodic Hann window, 512-point real FFT
// magnitude, 128 HTK mel bands, natural log (egemma2_audio.rs, module
// documentation step 2, mel_filter_bank and MelFrontend::log_mel).
//
// One wavefront per frame. The 512-point real FFT is a 256-point complex
// FFT of z[n] = x[2n] + i x[2n+1]: four radix-4 Stockham stages, one
// butterfly per lane per stage (256 = 4 x 64), ping-ponging through LDS,
// then the even/odd split X[k] = E[k] + e^{-2 pi i k/512} O[k]. The first
// stage reads its four inputs straight from the waveform (the window is
// applied on the way), so a frame costs one pass over 320 samples; frames
// of one block overlap by half and share the cache lines. The mel bank
// has at most two nonzero weights per bin (506 in all), so each band is a
// short contiguous dot product over its own bins, not a dense 257x128
// product. Tables (window, twiddles, bands) are computed on the host in
// double and rounded to float once.
#include <math.h>

#include <mutex>
#include <vector>

#include "launch.h"

namespace ae {
namespace {

constexpr int kMaxBandW = 640;

struct MelTables {
  float hann[kFrame];
  float2 tw[kFft];          // exp(-2 pi i m / 512)
  int band_start[kMels];
  int band_count[kMels];
  int band_woff[kMels];
  float band_w[kMaxBandW];
};

__constant__ MelTables g_mel;

// numpy-style linspace with the last point set exactly.
std::vector<double> linspace_d(double a, double b, int n) {
  std::vector<double> v(n);
  const double step = (b - a) / (n - 1);
  for (int i = 0; i < n; ++i) v[i] = a + i * step;
  v[n - 1] = b;
  return v;
}

bool build_tables(MelTables* t) {
  for (int n = 0; n < kFrame; ++n)
    t->hann[n] = (float)(0.5 - 0.5 * cos(2.0 * M_PI * n / kFrame));
  for (int m = 0; m < kFft; ++m) {
    const double a = -2.0 * M_PI * m / kFft;
    t->tw[m] = make_float2((float)cos(a), (float)sin(a));
  }
  // HTK mel scale, 130 edges over 0..8 kHz, triangles on 257 bins, no norm.
  auto hz2mel = [](double f) { return 2595.0 * log10(1.0 + f / 700.0); };
  auto mel2hz = [](double m) { return 700.0 * (pow(10.0, m / 2595.0) - 1.0); };
  std::vector<double> mels = linspace_d(hz2mel(0.0), hz2mel(kSampleRate / 2), kMels + 2);
  std::vector<double> ff(kMels + 2);
  for (int i = 0; i < kMels + 2; ++i) ff[i] = mel2hz(mels[i]);
  std::vector<double> fk = linspace_d(0.0, kSampleRate / 2, kBins);
  int woff = 0;
  for (int m = 0; m < kMels; ++m) {
    int start = -1, count = 0;
    for (int k = 0; k < kBins; ++k) {
      const double down = -(ff[m] - fk[k]) / (ff[m + 1] - ff[m]);
      const double up = (ff[m + 2] - fk[k]) / (ff[m + 2] - ff[m + 1]);
      const double w = fmax(0.0, fmin(down, up));
      if (w > 0.0) {
        if (start < 0) start = k;
        if (k != start + count) return false;  // support must be contiguous
        if (woff + count >= kMaxBandW) return false;
        t->band_w[woff + count] = (float)w;
        ++count;
      }
    }
    t->band_start[m] = start < 0 ? 0 : start;
    t->band_count[m] = count;
    t->band_woff[m] = woff;
    woff += count;
  }
  return true;
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// 4 frames per 256-thread block, one per wavefront; grid-stride over frames.
__global__ void __launch_bounds__(256) k_logmel(const float* __restrict__ wave,
                                                const int64_t* __restrict__ sample_off,
                                                const int64_t* __restrict__ frame_off, int B,
                                                int64_t total, float* __restrict__ mel) {
  __shared__ float2 buf[4][2][256];
  __shared__ float mag[4][260];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int64_t g0 = (int64_t)blockIdx.x * 4; g0 < total; g0 += (int64_t)gridDim.x * 4) {
    const int64_t g = g0 + w;
    const bool active = g < total;
    int64_t base = 0, start = 0;
    if (active) {
      const int c = find_clip(frame_off, B, g);
      start = sample_off[c];
      base = start + (g - frame_off[c]) * kHop - kHop;  // frame starts 160 samples early
    }
    // stage 0 inputs: z[lane + 64 r] = x[2n] + i x[2n+1], n < 160 nonzero
    float2 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = lane + 64 * r;
      float x0 = 0.f, x1 = 0.f;
      if (active && n < kFrame / 2) {
        const int64_t s0 = base + 2 * n;
        if (s0 >= start) x0 = wave[s0] * g_mel.hann[2 * n];
        if (s0 + 1 >= start) x1 = wave[s0 + 1] * g_mel.hann[2 * n + 1];
      }
      v[r] = make_float2(x0, x1);
    }
    // four radix-4 Stockham stages (autosort: natural order out)
    int dst = 0;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int Ns = 1 << (2 * st);
      if (st > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = buf[w][dst ^ 1][lane + 64 * r];
      }
      const int k = lane & (Ns - 1);
      const int step = 128 >> (2 * st);  // 512 / (4 Ns)
#pragma unroll
      for (int r = 1; r < 4; ++r) v[r] = cmul(v[r], g_mel.tw[(r * k * step) & 511]);
      const float2 s02 = make_float2(v[0].x + v[2].x, v[0].y + v[2].y);
      const float2 d02 = make_float2(v[0].x - v[2].x, v[0].y - v[2].y);
      const float2 s13 = make_float2(v[1].x + v[3].x, v[1].y + v[3].y);
      const float2 d13 = make_float2(v[1].x - v[3].x, v[1].y - v[3].y);
      // y1 = d02 - i d13, y3 = d02 + i d13
      const float2 y0 = make_float2(s02.x + s13.x, s02.y + s13.y);
      const float2 y1 = make_float2(d02.x + d13.y, d02.y - d13.x);
      const float2 y2 = make_float2(s02.x - s13.x, s02.y - s13.y);
      const float2 y3 = make_float2(d02.x - d13.y, d02.y + d13.x);
      const int idx = (lane / Ns) * Ns * 4 + k;
      buf[w][dst][idx] = y0;
      buf[w][dst][idx + Ns] = y1;
      buf[w][dst][idx + 2 * Ns] = y2;
      buf[w][dst][idx + 3 * Ns] = y3;
      __syncthreads();
      dst ^= 1;
    }
    const float2* Z = buf[w][dst ^ 1];
    // real split: X[k] = E[k] + e^{-2 pi i k / 512} O[k]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = lane + 64 * r;
      const float2 zk = Z[k], zn = Z[(256 - k) & 255];
      const float2 E = make_float2(0.5f * (zk.x + zn.x), 0.5f * (zk.y - zn.y));
      const float2 O = make_float2(0.5f * (zk.y + zn.y), -0.5f * (zk.x - zn.x));
      const float2 X = cmul(g_mel.tw[k], O);
      const float re = E.x + X.x, im = E.y + X.y;
      mag[w][k] = sqrtf(re * re + im * im);
    }
    if (lane == 0) mag[w][256] = fabsf(Z[0].x - Z[0].y);
    __syncthreads();
    // mel bands and log
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = lane + 64 * r;
      const int s = g_mel.band_start[b], cnt = g_mel.band_count[b], wo = g_mel.band_woff[b];
      float acc = 0.f;
      for (int q = 0; q < cnt; ++q) acc += mag[w][s + q] * g_mel.band_w[wo + q];
      if (active) mel[g * kMels + b] = logf(acc + kMelFloor);
    }
    __syncthreads();
  }
}

std::mutex g_init_mu;
bool g_init_done[64];

}  // namespace

hipError_t mel_tables_init() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_init_mu);
  if (g_init_done[dev]) return hipSuccess;
  static MelTables host;
  static bool built = false;
  if (!built) {
    if (!build_tables(&host)) return hipErrorInvalidValue;
    built = true;
  }
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_mel), &host, sizeof(MelTables), 0, hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  g_init_done[dev] = true;
  return hipSuccess;
}

hipError_t launch_logmel(const float* wave, const int64_t* sample_off, const int64_t* frame_off,
                         int B, int64_t total_frames, float* mel, hipStream_t s) {
  if (total_frames <= 0) return hipSuccess;
  const int64_t blocks = (total_frames + 3) / 4;
  const int grid = (int)(blocks < (1 << 20) ? blocks : (1 << 20));
  hipLaunchKernelGGL(k_logmel, dim3(grid), dim3(256), 0, s, wave, sample_off, frame_off, B,
                     total_frames, mel);
  return hipGetLastError();
}

}  // namespace ae
