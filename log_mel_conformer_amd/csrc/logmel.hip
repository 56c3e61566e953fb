// Log-mel front end: framing, periodic Hann window, 512-point real FFT
// magnitude, 128 HTK mel bands, natural log (egemma2_audio.rs, module
// documentation step 2, mel_filter_bank and MelFrontend::log_mel).
//
// Sixteen lanes per frame, four frames per wavefront. The 512-point real
// FFT is a 256-point complex FFT of z[n] = x[2n] + i x[2n+1] (the last 96
// z are zero: the frame is 320 samples), split as 256 = 16 x 16: lane j
// first takes the 16-point DFT over z[16 m + j] in registers (ten nonzero
// inputs), multiplies by e^{-2 pi i j k / 256}, and the wavefront
// transposes through LDS; lane j then takes the 16-point DFT over the other
// index and holds Z[j + 16 k]. The real spectrum follows from
// 2 X[k] = (Z[k] + conj Z[256-k]) - i e^{-2 pi i k / 512} (Z[k] - conj Z[256-k])
// (the partner read from LDS); the factor 2 is taken out of the mel
// weights, which are halved on the host (exact). The mel bank has at most
// two nonzero weights per bin (506 in all), so each band is a short
// contiguous dot product over its own bins; lane j takes bands j, j + 16,
// ..., so the i-th band of every lane comes from the same group of sixteen,
// and each group reads a fixed number of bins (its widest band's count,
// the others' weight lists padded with zeros): the loop counts are uniform
// across the wavefront. All exchanges stay inside a wavefront.
//
// Instruction economy (the kernel is VALU-bound): a frame's samples are
// read through one pointer with immediate offsets (only a clip's first
// frame, which starts before the clip, takes a checked path), the lane's
// window weights stay in registers, and the square root and logarithm are
// the hardware ones (v_sqrt_f32, v_log_f32: about one ulp, far inside the
// front end's 1e-4 tolerance). Window, twiddle and band tables are
// computed on the host in double, rounded to float once, and staged in LDS.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "fft16.h"
#include "launch.h"

namespace ae {
namespace {

constexpr int kMaxBandW = 1024;
constexpr int kGroups = kMels / 16;  // band groups: bands 16 i .. 16 i + 15
constexpr int FPB = 16;        // frames per block (4 per wavefront)

struct MelTables {
  float hann[kFrame];
  float2 tw256[256];        // exp(-2 pi i m / 256)
  float2 tw512[256];        // exp(-2 pi i m / 512), m < 256
  int band_start[kMels];    // first bin a band reads (its padded list stays below bin 257)
  int group_len[kGroups];   // bins read per band of the group (its widest band's count)
  int group_woff[kGroups];  // group's weights: [q][16 bands] from here
  float band_w[kMaxBandW];  // half the filter weights, zero padded
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
  for (int m = 0; m < 256; ++m) {
    const double a = -2.0 * M_PI * m / 256.0, b = -2.0 * M_PI * m / 512.0;
    t->tw256[m] = make_float2((float)cos(a), (float)sin(a));
    t->tw512[m] = make_float2((float)cos(b), (float)sin(b));
  }
  // HTK mel scale, 130 edges over 0..8 kHz, triangles on 257 bins, no norm.
  auto hz2mel = [](double f) { return 2595.0 * log10(1.0 + f / 700.0); };
  auto mel2hz = [](double m) { return 700.0 * (pow(10.0, m / 2595.0) - 1.0); };
  std::vector<double> mels = linspace_d(hz2mel(0.0), hz2mel(kSampleRate / 2), kMels + 2);
  std::vector<double> ff(kMels + 2);
  for (int i = 0; i < kMels + 2; ++i) ff[i] = mel2hz(mels[i]);
  std::vector<double> fk = linspace_d(0.0, kSampleRate / 2, kBins);
  // each band's contiguous support and weights
  std::vector<int> start(kMels, 0), count(kMels, 0);
  std::vector<std::vector<double>> wts(kMels);
  for (int m = 0; m < kMels; ++m) {
    int st = -1;
    for (int k = 0; k < kBins; ++k) {
      const double down = -(ff[m] - fk[k]) / (ff[m + 1] - ff[m]);
      const double up = (ff[m + 2] - fk[k]) / (ff[m + 2] - ff[m + 1]);
      const double w = fmax(0.0, fmin(down, up));
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
  // shifted to the end of the list
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
            (e >= 0 && e < count[b]) ? (float)(0.5 * wts[b][e]) : 0.0f;
      }
    }
    woff += 16 * q_len;
  }
  return true;
}

constexpr int TLD = 17;    // transpose row stride (float2)
constexpr int MAXB_LDS = 512;  // clips whose offsets are staged in LDS

// Largest c with off[c] <= r over off[0..B] held in LDS.
__device__ __forceinline__ int find_clip_lds(const int64_t* off, int B, int64_t r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// 16-point DFT (as dft16) of inputs of which only x[0..9] are nonzero: the
// first radix-4 stage skips the known zeros.
__device__ __forceinline__ void dft16_head10(float2 (&x)[16]) {
#pragma unroll
  for (int m2 = 0; m2 < 4; ++m2) {
    // inputs x[m2], x[4 + m2], x[8 + m2] (zero for m2 >= 2), x[12 + m2] = 0
    const float2 a0 = x[m2], a1 = x[4 + m2];
    const float2 d13 = mul_mi(a1);
    float2 s02 = a0, d02 = a0;
    if (m2 < 2) {
      s02 = cadd(a0, x[8 + m2]);
      d02 = csub(a0, x[8 + m2]);
    }
    x[m2] = cadd(s02, a1);
    x[4 + m2] = cadd(d02, d13);
    x[8 + m2] = csub(s02, a1);
    x[12 + m2] = csub(d02, d13);
  }
#pragma unroll
  for (int m2 = 1; m2 < 4; ++m2)
#pragma unroll
    for (int k1 = 1; k1 < 4; ++k1) x[4 * k1 + m2] = cmul(x[4 * k1 + m2], w16(m2 * k1));
  float2 y[16];
#pragma unroll
  for (int k1 = 0; k1 < 4; ++k1) {
    float2 a0 = x[4 * k1], a1 = x[4 * k1 + 1], a2 = x[4 * k1 + 2], a3 = x[4 * k1 + 3];
    dft4(a0, a1, a2, a3);
    y[k1] = a0;
    y[k1 + 4] = a1;
    y[k1 + 8] = a2;
    y[k1 + 12] = a3;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = y[i];
}

__global__ void __launch_bounds__(256) k_logmel(const float* __restrict__ wave,
                                                const int64_t* __restrict__ sample_off,
                                                const int64_t* __restrict__ frame_off, int B,
                                                int64_t total, float* __restrict__ mel) {
  __shared__ float2 tw256[256];
  __shared__ float2 tw512[256];
  __shared__ float hann[kFrame];
  __shared__ int bstart[kMels];
  __shared__ float bw[kMaxBandW];
  __shared__ int64_t soff[MAXB_LDS + 1], foff[MAXB_LDS + 1];
  // per frame: transpose buffer, then Z in natural order, then magnitudes,
  // then the 128 outputs
  __shared__ __attribute__((aligned(16))) float2 xbuf[FPB][16 * TLD];
  for (int i = threadIdx.x; i < 256; i += 256) {
    tw256[i] = g_mel.tw256[i];
    tw512[i] = g_mel.tw512[i];
  }
  for (int i = threadIdx.x; i < kFrame; i += 256) hann[i] = g_mel.hann[i];
  for (int i = threadIdx.x; i < kMels; i += 256) bstart[i] = g_mel.band_start[i];
  for (int i = threadIdx.x; i < kMaxBandW; i += 256) bw[i] = g_mel.band_w[i];
  const bool lds_off = B <= MAXB_LDS;
  if (lds_off)
    for (int i = threadIdx.x; i <= B; i += 256) {
      soff[i] = sample_off[i];
      foff[i] = frame_off[i];
    }
  __syncthreads();

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int fl = wv * 4 + (lane >> 4);   // frame slot in the block
  const int j = lane & 15;
  float2* T = xbuf[fl];
  float* M = (float*)xbuf[fl];            // magnitudes, after the split
  // this lane's samples of a frame are 32 m + 2 j + e (m < 10, e < 2): their
  // window weights, for every frame
  float wj[20];
#pragma unroll
  for (int m = 0; m < 10; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) wj[2 * m + e] = hann[32 * m + 2 * j + e];
  // Raw samples of the frame group a block handles next: loaded one group
  // ahead (register double buffer). A frame starts 160 samples early; only
  // a clip's first frame reaches before the clip, and it (and a slot past
  // the last frame) takes the checked path, where samples before the clip
  // are zeros.
  float xr[20];
  auto fetch = [&](int64_t g0) {
    const int64_t g = g0 + fl;
    int64_t base = 0;
    int lim = 1 << 30;  // samples below this index are zeros (all, past the end)
    if (g < total) {
      int c;
      int64_t start;
      if (lds_off) {
        c = find_clip_lds(foff, B, g);
        start = soff[c];
        base = start + (g - foff[c]) * kHop - kHop;
      } else {
        c = find_clip(frame_off, B, g);
        start = sample_off[c];
        base = start + (g - frame_off[c]) * kHop - kHop;
      }
      lim = start > base ? (int)(start - base) : 0;
    }
    if (lim == 0) {
      const float* p = wave + base + 2 * j;
#pragma unroll
      for (int m = 0; m < 10; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e) xr[2 * m + e] = p[32 * m + e];
    } else {
#pragma unroll
      for (int m = 0; m < 10; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int idx = 32 * m + 2 * j + e;
          xr[2 * m + e] = idx >= lim ? wave[base + idx] : 0.f;
        }
    }
  };
  int64_t g0 = (int64_t)blockIdx.x * FPB;
  if (g0 < total) fetch(g0);
  for (; g0 < total; g0 += (int64_t)gridDim.x * FPB) {
    const int64_t g = g0 + fl;
    const bool active = g < total;
    // pass 1: lane j = n2, DFT over m of z[16 m + j]; z is zero for m >= 10
    float2 x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
      x[m] = m < 10 ? make_float2(xr[2 * m] * wj[2 * m], xr[2 * m + 1] * wj[2 * m + 1])
                    : make_float2(0.f, 0.f);
    const int64_t g1 = g0 + (int64_t)gridDim.x * FPB;
    if (g1 < total) fetch(g1);
    dft16_head10(x);
#pragma unroll
    for (int k1 = 0; k1 < 16; ++k1) {
      const float2 t = k1 == 0 ? x[0] : cmul(x[k1], tw256[(j * k1) & 255]);
      T[k1 * TLD + j] = t;
    }
    wave_sync();
    // pass 2: lane j = k1, DFT over n2
#pragma unroll
    for (int n2 = 0; n2 < 16; ++n2) x[n2] = T[j * TLD + n2];
    dft16(x);                       // x[k2] = Z[j + 16 k2]
    wave_sync();
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) T[j + 16 * k2] = x[k2];
    wave_sync();
    // real split: twice the magnitudes of bins j + 16 k2 (and 256 on lane 0)
    float mg[16];
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) {
      const int k = j + 16 * k2;
      const float2 zk = x[k2], zn = T[(256 - k) & 255];
      const float ex = zk.x + zn.x, ey = zk.y - zn.y;  // 2 E[k]
      const float ox = zk.y + zn.y, oy = zn.x - zk.x;  // 2 O[k]
      const float2 w = tw512[k];
      const float xx = fmaf(w.x, ox, fmaf(-w.y, oy, ex));
      const float xy = fmaf(w.x, oy, fmaf(w.y, ox, ey));
      mg[k2] = __builtin_amdgcn_sqrtf(fmaf(xx, xx, xy * xy));
    }
    const float m256 = 2.0f * fabsf(x[0].x - x[0].y);
    wave_sync();
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) M[j + 16 * k2] = mg[k2];
    if (j == 0) M[256] = m256;
    wave_sync();
    // mel bands j, j + 16, ..., then the log (v_log_f32 is log2)
    float out[8];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const float* mp = M + bstart[j + 16 * i];
      const float* wp = bw + g_mel.group_woff[i] + j;
      const int q_len = g_mel.group_len[i];
      float acc = 0.f;
      for (int q = 0; q < q_len; ++q) acc = fmaf(mp[q], wp[16 * q], acc);
      out[i] = __builtin_amdgcn_logf(acc + kMelFloor) * 0.69314718055994530942f;
    }
    wave_sync();
    // the frame's 128 outputs through LDS, then 32 contiguous bytes per lane
    float* O = M + 260;
#pragma unroll
    for (int i = 0; i < 8; ++i) O[j + 16 * i] = out[i];
    wave_sync();
    if (active) {
      const float4 a = *(const float4*)(O + 8 * j), c = *(const float4*)(O + 8 * j + 4);
      float* dst = mel + g * kMels + 8 * j;
      *(float4*)dst = a;
      *(float4*)(dst + 4) = c;
    }
    wave_sync();
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
  const int64_t blocks = (total_frames + FPB - 1) / FPB;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(k_logmel, dim3(grid), dim3(256), 0, s, wave, sample_off, frame_off, B,
                     total_frames, mel);
  return hipGetLastError();
}

}  // namespace ae
