// Log-mel front end: framing, periodic Hann window, 512-point real FFT
// magnitude, 128 HTK mel bands, natural log (egemma2_audio.rs, module
// documentation step 2, mel_filter_bank and MelFrontend::log_mel).
//
// Sixteen lanes per frame, four frames per wavefront. The 512-point real
// FFT is a 256-point complex FFT of z[n] = x[2n] + i x[2n+1] (the last 96
// z are zero: the frame is 320 samples), split as 256 = 16 x 16: lane j
// first takes the 16-point DFT over z[16 m + j] in registers (ten nonzero
// inputs), multiplies by e^{-2 pi i j k / 256} (the lane's 15 twiddles kept
// in registers), and the wavefront transposes through LDS; lane j then
// takes the 16-point DFT over the other index and holds Z[j + 16 k]. The
// real spectrum follows from pairs (k, 256 - k):
// 2 X[k] = 2E + w 2O and 2 X[256-k] = conj(2E - w 2O), with
// 2E = Z[k] + conj Z[256-k], 2O = -i (Z[k] - conj Z[256-k]) and
// w = e^{-2 pi i k / 512}; the partner Z[256-k] comes from lane
// (16 - j) mod 16 by ds_bpermute, so one pair gives two bins. The factor 2
// is taken out of the mel weights, which are halved on the host (exact).
// The mel bank has at most two nonzero weights per bin (506 in all), so
// each band is a short contiguous dot product over its own bins; lane j
// takes bands j, j + 16, ..., and each group of sixteen bands reads a
// fixed, compile-time number of bins (its widest band's count, the others'
// weights padded with zeros). All exchanges stay inside a wavefront.
//
// Instruction economy (the kernel is bound by VALU issue): a block walks a
// contiguous run of frames, so a lane finds its clip by one binary search
// and then only steps forward; a frame's samples are read through one
// pointer with immediate offsets (only a clip's first frame, which starts
// before the clip, takes a checked path); the window weights and twiddles
// stay in registers; the square root and logarithm are the hardware ones
// (v_sqrt_f32, v_log_f32: about one ulp, far inside the front end's 1e-4
// tolerance). Window, twiddle and band tables are computed on the host in
// double, rounded to float once.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "fft16.h"
#include "launch.h"

namespace ae {
namespace {

constexpr int kMaxBandW = 1024;
constexpr int kGroups = kMels / 16;  // band groups: bands 16 i .. 16 i + 15
constexpr int FPB = 16;        // frames per block (4 per wavefront)
// Bins read per band of each group (the group's widest band): fixed by the
// bank (16 kHz, 512-point FFT, 128 HTK bands, 130 edges over 0..8 kHz) and
// checked against the bank the host builds, so the band loops unroll. Each
// band's weights sit in a list of its own, padded to whole float4s.
constexpr int kGroupLen[kGroups] = {2, 2, 2, 3, 4, 6, 8, 11};
constexpr int group_stride(int i) { return (kGroupLen[i] + 3) & ~3; }
constexpr int group_woff(int i) { return i == 0 ? 0 : group_woff(i - 1) + 16 * group_stride(i - 1); }
static_assert(group_woff(kGroups) <= kMaxBandW, "band weights fit the table");

struct MelTables {
  float hann[kFrame];
  float2 tw256[256];        // exp(-2 pi i m / 256)
  float2 tw512[256];        // exp(-2 pi i m / 512), m < 256
  int band_start[kMels];    // first bin a band reads (its padded list stays below bin 257)
  float band_w[kMaxBandW];  // half the filter weights: group i, band j of it, bin q at
                            // group_woff(i) + j * group_stride(i) + q, zero padded
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
  for (int i = 0; i < kMaxBandW; ++i) t->band_w[i] = 0.0f;
  for (int i = 0; i < kGroups; ++i) {
    int q_len = 0;
    for (int j = 0; j < 16; ++j) q_len = std::max(q_len, count[16 * i + j]);
    if (q_len != kGroupLen[i]) return false;  // the kernel's unrolled band loops
    for (int j = 0; j < 16; ++j) {
      const int b = 16 * i + j;
      const int s0 = std::min(start[b], kBins - q_len);
      const int shift = start[b] - s0;
      t->band_start[b] = s0;
      for (int q = 0; q < q_len; ++q) {
        const int e = q - shift;
        t->band_w[group_woff(i) + j * group_stride(i) + q] =
            (e >= 0 && e < count[b]) ? (float)(0.5 * wts[b][e]) : 0.0f;
      }
    }
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

// Per-frame LDS image: the 16x16 transpose (float2, rows padded to 17),
// later the 257 magnitudes and the 128 outputs at a per-frame offset of
// 0, 48, 32 or 16 floats (the frame's slot in its wavefront), so the four
// frames of a wavefront write their magnitudes and outputs into distinct
// banks.
__device__ __forceinline__ int mag_off(int f4) { return (64 - 16 * f4) & 63; }

// The partner of lane j's pass-2 bin j + 16 k2 is bin 256 - j - 16 k2,
// held by lane (16 - j) mod 16 of the same frame in register 15 - k2
// (lanes 0 and 8 are their own partners; lane 0's partner of k2 sits one
// register further, in x[(16 - k2) mod 16]).
__device__ __forceinline__ float bperm(int addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}

__global__ void __launch_bounds__(256) k_logmel(const float* __restrict__ wave,
                                                const int64_t* __restrict__ sample_off,
                                                const int64_t* __restrict__ frame_off, int B,
                                                int64_t total, float* __restrict__ mel) {
  __shared__ float2 tw256[256];
  __shared__ float2 tw512[256];
  __shared__ float hann[kFrame];
  __shared__ int bstart[kMels];
  __shared__ __attribute__((aligned(16))) float bw[kMaxBandW];
  __shared__ int64_t soff[MAXB_LDS + 1], foff[MAXB_LDS + 1];
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
  const int f4 = lane >> 4;
  const int fl = wv * 4 + f4;            // frame slot in the block
  const int j = lane & 15;
  float2* T = xbuf[fl];
  float* M = (float*)xbuf[fl] + mag_off(f4);  // magnitudes, after the split
  float* O = M + 260;                         // the frame's 128 outputs
  // this lane's samples of a frame are 32 m + 2 j + e (m < 10, e < 2): their
  // window weights, for every frame
  float wj[20];
#pragma unroll
  for (int m = 0; m < 10; ++m)
#pragma unroll
    for (int e = 0; e < 2; ++e) wj[2 * m + e] = hann[32 * m + 2 * j + e];
  // the lane's twiddles: e^{-2 pi i j k1 / 256} between the passes (j k1 <
  // 256) and e^{-2 pi i (j + 16 k2) / 512} of its split pairs
  float2 tw1[16], tw2[8];
#pragma unroll
  for (int k1 = 1; k1 < 16; ++k1) tw1[k1] = tw256[j * k1];
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) tw2[k2] = tw512[j + 16 * k2];
  const int bp_addr = 4 * ((lane & 48) | ((16 - j) & 15));
  const bool self0 = j == 0;
  // the lane's mel bands j + 16 i: first bin read
  int bs[kGroups];
#pragma unroll
  for (int i = 0; i < kGroups; ++i) bs[i] = bstart[j + 16 * i];
  // Each block takes a contiguous run of frames, FPB at a time, so a lane's
  // clip index only moves forward: a binary search for its first frame,
  // then a step past any clip that ended since the last group (clips of no
  // frames are stepped over).
  const int64_t per = ((total + (int64_t)gridDim.x * FPB - 1) / ((int64_t)gridDim.x * FPB)) * FPB;
  const int64_t gbeg = (int64_t)blockIdx.x * per;
  const int64_t gend = gbeg + per < total ? gbeg + per : total;
  int clip = -1;
  auto fo = [&](int i) -> int64_t { return lds_off ? foff[i] : frame_off[i]; };
  auto so = [&](int i) -> int64_t { return lds_off ? soff[i] : sample_off[i]; };
  // the lane's clip kept in registers: its first frame and sample and the
  // next clip's first frame, read again only when a frame crosses into a
  // later clip (256 x 30 s: 358 -> 352 us against an LDS read per frame)
  int64_t fo_cur = 0, fo_next = 0, so_cur = 0;
  // Raw samples of the frame group a block handles next: loaded one group
  // ahead (register double buffer). A frame starts 160 samples early; only
  // a clip's first frame reaches before the clip, and it (and a slot past
  // the block's last frame) takes the checked path, where samples before
  // the clip are zeros.
  float xr[20];
  auto fetch = [&](int64_t g0) {
    const int64_t g = g0 + fl;
    int64_t base = 0;
    int lim = 1 << 30;  // samples below this index are zeros (all, past the end)
    if (g < gend) {
      if (clip < 0 || g >= fo_next) {
        if (clip < 0) clip = lds_off ? find_clip_lds(foff, B, g) : find_clip(frame_off, B, g);
        else
          while (fo(clip + 1) <= g) ++clip;
        fo_cur = fo(clip);
        fo_next = fo(clip + 1);
        so_cur = so(clip);
      }
      const int64_t start = so_cur;
      base = start + (g - fo_cur) * kHop - kHop;
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
  if (gbeg < gend) fetch(gbeg);
  for (int64_t g0 = gbeg; g0 < gend; g0 += FPB) {
    const int64_t g = g0 + fl;
    const bool active = g < gend;
    // pass 1: lane j = n2, DFT over m of z[16 m + j]; z is zero for m >= 10
    float2 x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
      x[m] = m < 10 ? make_float2(xr[2 * m] * wj[2 * m], xr[2 * m + 1] * wj[2 * m + 1])
                    : make_float2(0.f, 0.f);
    if (g0 + FPB < gend) fetch(g0 + FPB);
    dft16_head10(x);
    T[j] = x[0];
#pragma unroll
    for (int k1 = 1; k1 < 16; ++k1) T[k1 * TLD + j] = cmul(x[k1], tw1[k1]);
    wave_sync();
    // pass 2: lane j = k1, DFT over n2
#pragma unroll
    for (int n2 = 0; n2 < 16; ++n2) x[n2] = T[j * TLD + n2];
    dft16(x);                       // x[k2] = Z[j + 16 k2]
    // partners Z[256 - j - 16 k2], k2 < 8, from lane (16 - j) mod 16
    float2 zp[8];
    {
      float2 r[8];
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2)
        r[k2] = make_float2(bperm(bp_addr, x[15 - k2].x), bperm(bp_addr, x[15 - k2].y));
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) {
        const float2 own = k2 == 0 ? x[0] : r[k2 - 1];
        zp[k2] = make_float2(self0 ? own.x : r[k2].x, self0 ? own.y : r[k2].y);
      }
    }
    // Real split on pairs (k, 256 - k), k = j + 16 k2: with 2E = Z[k] +
    // conj Z[256-k] and 2O = -i (Z[k] - conj Z[256-k]), 2 X[k] = 2E + w 2O
    // and 2 X[256-k] = conj(2E - w 2O), w = e^{-2 pi i k / 512}. Lane 0's
    // k2 = 0 pair gives X[0] and X[256]; bin 128 (its own partner) is
    // |2 X[128]| = 2 |Z[128]|, lane 0's x[8]. The factor 2 is taken out of
    // the mel weights.
    float mk[8], mn[8];
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
      const float2 zk = x[k2], zn = zp[k2];
      const float ex = zk.x + zn.x, ey = zk.y - zn.y;  // 2E
      const float ox = zk.y + zn.y, oy = zn.x - zk.x;  // 2O
      const float2 w = tw2[k2];
      const float px = fmaf(w.x, ox, -w.y * oy), py = fmaf(w.x, oy, w.y * ox);
      const float ax = ex + px, ay = ey + py, bx = ex - px, by = ey - py;
      mk[k2] = __builtin_amdgcn_sqrtf(fmaf(ax, ax, ay * ay));
      mn[k2] = __builtin_amdgcn_sqrtf(fmaf(bx, bx, by * by));
    }
    const float m128 = 2.0f * __builtin_amdgcn_sqrtf(fmaf(x[8].x, x[8].x, x[8].y * x[8].y));
    wave_sync();  // every lane's pass-2 reads of T are done before M overwrites it
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
      M[j + 16 * k2] = mk[k2];
      M[256 - j - 16 * k2] = mn[k2];
    }
    if (self0) M[128] = m128;
    wave_sync();
    // mel bands j, j + 16, ..., then the log (v_log_f32 is log2)
    float out[8];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const float* mp = M + bs[i];
      const float4* wp = (const float4*)(bw + group_woff(i) + j * group_stride(i));
      float acc = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < group_stride(i) / 4; ++q4) {
        const float4 w = wp[q4];
        const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q4 + e < kGroupLen[i]) acc = fmaf(mp[4 * q4 + e], wv[e], acc);
      }
      out[i] = __builtin_amdgcn_logf(acc + kMelFloor) * 0.69314718055994530942f;
    }
    // the frame's 128 outputs through LDS (O does not overlap M), then
    // 256 contiguous bytes per store instruction of the frame's 16 lanes
#pragma unroll
    for (int i = 0; i < 8; ++i) O[j + 16 * i] = out[i];
    wave_sync();
    if (active) {
      const float4 a = *(const float4*)(O + 4 * j), c = *(const float4*)(O + 64 + 4 * j);
      float* dst = mel + g * kMels + 4 * j;
      *(float4*)dst = a;
      *(float4*)(dst + 64) = c;
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
  // One round of blocks, three per CU (the block's 51.8 KB of LDS allows no
  // more), each walking an equal run of frames, so every block sets up its
  // registers and tables once: 32 x 30 s took 52.5 us against 59.4 for a
  // grid of up to 4096 blocks (two groups each), 256 x 30 s 374 against
  // 381 us; two and three rounds measured in between.
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
  const int64_t blocks = (total_frames + FPB - 1) / FPB;
  const int64_t slots = 3 * (int64_t)n_cu;
  const int grid = (int)(blocks < slots ? blocks : slots);
  hipLaunchKernelGGL(k_logmel, dim3(grid), dim3(256), 0, s, wave, sample_off, frame_off, B,
                     total_frames, mel);
  return hipGetLastError();
}

}  // namespace ae
