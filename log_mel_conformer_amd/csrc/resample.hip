// Channel mixdown and band-limited resampling, the step ahead of the
// log-mel (egemma2_audio.rs, to_mono_16k and resample_hq).
//
// Resampling from rate F to rate T (g = gcd, o = F/g input samples per
// nw = T/g outputs): output m = f nw + j sits at input position
// f o + j o / nw, and
//   y[m] = sum_n x[n] h(n - m F/T),
//   h(d) = c sinc(c d) I0(beta sqrt(1 - (c d / 64)^2)) / I0(beta) for |c d| < 64,
// c = min(1, T/F) * 0.958, beta = 12.8, summed in float64 and rounded to
// float32. All outputs of phase j apply the same taps at the same integer
// offsets around f o, so the resampler is planned once per rate pair: a
// device table of those taps, phase-minor ([q][j], q = tap index from the
// phase's first offset lo[j]), in float64.
//
// Resampling kernel: a wavefront takes JW = min(nw, 64) consecutive phases
// times FW = 64 / JW frames per lane group, R frames per lane (strided by
// FW, so neighbouring lanes read neighbouring frames). It stages every input
// sample its outputs touch, the union [f0 o + lo[j0], ...), in LDS as
// float (zeros outside the clip), then each lane walks the taps: one table
// load (coalesced over phases, a broadcast for a single phase) feeds R
// float64 FMAs on samples read from LDS.
#include <math.h>

#include <algorithm>
#include <string>
#include <vector>

#include "launch.h"

namespace ae {
namespace {

constexpr double kZeroCrossings = 64.0;
constexpr double kRolloff = 0.958;
constexpr double kKaiserBeta = 12.8;
constexpr int kWaves = 4;                 // wavefronts per block
constexpr int kMaxRate = 768000;
constexpr size_t kLdsBudget = 64 * 1024;  // per block, so two blocks share a CU
constexpr size_t kLdsMax = 160 * 1024;

// I0 by its power series: the k-th term is the (k-1)-th times (x/2)^2 / k^2;
// summed until a term drops below 1e-17 of the total.
__device__ double bessel_i0(double x) {
  const double q = 0.25 * x * x;
  double term = 1.0, total = 1.0;
  for (int k = 1; k < 400; ++k) {
    term = term * q / ((double)k * (double)k);
    total += term;
    if (term < total * 1e-17) break;
  }
  return total;
}

// table[q * nw + j] = h(lo[j] + q - j o / nw) for q < qmax.
__global__ void k_resample_table(int o, int nw, int qmax, double c, const int* __restrict__ lo,
                                 double* __restrict__ table) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)qmax * nw) return;
  const int q = (int)(i / nw), j = (int)(i - (int64_t)q * nw);
  const double e = (double)j * (double)o / (double)nw;
  const double t = ((double)(lo[j] + q) - e) * c;
  double h = 0.0;
  if (fabs(t) < kZeroCrossings) {
    const double r = t / kZeroCrossings;
    const double win = bessel_i0(kKaiserBeta * sqrt(1.0 - r * r)) / bessel_i0(kKaiserBeta);
    const double pt = M_PI * t;
    const double sinc = pt == 0.0 ? 1.0 : sin(pt) / pt;
    h = c * sinc * win;
  }
  table[i] = h;
}

struct RsGeom {
  int o, nw, qmax, jw, fw, jg;  // jg = phase groups = ceil(nw / jw)
  int u;                        // LDS floats per wavefront
  const double* table;          // [qmax][nw]
  const int* lo;                // [nw]
};

template <int R>
__global__ void __launch_bounds__(kWaves * 64) k_resample(const float* __restrict__ x,
                                                          const int64_t* __restrict__ offs, int B,
                                                          RsGeom g, float* __restrict__ y) {
  // offs: in_off [B+1], out_off [B+1], unit_off [B+1]
  const int64_t* in_off = offs;
  const int64_t* out_off = offs + (B + 1);
  const int64_t* unit_off = offs + 2 * (B + 1);
  extern __shared__ float xs[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * kWaves + wave;
  const bool active = u < unit_off[B];
  float* xw = xs + (size_t)wave * g.u;

  int c = 0, j0 = 0, lo0 = 0;
  int64_t f0 = 0, n = 0, m_clip = 0;
  if (active) {
    c = find_clip(unit_off, B, u);
    const int64_t ul = u - unit_off[c];
    const int jgi = (int)(ul % g.jg);
    const int64_t fb = ul / g.jg;
    n = in_off[c + 1] - in_off[c];
    m_clip = out_off[c + 1] - out_off[c];
    j0 = jgi * g.jw;
    const int jmax = min(j0 + g.jw, g.nw) - 1;
    f0 = fb * (int64_t)(g.fw * R);
    lo0 = g.lo[j0];
    const int64_t p0 = f0 * g.o + lo0;
    const int64_t len = (int64_t)(g.fw * R - 1) * g.o + (g.lo[jmax] - lo0) + g.qmax;
    const float* xc = x + in_off[c];
    for (int64_t i = lane; i < len; i += 64) {
      const int64_t p = p0 + i;
      xw[i] = (p >= 0 && p < n) ? xc[p] : 0.0f;
    }
  }
  __syncthreads();
  if (!active) return;

  const int jl = lane % g.jw, fl = lane / g.jw;
  const int j = j0 + jl;
  const bool ok = fl < g.fw && j < g.nw;
  // lanes without an output read valid addresses (phase j0, frame 0)
  const int jj = ok ? j : j0, ff = ok ? fl : 0;
  const float* xl = xw + ff * g.o + (g.lo[jj] - lo0);
  const double* hc = g.table + jj;
  const int step = g.fw * g.o;
  double acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0;
  for (int q = 0; q < g.qmax; ++q) {
    const double h = hc[(int64_t)q * g.nw];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = fma(h, (double)xl[r * step + q], acc[r]);
  }
  if (!ok) return;
  float* yc = y + out_off[c];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t m = (f0 + fl + (int64_t)r * g.fw) * g.nw + j;
    if (m < m_clip) yc[m] = (float)acc[r];
  }
}

// Phase-major copy of the taps with zero padding for the blocked kernel:
// hp[j * qp + padl + q] = table[q][j] for q < qmax, zero elsewhere.
__global__ void k_resample_pad(const double* __restrict__ table, int nw, int qmax, int padl,
                               int qp, double* __restrict__ hp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)nw * qp) return;
  const int j = (int)(i / qp), k = (int)(i - (int64_t)j * qp) - padl;
  hp[i] = (k >= 0 && k < qmax) ? table[(int64_t)k * nw + j] : 0.0;
}

struct FirGeom {
  int o, nw, qp, padl, s8;  // s8: samples a lane walks, a multiple of 8
  int u;                    // LDS floats per wavefront
  const double* hp;         // [nw][qp]
};

// Blocked form for rate pairs whose tap windows overlap from frame to frame
// (o well below the tap count): a wavefront serves ONE phase j, so its taps
// are the same in every lane and come through scalar loads; lane l takes the
// R consecutive frames F0 + l R + r. Frame r's taps start o r samples after
// frame 0's, so walking the lane's samples s = 0 .. (R - 1) o + qmax once,
// each sample read (and converted) once feeds R FMAs:
//   acc[r] += h_j[s - o r] x[base + s]   (h_j zero outside its taps).
template <int R>
__global__ void __launch_bounds__(kWaves * 64) k_resample_fir(const float* __restrict__ x,
                                                              const int64_t* __restrict__ offs,
                                                              int B, FirGeom g,
                                                              const int* __restrict__ lo,
                                                              float* __restrict__ y) {
  const int64_t* in_off = offs;
  const int64_t* out_off = offs + (B + 1);
  const int64_t* unit_off = offs + 2 * (B + 1);
  extern __shared__ float xs[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * kWaves + wave;
  const bool active = u < unit_off[B];
  float* xw = xs + (size_t)wave * g.u;
  int c = 0, j = 0;
  int64_t f0 = 0, m_clip = 0;
  if (active) {
    c = find_clip(unit_off, B, u);
    const int64_t ul = u - unit_off[c];
    j = (int)(ul % g.nw);
    f0 = (ul / g.nw) * (int64_t)(64 * R);
    const int64_t n = in_off[c + 1] - in_off[c];
    m_clip = out_off[c + 1] - out_off[c];
    const int64_t p0 = f0 * g.o + lo[j];
    const int len = 63 * R * g.o + g.s8;
    const float* xc = x + in_off[c];
    for (int i = lane; i < len; i += 64) {
      const int64_t p = p0 + i;
      xw[i] = (p >= 0 && p < n) ? xc[p] : 0.0f;
    }
  }
  __syncthreads();
  if (!active) return;
  j = __builtin_amdgcn_readfirstlane(j);
  const float* xl = xw + lane * R * g.o;
  const double* hj = g.hp + (int64_t)j * g.qp + g.padl;
  double acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0;
  for (int s0 = 0; s0 < g.s8; s0 += 8) {
    double xv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) xv[k] = (double)xl[s0 + k];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const double* h = hj + s0 - r * g.o;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[r] = fma(h[k], xv[k], acc[r]);
    }
  }
  float* yc = y + out_off[c];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t m = (f0 + (int64_t)lane * R + r) * g.nw + j;
    if (m < m_clip) yc[m] = (float)acc[r];
  }
}

// mono[i] = (in[i][0] + in[i][1] + ...) / channels, float32, in channel order.
__global__ void k_mixdown(const float* __restrict__ in, int64_t n, int ch, float* __restrict__ mono) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float* p = in + i * ch;
  float s = p[0];
  for (int k = 1; k < ch; ++k) s += p[k];
  mono[i] = s / (float)ch;
}

__global__ void k_mixdown2(const float2* __restrict__ in, int64_t n, float* __restrict__ mono) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float2 v = in[i];
  mono[i] = (v.x + v.y) / 2.0f;
}

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace
}  // namespace ae

using namespace ae;

struct ae_resampler {
  int from = 0, to = 0, device = 0;
  int o = 1, nw = 1, qmax = 0, jw = 1, fw = 64, jg = 1, R = 1, u = 0;
  double c = 0.0;
  int64_t taps_nonzero_per_cycle = 0;  // nonzero taps summed over the nw phases
  double* table = nullptr;             // device [qmax][nw]
  int* lo = nullptr;                   // device [nw]
  std::vector<int> lo_host;
  // blocked form (k_resample_fir), when consecutive frames' windows overlap
  bool fir = false;
  int fir_r = 1, qp = 0, padl = 0, s8 = 0, fir_u = 0;
  double* hp = nullptr;                // device [nw][qp]
};

extern "C" {

int64_t ae_resampled_length(int64_t n, int32_t from_rate, int32_t to_rate) {
  if (n < 0 || from_rate <= 0 || to_rate <= 0) return -1;
  if (from_rate == to_rate || n == 0) return n;
  const int64_t g = gcd64(from_rate, to_rate);
  const int64_t o = from_rate / g, nw = to_rate / g;
  if (n > (INT64_MAX - o) / nw) return -1;
  return (nw * n + o - 1) / o;
}

ae_status ae_resampler_create(int32_t from_rate, int32_t to_rate, ae_stream stream,
                              ae_resampler** out) {
  if (!out) return set_error(AE_ERR_INVALID, "ae_resampler_create: null output pointer");
  *out = nullptr;
  if (from_rate <= 0 || to_rate <= 0 || from_rate > kMaxRate || to_rate > kMaxRate)
    return set_error(AE_ERR_INVALID, "ae_resampler_create: rates must be in 1.." +
                                         std::to_string(kMaxRate) + " Hz");
  ae_resampler* r = new ae_resampler();
  r->from = from_rate;
  r->to = to_rate;
  hipError_t e = hipGetDevice(&r->device);
  if (e != hipSuccess) {
    delete r;
    return set_error(AE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  }
  if (from_rate != to_rate) {
    const int64_t g = gcd64(from_rate, to_rate);
    r->o = (int)(from_rate / g);
    r->nw = (int)(to_rate / g);
    r->c = (double)std::min(r->o, r->nw) / (double)r->o * kRolloff;
    const double half = kZeroCrossings / r->c;
    r->lo_host.resize(r->nw);
    int qmax = 0;
    int64_t nz = 0;
    for (int j = 0; j < r->nw; ++j) {
      const double e = (double)j * (double)r->o / (double)r->nw;
      const int lo = (int)floor(e - half), hi = (int)ceil(e + half);
      r->lo_host[j] = lo;
      qmax = std::max(qmax, hi - lo + 1);
      for (int d = lo; d <= hi; ++d)
        if (fabs(((double)d - e) * r->c) < kZeroCrossings) ++nz;
    }
    r->qmax = qmax;
    r->taps_nonzero_per_cycle = nz;
    r->jw = std::min(r->nw, 64);
    r->fw = 64 / r->jw;
    r->jg = (r->nw + r->jw - 1) / r->jw;
    int dlo = 0;
    for (int k = 0; k < r->jg; ++k) {
      const int j0 = k * r->jw, j1 = std::min(j0 + r->jw, r->nw) - 1;
      dlo = std::max(dlo, r->lo_host[j1] - r->lo_host[j0]);
    }
    auto lds_floats = [&](int R) {
      return (int64_t)(r->fw * R - 1) * r->o + dlo + r->qmax;
    };
    int R = 8;
    while (R > 1 && (size_t)lds_floats(R) * 4 * kWaves > kLdsBudget) R /= 2;
    if ((size_t)lds_floats(R) * 4 * kWaves > kLdsMax) {
      delete r;
      return set_error(AE_ERR_UNSUPPORTED, "ae_resampler_create: a " +
                                               std::to_string(from_rate) + " -> " +
                                               std::to_string(to_rate) +
                                               " Hz kernel needs more LDS than a CU has");
    }
    r->R = R;
    r->u = (int)lds_floats(R);
    // blocked form: one phase per wavefront, R consecutive frames per lane;
    // odd R keeps the lanes' LDS strides off the 64-bank period for odd o
    if (2 * r->o <= r->qmax) {
      for (int fr : {9, 5, 3, 1}) {
        const int s8 = (((fr - 1) * r->o + r->qmax) + 7) / 8 * 8;
        const int64_t u = (int64_t)63 * fr * r->o + s8;
        if ((size_t)u * 4 * kWaves <= kLdsBudget || (fr == 1 && (size_t)u * 4 * kWaves <= kLdsMax)) {
          r->fir = true;
          r->fir_r = fr;
          r->s8 = s8;
          r->padl = (fr - 1) * r->o;
          r->qp = r->padl + s8;
          r->fir_u = (int)u;
          break;
        }
      }
    }
    const int64_t entries = (int64_t)r->qmax * r->nw;
    if (entries > ((int64_t)1 << 28)) {
      delete r;
      return set_error(AE_ERR_UNSUPPORTED, "ae_resampler_create: tap table beyond 2^28 entries");
    }
    e = hipMalloc(&r->table, sizeof(double) * (size_t)entries);
    if (e == hipSuccess) e = hipMalloc(&r->lo, sizeof(int) * (size_t)r->nw);
    if (e == hipSuccess)
      e = hipMemcpyAsync(r->lo, r->lo_host.data(), sizeof(int) * (size_t)r->nw,
                         hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_resample_table, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0,
                         stream, r->o, r->nw, r->qmax, r->c, r->lo, r->table);
      e = hipGetLastError();
    }
    if (e == hipSuccess && r->fir) {
      const int64_t pe = (int64_t)r->nw * r->qp;
      e = hipMalloc(&r->hp, sizeof(double) * (size_t)pe);
      if (e == hipSuccess) {
        hipLaunchKernelGGL(k_resample_pad, dim3((unsigned)((pe + 255) / 256)), dim3(256), 0,
                           stream, r->table, r->nw, r->qmax, r->padl, r->qp, r->hp);
        e = hipGetLastError();
      }
    }
    // the host copy of lo must outlive the asynchronous upload
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
      if (r->table) hipFree(r->table);
      if (r->lo) hipFree(r->lo);
      if (r->hp) hipFree(r->hp);
      delete r;
      return set_error(AE_ERR_HIP, std::string("ae_resampler_create: ") + hipGetErrorString(e));
    }
  }
  *out = r;
  return AE_OK;
}

void ae_resampler_destroy(ae_resampler* r) {
  if (!r) return;
  int prev = 0;
  hipGetDevice(&prev);
  hipSetDevice(r->device);
  if (r->table) hipFree(r->table);
  if (r->lo) hipFree(r->lo);
  if (r->hp) hipFree(r->hp);
  hipSetDevice(prev);
  delete r;
}

size_t ae_resample_workspace_bytes(int32_t B, int64_t total_frames, int32_t channels) {
  if (B < 0 || total_frames < 0) return 0;
  size_t b = align256(sizeof(int64_t) * 3 * ((size_t)B + 1));
  if (channels > 1) b += align256(sizeof(float) * (size_t)total_frames);
  return b;
}

ae_status ae_resampler_info(const ae_resampler* r, int32_t* taps_per_phase_max,
                            int64_t* nonzero_taps_per_cycle, int32_t* phases,
                            int32_t* in_per_cycle) {
  if (!r) return set_error(AE_ERR_INVALID, "ae_resampler_info: null resampler");
  if (taps_per_phase_max) *taps_per_phase_max = r->qmax;
  if (nonzero_taps_per_cycle) *nonzero_taps_per_cycle = r->taps_nonzero_per_cycle;
  if (phases) *phases = r->nw;
  if (in_per_cycle) *in_per_cycle = r->o;
  return AE_OK;
}

ae_status ae_mixdown(const float* in, int64_t n_frames, int32_t channels, float* mono,
                     ae_stream stream) {
  if (n_frames < 0 || channels < 1)
    return set_error(AE_ERR_INVALID, "ae_mixdown: n_frames >= 0 and channels >= 1 required");
  if (n_frames == 0) return AE_OK;
  if (!in || !mono) return set_error(AE_ERR_INVALID, "ae_mixdown: null pointer");
  const unsigned grid = (unsigned)((n_frames + 255) / 256);
  timing_begin(AE_K_MIXDOWN, stream);
  if (channels == 1) {
    AE_HIP_TRY(hipMemcpyAsync(mono, in, sizeof(float) * (size_t)n_frames,
                              hipMemcpyDeviceToDevice, stream));
  } else if (channels == 2 && ((uintptr_t)in & 7) == 0) {
    hipLaunchKernelGGL(k_mixdown2, dim3(grid), dim3(256), 0, stream, (const float2*)in, n_frames,
                       mono);
  } else {
    hipLaunchKernelGGL(k_mixdown, dim3(grid), dim3(256), 0, stream, in, n_frames, channels,
                       mono);
  }
  timing_end(AE_K_MIXDOWN, stream);
  AE_HIP_TRY(hipGetLastError());
  return AE_OK;
}

ae_status ae_resample(const ae_resampler* r, const float* x, const int64_t* in_off, int32_t B,
                      float* y, void* ws, size_t ws_bytes, ae_stream stream) {
  if (!r) return set_error(AE_ERR_INVALID, "ae_resample: null resampler");
  if (B < 0 || (B > 0 && !in_off)) return set_error(AE_ERR_INVALID, "ae_resample: bad batch");
  if (B == 0) return AE_OK;
  if (in_off[0] != 0) return set_error(AE_ERR_INVALID, "ae_resample: in_off[0] must be 0");
  std::vector<int64_t> offs(3 * ((size_t)B + 1));
  int64_t* out_off = offs.data() + (B + 1);
  int64_t* unit_off = offs.data() + 2 * (B + 1);
  out_off[0] = unit_off[0] = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t len = in_off[i + 1] - in_off[i];
    if (len < 0) return set_error(AE_ERR_INVALID, "ae_resample: in_off must be non-decreasing");
    const int64_t m = ae_resampled_length(len, r->from, r->to);
    if (m < 0) return set_error(AE_ERR_CAPACITY, "ae_resample: clip too long");
    offs[i] = in_off[i];
    out_off[i + 1] = out_off[i] + m;
    int64_t units = 0;
    if (r->from != r->to) {
      const int64_t frames = (m + r->nw - 1) / r->nw;
      if (r->fir)
        units = (int64_t)r->nw * ((frames + 64 * r->fir_r - 1) / (64 * r->fir_r));
      else
        units = (int64_t)r->jg * ((frames + (int64_t)r->fw * r->R - 1) / ((int64_t)r->fw * r->R));
    }
    unit_off[i + 1] = unit_off[i] + units;
  }
  offs[B] = in_off[B];
  if (out_off[B] == 0) return AE_OK;
  if (!x || !y) return set_error(AE_ERR_INVALID, "ae_resample: null data pointer");
  if (r->from == r->to) {
    AE_HIP_TRY(hipMemcpyAsync(y, x, sizeof(float) * (size_t)in_off[B], hipMemcpyDeviceToDevice,
                              stream));
    return AE_OK;
  }
  const size_t need = align256(sizeof(int64_t) * offs.size());
  if (!ws || ws_bytes < need)
    return set_error(AE_ERR_CAPACITY, "ae_resample: workspace needs " + std::to_string(need) +
                                          " bytes");
  int dev = 0;
  AE_HIP_TRY(hipGetDevice(&dev));
  if (dev != r->device)
    return set_error(AE_ERR_INVALID, "ae_resample: the resampler belongs to another device");
  const int64_t units = unit_off[B];
  if ((units + kWaves - 1) / kWaves > INT32_MAX)
    return set_error(AE_ERR_CAPACITY, "ae_resample: batch too large for one launch");
  int64_t* d_offs = (int64_t*)ws;
  AE_HIP_TRY(launch_write_i64(d_offs, offs.data(), (int)offs.size(), stream));
  const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(kWaves * 64);
  if (r->fir) {
    FirGeom fg;
    fg.o = r->o;
    fg.nw = r->nw;
    fg.qp = r->qp;
    fg.padl = r->padl;
    fg.s8 = r->s8;
    fg.u = r->fir_u;
    fg.hp = r->hp;
    const size_t lds = sizeof(float) * (size_t)r->fir_u * kWaves;
    const void* fn = r->fir_r == 9 ? (const void*)k_resample_fir<9>
                     : r->fir_r == 5 ? (const void*)k_resample_fir<5>
                     : r->fir_r == 3 ? (const void*)k_resample_fir<3>
                                     : (const void*)k_resample_fir<1>;
    if (lds > 64 * 1024)
      AE_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    timing_begin(AE_K_RESAMPLE, stream);
    switch (r->fir_r) {
      case 9: hipLaunchKernelGGL(k_resample_fir<9>, grid, block, lds, stream, x, d_offs, B, fg, r->lo, y); break;
      case 5: hipLaunchKernelGGL(k_resample_fir<5>, grid, block, lds, stream, x, d_offs, B, fg, r->lo, y); break;
      case 3: hipLaunchKernelGGL(k_resample_fir<3>, grid, block, lds, stream, x, d_offs, B, fg, r->lo, y); break;
      default: hipLaunchKernelGGL(k_resample_fir<1>, grid, block, lds, stream, x, d_offs, B, fg, r->lo, y); break;
    }
    timing_end(AE_K_RESAMPLE, stream);
    AE_HIP_TRY(hipGetLastError());
    return AE_OK;
  }
  RsGeom g;
  g.o = r->o;
  g.nw = r->nw;
  g.qmax = r->qmax;
  g.jw = r->jw;
  g.fw = r->fw;
  g.jg = r->jg;
  g.u = r->u;
  g.table = r->table;
  g.lo = r->lo;
  const size_t lds = sizeof(float) * (size_t)r->u * kWaves;
  if (lds > 64 * 1024) {
    const void* fn = r->R == 8 ? (const void*)k_resample<8>
                     : r->R == 4 ? (const void*)k_resample<4>
                     : r->R == 2 ? (const void*)k_resample<2> : (const void*)k_resample<1>;
    AE_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  }
  timing_begin(AE_K_RESAMPLE, stream);
  switch (r->R) {
    case 8: hipLaunchKernelGGL(k_resample<8>, grid, block, lds, stream, x, d_offs, B, g, y); break;
    case 4: hipLaunchKernelGGL(k_resample<4>, grid, block, lds, stream, x, d_offs, B, g, y); break;
    case 2: hipLaunchKernelGGL(k_resample<2>, grid, block, lds, stream, x, d_offs, B, g, y); break;
    default: hipLaunchKernelGGL(k_resample<1>, grid, block, lds, stream, x, d_offs, B, g, y); break;
  }
  timing_end(AE_K_RESAMPLE, stream);
  AE_HIP_TRY(hipGetLastError());
  return AE_OK;
}

ae_status ae_to_mono_16k(const ae_resampler* r, const float* in, const int64_t* in_off,
                         int32_t B, int32_t channels, float* y, void* ws, size_t ws_bytes,
                         ae_stream stream) {
  if (!r) return set_error(AE_ERR_INVALID, "ae_to_mono_16k: null resampler");
  if (r->to != 16000)
    return set_error(AE_ERR_INVALID, "ae_to_mono_16k: the resampler must target 16000 Hz");
  if (channels < 1) return set_error(AE_ERR_INVALID, "ae_to_mono_16k: channels >= 1 required");
  if (B < 0 || (B > 0 && !in_off)) return set_error(AE_ERR_INVALID, "ae_to_mono_16k: bad batch");
  if (B == 0) return AE_OK;
  const int64_t frames = in_off[B];
  if (channels == 1) return ae_resample(r, in, in_off, B, y, ws, ws_bytes, stream);
  const size_t need = ae_resample_workspace_bytes(B, frames, channels);
  if (!ws || ws_bytes < need)
    return set_error(AE_ERR_CAPACITY, "ae_to_mono_16k: workspace needs " + std::to_string(need) +
                                          " bytes");
  const size_t off_bytes = align256(sizeof(int64_t) * 3 * ((size_t)B + 1));
  float* mono = (float*)((char*)ws + off_bytes);
  ae_status st = ae_mixdown(in, frames, channels, mono, stream);
  if (st != AE_OK) return st;
  return ae_resample(r, mono, in_off, B, y, ws, off_bytes, stream);
}

}  // extern "C"
