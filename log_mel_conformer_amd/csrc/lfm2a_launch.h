// Internal launchers of the LFM2A encoder kernels (cera 0.5.3,
// src/model/audio_encoder_gpu.rs). Shapes are validated by the C-ABI layer.
#pragma once

#include "launch.h"
#include "../../include/lfm2a.h"

namespace ae {
namespace lfm {

constexpr int kNFft = 512;
constexpr int kBins = kNFft / 2 + 1;   // 257
constexpr int kWin = 400;
constexpr int kHop = 160;
constexpr int kCenterPad = kNFft / 2;  // 256 zeros before the clip
constexpr int kMel = 128;
constexpr float kPreemph = 0.97f;
constexpr float kLogEps = 5.9604644775390625e-08f;  // 2^-24
constexpr float kNormEps = 1e-5f;
constexpr int kStemCh = 256;
constexpr int kF1 = 64, kF2 = 32, kF3 = 16;  // frequencies after each stride-2 layer
constexpr int kD = 512;
constexpr int kHeads = 8;
constexpr int kHd = 64;
constexpr int kKern = 9;
constexpr int kStatSlices = 16;

// ------------------------------------------------------------- front end
hipError_t frontend_init();
// raw ln(mel + 2^-24) [total_frames][128]
hipError_t launch_logmel_raw(const float* wave, const int64_t* sample_off,
                             const int64_t* frame_off, int B, int64_t total_frames, float* mel,
                             hipStream_t s);
// per-clip, per-band mean and 1 / (std + eps) over the first n / 160
// frames -> stats [B][128][2]; part: [B][kStatSlices][128][2] doubles
hipError_t launch_mel_stats(const float* mel, const int64_t* sample_off,
                            const int64_t* frame_off, int B, double* part, float* stats,
                            hipStream_t s);
// in place: (x - mean) * inv for the statistics frames, 0 after them
hipError_t launch_mel_norm(float* mel, const int64_t* sample_off, const int64_t* frame_off, int B,
                           int64_t total_frames, const float* stats, hipStream_t s);

// ------------------------------------------------------------------ stem
// layers 0 and 1 in one pass: 3x3 stride 2 pad 1, 1 -> 256 channels, +
// bias, ReLU, then depthwise 3x3 stride 2 pad 1 + bias. feat [frames][128]
// float -> y2 [rows2][32][256] bf16 (channels last); wt1: layer 1's taps
// [9][256]
hipError_t launch_stem01(const float* feat, const int64_t* frame_off, const int64_t* row1_off,
                         const int64_t* row2_off, int B, int64_t rows2, const float* w0,
                         const float* b0, const float* wt1, const float* b1, bf16* y2,
                         hipStream_t s);
// depthwise 3x3 stride 2 pad 1 + bias on channels-last planes:
// y [rows_in][w_in][256] -> z [rows_out][w_in / 2][256]; wt: taps [9][256]
hipError_t launch_dw3s2(const bf16* y, const int64_t* in_off, const int64_t* out_off, int B,
                        int64_t rows_out, int w_in, const float* wt, const float* b, bf16* z,
                        hipStream_t s);

// ------------------------------------------------------------ row kernels
// y = LN(x; w1, b1) per 512-wide row; if write_x: x = y; if w2: a = LN(y;
// w2, b2) else if a: a = y (a in bf16).
struct LnParams {
  int64_t n;
  float* x;
  const float* w1;
  const float* b1;
  bool write_x;
  const float* w2;
  const float* b2;
  bf16* a;
  float eps;
};
hipError_t launch_layernorm(const LnParams& p, hipStream_t s);

// c = silu((dwconv(g) + b) * aw + ab) along each clip's time axis, zero
// padding (k - 1) / 2 before and k - 1 - (k - 1) / 2 after; g, c bf16
// [n][512]; wt: the taps transposed, [k][512].
hipError_t launch_dwconv(const bf16* g, const int32_t* tok_pos, const int32_t* tok_clip,
                         const int64_t* token_off, int64_t n, const float* wt, int k,
                         const float* b, const float* aw, const float* ab, bf16* c,
                         hipStream_t s);

// pe [2 t_max - 1][dim] bf16: row r at position t_max - 1 - r
hipError_t launch_pos_table(int64_t t_max, int dim, bf16* pe, hipStream_t s);

// ------------------------------------------------------------- attention
// qtile_off [B+1] (device): prefix sums of ceil(t_i / 128) query tiles
hipError_t launch_xl_attention(const bf16* qkv, const bf16* p, int64_t t_max, const float* u,
                               const float* v, const int64_t* token_off,
                               const int64_t* qtile_off, int B, int64_t n_qtiles, bf16* o,
                               hipStream_t s);
constexpr int kQueriesPerBlock = 128;

// ------------------------------------------------------------- model prep
hipError_t launch_f32_to_bf16(const float* src, bf16* dst, int64_t n, hipStream_t s);
// dst[o][f * C + c] = src[o][c * F + f] (rows of C * F)
hipError_t launch_flatten_permute(const bf16* src, int rows, int C, int F, bf16* dst,
                                  hipStream_t s);
// dst[j][c] = src[c][j], src [C][K] float
hipError_t launch_transpose_f32(const float* src, int C, int K, float* dst, hipStream_t s);
hipError_t launch_concat3(const float* a, const float* b, const float* c, int n, float* dst,
                          hipStream_t s);

}  // namespace lfm
}  // namespace ae
