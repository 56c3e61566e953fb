/*
 * lfm2a.h -- C ABI (in libae.so) of the second encoder: the forward pass of
 * the LFM2A Conformer audio encoder on MI355X (gfx950), in hand-written HIP
 * kernels.
 *
 * The operations follow the docs.rs source page of cera 0.5.3,
 * src/model/audio_encoder_gpu.rs ("the page" below): the module
 * documentation, GpuMelFrontend, log_mel_spectrogram_gpu,
 * STEM_LAYER_MODES / STEM_RELU_AFTER, conv_stem_gpu, encode_audio_gpu,
 * macaron_ffn and the AudioEncoderGpuOps method documentation. The page
 * does not print the constants of its CPU modules; this library takes:
 * N_FFT 512 (the page's 4 KB twiddle table), a 400-sample periodic Hann
 * window centred in the 512-point frame, hop 160, center padding of 256
 * zeros per side, pre-emphasis 0.97, 128 Slaney mel bands (area
 * normalised) over 0..8 kHz, ln(power + 2^-24), per-bin normalisation
 * (x - mean) / (std + 1e-5) with the n - 1 divisor over the first n / 160
 * frames, 3x3 stem kernels, LayerNorm eps 1e-5, sinusoidal relative
 * positions with row r of the (2t - 1)-row table at position t - 1 - r.
 *
 * Conventions: as in ae.h (device pointers owned by the caller, every
 * compute call asynchronous on `stream`, allocation-free, validated before
 * any work is queued; errors through ae_status and ae_last_error()).
 * Clips are packed back to back; host offset arrays have B + 1 entries,
 * entry 0 = 0, non-decreasing.
 */
#ifndef LFM2A_H
#define LFM2A_H

#include <stddef.h>
#include <stdint.h>

#include "ae.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Encoder hyper-parameters. Only the defaults are implemented; any other
 * value is AE_ERR_UNSUPPORTED (the kernels are specialised for them). */
typedef struct {
  int32_t n_mel;        /* 128 mel bands */
  int32_t stem_ch;      /* 256 stem channels */
  int32_t n_embd;       /* 512 */
  int32_t n_head;       /* 8 (head_dim 64) */
  int32_t n_ff;         /* 2048 */
  int32_t n_layer;      /* 17 Conformer blocks */
  int32_t conv_kernel;  /* 9 depthwise taps */
  int32_t pos_dim;      /* 512, width of the relative-position table */
  int32_t adapter;      /* 2048, adapter intermediate width */
  int32_t llm_hidden;   /* 2048, output width */
  float eps;            /* 1e-5, LayerNorm eps */
} lfm2a_config;

/* One Conformer block (the page: GpuConformerBlock). Matrices ("mat") are
 * [out][in] row-major bf16 (y = x W^T); vectors are float32. All device
 * pointers, 16-byte aligned, borrowed: they must outlive the model. */
typedef struct {
  const float *ffn_norm_w, *ffn_norm_b;
  const void* ffn_up_w;      const float* ffn_up_b;      /* [n_ff][n_embd] */
  const void* ffn_down_w;    const float* ffn_down_b;    /* [n_embd][n_ff] */
  const float *ln1_w, *ln1_b;
  const void* attn_q_w;      const float* attn_q_b;      /* [n_embd][n_embd] */
  const void* attn_k_w;      const float* attn_k_b;
  const void* attn_v_w;      const float* attn_v_b;
  const void* attn_o_w;      const float* attn_o_b;
  const float *pos_bias_u, *pos_bias_v;                  /* [n_embd] = [n_head][64] */
  const void* linear_pos_w;                              /* [n_embd][pos_dim], no bias */
  const float *norm_conv_w, *norm_conv_b;                /* LayerNorm of the conv module */
  const void* conv_pw1_w;    const float* conv_pw1_b;    /* [2 n_embd][n_embd] */
  const float* conv_dw_w;    const float* conv_dw_b;     /* [n_embd][conv_kernel], [n_embd] */
  const float *conv_norm_w, *conv_norm_b;                /* per-channel affine before SiLU */
  const void* conv_pw2_w;    const float* conv_pw2_b;    /* [n_embd][n_embd] */
  const float *ffn_norm_1_w, *ffn_norm_1_b;
  const void* ffn_up_1_w;    const float* ffn_up_1_b;
  const void* ffn_down_1_w;  const float* ffn_down_1_b;
  const float *ln2_w, *ln2_b;
} lfm2a_block_weights;

/* The whole encoder. Stem weights are float32 in the page's
 * [out_ch][in_per_group][kh][kw] layout: stem_w[0] [256][1][3][3],
 * stem_w[1] and stem_w[3] depthwise [256][1][3][3], stem_w[2] and
 * stem_w[4] pointwise [256][256][1][1]; stem_b[i] [256]. pre_encode_out_w
 * is bf16 [n_embd][stem_ch * n_mel / 8] with input column c * 16 + f
 * (channel-major flatten). `blocks` is a host array of n_layer entries,
 * read during lfm2a_model_create; everything else is device memory. */
typedef struct {
  const float* stem_w[5];
  const float* stem_b[5];
  const void* pre_encode_out_w;  const float* pre_encode_out_b;
  const lfm2a_block_weights* blocks;
  const float *adapter_norm_w, *adapter_norm_b;
  const void* adapter_up_w;      const float* adapter_up_b;     /* [adapter][n_embd] */
  const void* adapter_down_w;    const float* adapter_down_b;   /* [llm_hidden][adapter] */
} lfm2a_weights;

typedef struct lfm2a_model lfm2a_model; /* opaque */

void lfm2a_config_default(lfm2a_config* cfg);

/* --- sizes (host only) ------------------------------------------------ */

/* STFT frames of an n-sample clip: 0 if n <= 0, else 1 + n / 160. */
int64_t lfm2a_num_frames(int64_t n_samples);
/* Tokens after the stem: the frame count through three stride-2 3x3
 * convolutions with padding 1, h -> (h - 1) / 2 + 1 each. */
int64_t lfm2a_num_tokens(int64_t n_samples);

/* Prefix sums of B clips of n_samples[i] samples (host arrays of B + 1
 * entries written by the call): samples, frames and tokens. Any output may
 * be NULL. A negative length is AE_ERR_INVALID; a clip of 1..319 samples
 * has fewer than two statistics frames and is AE_ERR_SHAPE (an empty clip
 * is allowed: no frames, no tokens). */
ae_status lfm2a_plan(const int64_t* n_samples, int32_t B, int64_t* sample_off,
                     int64_t* frame_off, int64_t* token_off);
/* Token prefix sums from a packed feature layout (what lfm2a_stem
 * receives): frame_off host int64 [B+1], non-decreasing from 0; token_off
 * host int64 [B+1] written by the call (clip i: its frame count through the
 * stem's three stride-2 convolutions). AE_ERR_INVALID for bad offsets. */
ae_status lfm2a_plan_frames(const int64_t* frame_off, int32_t B, int64_t* token_off);

/* --- front end -------------------------------------------------------- */

/* Workspace bytes of lfm2a_logmel for B clips. */
size_t lfm2a_logmel_workspace_bytes(int32_t B);

/* Normalised log-mel features (the page: log_mel_spectrogram_gpu and the
 * stft_frames, power_spec, mel_project, mel_norm ops). wave: device float,
 * clip i at [sample_off[i], sample_off[i+1]) (host int64 [B+1]).
 * feat: device float [sum F_i][128] time-major, F_i = lfm2a_num_frames.
 * Frame j of a clip is the pre-emphasised clip, zero-padded by 256 on
 * each side, samples [160 j, 160 j + 512), times the centred window;
 * |DFT|^2 on 257 bins, the 128 Slaney bands, ln(band + 2^-24), then each
 * band normalised over the clip's first n / 160 frames; the frames after
 * those are 0. Clips of 1..319 samples are AE_ERR_SHAPE. */
ae_status lfm2a_logmel(const float* wave, const int64_t* sample_off, int32_t B, float* feat,
                       void* ws, size_t ws_bytes, ae_stream stream);

/* --- model ------------------------------------------------------------ */

/* Validate the configuration (every weight pointer non-NULL and 16-byte
 * aligned, else AE_ERR_INVALID) and build the model's own tables on the
 * current device (bf16 copies of the pointwise stem weights, the
 * projection input columns reordered to the channels-last flatten, the
 * transposed depthwise taps of the stem and of every block's convolution
 * module, the concatenated q|k|v biases). Only
 * dtype AE_BF16 is implemented (bf16 matrices and MFMA operands, float32
 * accumulation, residual stream, norms and softmax). On error *out is
 * NULL. */
ae_status lfm2a_model_create(const lfm2a_config* cfg, const lfm2a_weights* w, ae_dtype dtype,
                             ae_stream stream, lfm2a_model** out);
void lfm2a_model_destroy(lfm2a_model* m);

/* Workspace bytes of lfm2a_stem / lfm2a_block / lfm2a_adapter /
 * lfm2a_encode for B clips with these totals (samples, frames and tokens
 * over the batch) and the longest clip's token count. */
size_t lfm2a_workspace_bytes(const lfm2a_model* m, int32_t B, int64_t total_frames,
                             int64_t total_tokens, int64_t max_tokens);

/* --- compute ------------------------------------------------------------ */

/* Conv stem and input projection (the page: conv_stem_gpu). feat: device
 * float [sum F_i][128] with clip i at rows [frame_off[i], frame_off[i+1])
 * (host int64 [B+1]). x: device float [sum T_i][n_embd]. */
ae_status lfm2a_stem(const lfm2a_model* m, const float* feat, const int64_t* frame_off,
                     int32_t B, float* x, void* ws, size_t ws_bytes, ae_stream stream);

/* One Conformer block in place (the page: encode_audio_gpu, stage 3):
 * FFN-1/2, self-attention with the Transformer-XL relative-position term
 * over each whole clip, convolution module, FFN-1/2, final LayerNorm.
 * x: device float [n][n_embd], clip i at rows [token_off[i],
 * token_off[i+1]) (host int64 [B+1], n = token_off[B]). */
ae_status lfm2a_block(const lfm2a_model* m, int32_t layer, float* x, const int64_t* token_off,
                      int32_t B, void* ws, size_t ws_bytes, ae_stream stream);

/* MLP adapter (the page: encode_audio_gpu, stage 4): LayerNorm, up,
 * erf GELU, down. x: device float [n][n_embd]; out: device float
 * [n][llm_hidden]. */
ae_status lfm2a_adapter(const lfm2a_model* m, const float* x, int64_t n, float* out, void* ws,
                        size_t ws_bytes, ae_stream stream);

/* The whole encoder from 16 kHz PCM (the page: encode_audio_pcm_gpu) for
 * a batch: front end, stem, n_layer blocks, adapter. out: device float
 * [sum T_i][llm_hidden], clip after clip. */
ae_status lfm2a_encode(const lfm2a_model* m, const float* wave, const int64_t* sample_off,
                       int32_t B, float* out, void* ws, size_t ws_bytes, ae_stream stream);

/* The attention kernel alone (the page: xl_attention): per clip and head,
 * score(i, j) = ((q_i + u) . k_j + (q_i + v) . p[t_max - 1 - i + j]) / 8,
 * softmax over the clip's keys, output sum_j softmax_ij v_j.
 * qkv: device bf16 [n][3 n_embd] (q | k | v); p: device bf16
 * [2 t_max - 1][n_embd], row r the projected table row of position
 * t_max - 1 - r, t_max >= every clip's length; u, v: device float
 * [n_embd]; token_off: host int64 [B+1]; o: device bf16 [n][n_embd].
 * n_embd must be 512 and n_head 8. ws: lfm2a_attention_workspace_bytes. */
size_t lfm2a_attention_workspace_bytes(int32_t B);
ae_status lfm2a_xl_attention(const void* qkv, const void* p, int64_t t_max, const float* u,
                             const float* v, const int64_t* token_off, int32_t B, void* o,
                             void* ws, size_t ws_bytes, ae_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* LFM2A_H */
