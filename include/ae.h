/*
 * ae.h -- C ABI of libae.so: the forward pass of the log-mel + Conformer
 * audio encoder (the gemma4_audio tower of EmbeddingGemma 2) on MI355X
 * (gfx950), in hand-written HIP kernels.
 *
 * The operations follow the docs.rs source page of cortiq-engine 0.8.49,
 * cortiq_engine/egemma2_audio.rs ("the page" below): its module
 * documentation (steps 1-5), MelFrontend::log_mel, AudioTower::subsample,
 * ffn, attention, dwconv, glu, norm_silu and encode_locked.
 *
 * Conventions, for every entry point:
 *  - Data pointers marked "device" are device memory on the current HIP
 *    device, owned by the caller; they must stay valid until the work
 *    queued on `stream` has finished. Pointers marked "host" are read
 *    before the call returns.
 *  - Row-major layouts, rows = frames or tokens, packed clip after clip.
 *  - Every compute call is asynchronous on `stream` (0 = the null stream)
 *    and allocates no device memory; it validates its arguments first and
 *    returns an error before queuing any work.
 *  - Errors: a non-zero ae_status; ae_last_error() then returns a message
 *    for the calling thread. A failed launch reports AE_ERR_HIP.
 *  - A clip of <= 160 samples has 0 frames and 0 tokens (not an error);
 *    samples past 480000 (30 s at 16 kHz) are ignored.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef AE_H
#define AE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* ae_stream; /* a hipStream_t */

typedef enum {
  AE_OK = 0,
  AE_ERR_INVALID = 1,     /* null pointer, negative size, bad layer index */
  AE_ERR_SHAPE = 2,       /* a weight or size does not fit the configuration */
  AE_ERR_CAPACITY = 3,    /* workspace too small, or an index beyond int32 */
  AE_ERR_UNSUPPORTED = 4, /* a configuration the library does not implement */
  AE_ERR_HIP = 5          /* a HIP runtime call failed */
} ae_status;

/* Arithmetic of the tower. AE_F32: fp32 everywhere (fp32 MFMA for the
 * projections). AE_BF16: bf16 matrices and bf16 projection operands on
 * bf16 MFMA, fp32 accumulation, fp32 residual stream, norms, softmax. */
typedef enum { AE_F32 = 0, AE_BF16 = 1 } ae_dtype;

/* Tower hyper-parameters (the page: AudioTower::load and its defaults). */
typedef struct {
  int32_t hidden;          /* 1024 */
  int32_t heads;           /* 8 (head_dim = hidden / heads = 128) */
  int32_t layers;          /* 12 */
  int32_t ff;              /* 4096, width of the feed-forward */
  int32_t conv_kernel;     /* 5, light-conv depthwise taps */
  int32_t chunk;           /* 12, attention_chunk_size */
  int32_t ctx_left;        /* 13; a token sees ctx_left - 1 = 12 keys */
  int32_t ctx_right;       /* 0; any other value is AE_ERR_UNSUPPORTED */
  float softcap;           /* 50, tanh logit cap */
  float residual_weight;   /* 0.5, feed-forward residual scale */
  int32_t out_hidden;      /* 1536, output_proj width */
  int32_t out_dim;         /* 512, embed_audio width */
} ae_config;

/* Bounds of a clippable projection: the input is clamped to
 * [in_lo, in_hi] before the product and the output to [out_lo, out_hi]
 * after it (the page: ClipLin). +-INFINITY disables a bound. */
typedef struct { float in_lo, in_hi, out_lo, out_hi; } ae_clip;

/* One Conformer layer. Matrices ("mat") are [out][in] row-major in the
 * model's dtype (float or bf16); vectors are float. All device pointers,
 * borrowed: they must outlive the model. y = x W^T throughout. */
typedef struct {
  const float* ff1_pre;  const void* ff1_w1; ae_clip ff1_w1_clip;  /* [ff][hidden] */
  const void* ff1_w2;    ae_clip ff1_w2_clip; const float* ff1_post; /* [hidden][ff] */
  const float* attn_pre;
  const void* q; ae_clip q_clip;          /* [hidden][hidden] each */
  const void* k; ae_clip k_clip;
  const void* v; ae_clip v_clip;
  const void* post; ae_clip post_clip;
  const float* attn_post;
  const float* per_dim_scale;             /* [head_dim] */
  const void* rel_k;                      /* relative_k_proj [hidden][hidden], no clamp */
  const float* lc_pre;
  const void* lc_start; ae_clip lc_start_clip;  /* [2*hidden][hidden] */
  const float* lc_dw;                     /* [hidden][conv_kernel] */
  const float* lc_norm;
  const void* lc_end; ae_clip lc_end_clip;      /* [hidden][hidden] */
  const float* ff2_pre;  const void* ff2_w1; ae_clip ff2_w1_clip;
  const void* ff2_w2;    ae_clip ff2_w2_clip; const float* ff2_post;
  const float* norm_out;
} ae_layer_weights;

/* The whole encoder (device pointers except `layers`, a host array of
 * cfg.layers entries read during ae_model_create). */
typedef struct {
  const float* conv0;      /* [128][1][3][3] */
  const float* ln0;        /* [128] LayerNorm gain */
  const void* conv1;       /* [32][128][3][3], model dtype */
  const float* ln1;        /* [32] */
  const void* in_proj;     /* [hidden][1024], model dtype, no clamp */
  const ae_layer_weights* layers;
  const void* out_proj;    /* [out_hidden][hidden], model dtype */
  const float* out_bias;   /* [out_hidden] */
  const void* embed;       /* [out_dim][out_hidden], model dtype */
} ae_weights;

typedef struct ae_model ae_model; /* opaque */

/* Fill `cfg` with the release's defaults listed in ae_config. */
void ae_config_default(ae_config* cfg);

/* Message of the last error on this thread ("" if none). */
const char* ae_last_error(void);

/* --- sizes (host only; the page: num_frames, num_tokens) ------------- */

/* Log-mel frames of an n-sample clip: 0 if n <= 160, else
 * ceil((n - 160) / 160), after capping n at 480000. */
int64_t ae_num_frames(int64_t n_samples);
/* Soft tokens: ceil(ceil(frames / 2) / 2). */
int64_t ae_num_tokens(int64_t n_samples);

/* Prefix sums of a batch of B clips of n_samples[i] samples (host arrays,
 * each of B + 1 entries written by the call, entry 0 = 0): samples (capped
 * at 480000 per clip), frames, conv0 rows (ceil(frames / 2)) and tokens.
 * Any output may be NULL. Negative lengths are AE_ERR_INVALID. */
ae_status ae_plan(const int64_t* n_samples, int32_t B, int64_t* sample_off,
                  int64_t* frame_off, int64_t* row_off, int64_t* token_off);
/* The same prefix sums from a packed log-mel layout (what ae_subsample
 * receives): frame_off host int64 [B+1], non-decreasing from 0, at most
 * 2999 frames a clip; row_off (conv0 rows, ceil(F/2)) and token_off
 * (ceil(ceil(F/2)/2)) host int64 [B+1] written by the call, either NULL.
 * AE_ERR_INVALID / AE_ERR_SHAPE as ae_subsample refuses the offsets. */
ae_status ae_plan_frames(const int64_t* frame_off, int32_t B, int64_t* row_off,
                         int64_t* token_off);

/* --- model ----------------------------------------------------------- */

/* Validate the configuration and weights and build the derived tables
 * (relative keys R = PE rel_k^T per layer, softplus(per_dim_scale) folded
 * into the query scale, conv1 weights reordered for the implicit GEMM).
 * Allocates those tables (a few MB) on the current device; work is queued
 * on `stream` and finished before return. On error *out is NULL. */
ae_status ae_model_create(const ae_config* cfg, const ae_weights* w, ae_dtype dtype,
                          ae_stream stream, ae_model** out);
void ae_model_destroy(ae_model* m);

/* Per-output-row scales (float32, device, one per row of the matrix) of the
 * ten clippable projections of a layer, for a model with int8 matrices. */
typedef struct {
  const float *ff1_w1, *ff1_w2, *q, *k, *v, *post, *lc_start, *lc_end, *ff2_w1, *ff2_w2;
} ae_layer_scales;

/* A bf16 model whose ten clippable projections per layer (ff1_w1, ff1_w2,
 * q, k, v, post, lc_start, lc_end, ff2_w1, ff2_w2) are int8 [out][in] with
 * a float32 scale per output row (scales: host array of cfg.layers entries,
 * device pointers inside). Every other weight is as for AE_BF16. Each
 * forward widens a layer's int8 matrices to bf16(float32(q) * scale) in the
 * workspace before the layer runs, as the quantised linear layer of the
 * engine.py listing (hugingapi.com multimodalart/scenema-audio, _Int8Linear)
 * dequantises per forward; the layer then computes exactly as a bf16 model
 * holding those matrices. Weights and scales are borrowed (they must
 * outlive the model); calls that share such a model must not overlap in
 * time on one workspace. */
ae_status ae_model_create_q8(const ae_config* cfg, const ae_weights* w,
                             const ae_layer_scales* scales, ae_stream stream, ae_model** out);

/* Workspace bytes needed by ae_subsample / ae_conformer_layer / ae_encode
 * for a batch of B clips with these totals (frames, tokens over the batch). */
size_t ae_workspace_bytes(const ae_model* m, int32_t B, int64_t total_frames,
                          int64_t total_tokens);
/* Workspace bytes needed by ae_logmel for B clips. */
size_t ae_logmel_workspace_bytes(int32_t B);

/* --- compute --------------------------------------------------------- */

/* Log-mel features (the page: module documentation step 2 and
 * MelFrontend::log_mel). wave: device float, the B clips back to back,
 * clip i at [sample_off[i], sample_off[i+1]) (host int64 [B+1],
 * non-decreasing, sample_off[0] = 0). mel: device float [sum F_i][128],
 * clip after clip, F_i = ae_num_frames(length i). Frame j of a clip is
 * the 320 samples starting 160 (j - 1) (zeros before the clip start),
 * times the periodic Hann window, zero-padded to 512, |rFFT| on 257 bins,
 * 128 HTK mel bands over 0..8 kHz, ln(band + 0.001). */
ae_status ae_logmel(const float* wave, const int64_t* sample_off, int32_t B, float* mel,
                    void* ws, size_t ws_bytes, ae_stream stream);

/* Subsampler and input projection (the page: step 3, AudioTower::subsample
 * and input_proj_linear). mel: device float [sum F_i][128] with clip i at
 * rows [frame_off[i], frame_off[i+1]) (host int64 [B+1]). x: device float
 * [sum T_i][hidden], T_i = ceil(F_i / 4). */
ae_status ae_subsample(const ae_model* m, const float* mel, const int64_t* frame_off,
                       int32_t B, float* x, void* ws, size_t ws_bytes, ae_stream stream);

/* One Conformer layer in place (the page: step 4, encode_locked's loop
 * body): FFN1, local attention, light conv, FFN2, RMS norm_out.
 * h: device float [n][hidden]; pos: device int32 [n], each row's index
 * inside its clip (rows of one clip are consecutive, pos 0, 1, 2, ...).
 * The workspace must hold ae_workspace_bytes(m, 1, 0, n). */
ae_status ae_conformer_layer(const ae_model* m, int32_t layer, float* h, const int32_t* pos,
                             int64_t n, void* ws, size_t ws_bytes, ae_stream stream);

/* The whole encoder (the page: soft_tokens / encode_locked): log-mel,
 * subsampler, all layers, then output_proj + bias, a weightless RMS norm
 * and embed_audio. out: device float [sum T_i][out_dim], clip after clip.
 * trace (nullable, host array of cfg.layers + 2 device float pointers, each
 * entry nullable): [0] receives the subsampler output [sum T][hidden],
 * [1 + l] layer l's output [sum T][hidden], [layers + 1] the output
 * projection plus bias [sum T][out_hidden]. */
ae_status ae_encode(const ae_model* m, const float* wave, const int64_t* sample_off,
                    int32_t B, float* out, float* const* trace, void* ws, size_t ws_bytes,
                    ae_stream stream);

/* ae_encode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same computation, kernels and results as ae_encode
 * with trace = NULL; the workspace is instead a static device array of
 * AE_STATIC_SCRATCH_BYTES per device, which libae.so holds from load until
 * the process ends. The model, wave, sample_off and out are as for
 * ae_encode; the current device must be the model's. Allocates nothing: no
 * hipMalloc, hipFree or allocating library call (the first call on a device
 * looks up the array's device address once).
 * Errors: AE_ERR_CAPACITY when the batch needs more than
 * AE_STATIC_SCRATCH_BYTES (what ae_workspace_bytes reports for it; one 30 s
 * clip needs about 35 MB in bf16, 122 MB in f32); AE_ERR_INVALID for a
 * device mismatch or NULL pointers; as ae_encode otherwise.
 * Calls on one device share the array and the last call's contents stay
 * in it; every buffer in it is written before it is read within a call, so
 * nothing needs clearing. Calls that overlap on one device (other streams,
 * other threads) race on it: serialise them. */
#define AE_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
ae_status ae_encode_static(const ae_model* m, const float* wave, const int64_t* sample_off,
                           int32_t B, float* out, ae_stream stream);

/* --- mixdown and resampling to 16 kHz (ahead of ae_logmel) -------------
 * The page: to_mono_16k, resample_hq and the resampler constants. */

/* Samples after resampling n samples from from_rate to to_rate (Hz): n for
 * equal rates, else ceil(to_rate * n / from_rate). -1 for n < 0, a
 * non-positive rate, or a result beyond int64. */
int64_t ae_resampled_length(int64_t n, int32_t from_rate, int32_t to_rate);

typedef struct ae_resampler ae_resampler; /* opaque */

/* Plans band-limited resampling from from_rate to to_rate (each 1..768000
 * Hz) on the current device: with g = gcd, o = from/g, nw = to/g and
 * c = min(1, to/from) * 0.958, output m is
 *   sum over the clip's samples n of x[n] h(n - m from/to),
 *   h(d) = c sinc(c d) I0(12.8 sqrt(1 - (c d / 64)^2)) / I0(12.8), |c d| < 64,
 * (a Kaiser-windowed sinc with 64 zero crossings a side, beta 12.8, cut-off
 * at 0.958 of the lower Nyquist rate), accumulated in float64, rounded to
 * float32. Allocates and fills a device table of the nw phases' taps
 * (float64) with work on `stream`, and waits for it. Equal rates plan a
 * copy. AE_ERR_INVALID for rates out of range, AE_ERR_UNSUPPORTED when the
 * kernel's working set does not fit a CU's LDS or the table would exceed
 * 2^28 entries, AE_ERR_HIP when an allocation fails. */
ae_status ae_resampler_create(int32_t from_rate, int32_t to_rate, ae_stream stream,
                              ae_resampler** out);
/* Frees the table; no work using the resampler may still be queued. */
void ae_resampler_destroy(ae_resampler* r);
/* Plan facts for measurement (each output nullable): the largest tap count
 * of a phase, the nonzero taps summed over the nw phases (the method's
 * multiply-adds per nw outputs), nw and o. */
ae_status ae_resampler_info(const ae_resampler* r, int32_t* taps_per_phase_max,
                            int64_t* nonzero_taps_per_cycle, int32_t* phases,
                            int32_t* in_per_cycle);
/* Workspace bytes for ae_resample (channels = 1) or ae_to_mono_16k with B
 * clips of total_frames input frames. */
size_t ae_resample_workspace_bytes(int32_t B, int64_t total_frames, int32_t channels);

/* Channel mixdown (the page: to_mono_16k): in: device float
 * [n_frames][channels], interleaved; mono: device float [n_frames]; each
 * output is the channel values added in float32 in channel order, divided
 * by `channels` in float32 (one channel is copied). channels >= 1. */
ae_status ae_mixdown(const float* in, int64_t n_frames, int32_t channels, float* mono,
                     ae_stream stream);

/* Resampling of B packed clips (the page: resample_hq): x: device float,
 * clip i at [in_off[i], in_off[i+1]) (host int64 [B+1], in_off[0] = 0,
 * non-decreasing); y: device float, clip after clip, clip i holding
 * ae_resampled_length(length i, from, to) samples. Samples outside a clip
 * are absent from its sums. ws: device workspace of at least
 * ae_resample_workspace_bytes(B, in_off[B], 1) bytes (unused for equal
 * rates); it must be on the resampler's device. */
ae_status ae_resample(const ae_resampler* r, const float* x, const int64_t* in_off, int32_t B,
                      float* y, void* ws, size_t ws_bytes, ae_stream stream);

/* Mixdown then resampling to 16 kHz (the page: to_mono_16k): in: device
 * float, B clips of interleaved frames [frames][channels], clip i at frames
 * [in_off[i], in_off[i+1]); y as ae_resample's output. The resampler must
 * target 16000 Hz. ws: ae_resample_workspace_bytes(B, in_off[B], channels)
 * bytes (the mono signal lives there). */
ae_status ae_to_mono_16k(const ae_resampler* r, const float* in, const int64_t* in_off,
                         int32_t B, int32_t channels, float* y, void* ws, size_t ws_bytes,
                         ae_stream stream);

/* --- soft-token placement (around the encoder) -------------------------
 * The page: input_ids and embed_audio_inputs. */

/* Token ids of the placement: the audio placeholder (<|audio|>, also the id
 * of every soft-token position), the opening and closing audio markers
 * (<|audio>, <audio|>) and the text tokenizer's BOS and EOS. The release
 * uses audio 258881, boa 256000, eoa 258883. */
typedef struct {
  int32_t audio, boa, eoa, bos, eos;
} ae_token_ids;

/* Host-only expansion of one input (the page: input_ids): body (host int32
 * [len], the tokenized text, holding one audio placeholder per clip)
 * becomes [bos] + body + [eos] with placeholder k replaced by
 * [boa] + n_soft[k] x [audio] + [eoa]. out: host int32 [out_cap];
 * *out_len receives the expanded length (also when the call fails for
 * capacity). AE_ERR_SHAPE when the body's placeholder count is not
 * `clips`, AE_ERR_CAPACITY when the result exceeds max_tokens or out_cap. */
ae_status ae_expand_ids(const int32_t* body, int64_t len, const int64_t* n_soft, int32_t clips,
                        const ae_token_ids* tok, int64_t max_tokens, int32_t* out,
                        int64_t out_cap, int64_t* out_len);

/* Workspace bytes for ae_merge_soft_tokens over L ids. */
size_t ae_merge_workspace_bytes(int64_t L);

/* Merge of soft tokens into text embedding rows (the page:
 * embed_audio_inputs): ids: device int32 [L] (expanded sequences, packed);
 * x: device float [L][d], the rows' embeddings, updated in place: the r-th
 * row (in order) whose id equals `audio` receives soft row r, for
 * r < n_soft (soft: device float [n_soft][d], the encoder's output for the
 * clips in the same order). count: device int64 (nullable) receives the
 * number of audio rows; a caller checks it equals n_soft (the page refuses
 * otherwise; rows past n_soft keep their values). d a multiple of 4; x and
 * soft 16-byte aligned. */
ae_status ae_merge_soft_tokens(const int32_t* ids, int64_t L, int32_t audio, const float* soft,
                               int64_t n_soft, int32_t d, float* x, int64_t* count, void* ws,
                               size_t ws_bytes, ae_stream stream);

/* --- measurement ----------------------------------------------------- */

/* Kernel classes the library can time with HIP events recorded on the
 * stream each launch goes to. AE_K_GEMM_FFN1 is the feed-forward's first
 * (widening) projection, AE_K_GEMM_FFN2 its second; AE_K_GEMM_HEAD covers
 * input_proj, output_proj and embed_audio. */
typedef enum {
  AE_K_LOGMEL = 0, AE_K_CONV0 = 1, AE_K_CONV1 = 2, AE_K_GEMM_FFN1 = 3,
  AE_K_GEMM_FFN2 = 4, AE_K_GEMM_QKV = 5, AE_K_GEMM_POST = 6, AE_K_GEMM_LCSTART = 7,
  AE_K_GEMM_LCEND = 8, AE_K_GEMM_HEAD = 9, AE_K_ROWNORM = 10, AE_K_ATTN = 11,
  AE_K_LCONV = 12, AE_K_RESAMPLE = 13, AE_K_MIXDOWN = 14, AE_K_MERGE = 15, AE_K_DEQUANT = 16,
  /* the LFM2A encoder (lfm2a.h): front end (all four kernels), stem
   * convolutions, stem pointwise GEMMs with pre_encode_out, the blocks'
   * feed-forward GEMMs (up, down), attention GEMMs (q|k|v, linear_pos,
   * attn_o), convolution-module GEMMs (pw1, pw2), adapter GEMMs,
   * LayerNorms, attention, depthwise conv */
  AE_K_LFM_FRONT = 17, AE_K_LFM_STEM = 18, AE_K_LFM_GEMM_STEM = 19, AE_K_LFM_GEMM_FFN1 = 20,
  AE_K_LFM_GEMM_FFN2 = 21, AE_K_LFM_GEMM_ATTN = 22, AE_K_LFM_GEMM_CONV = 23,
  AE_K_LFM_GEMM_ADAPTER = 24, AE_K_LFM_LN = 25, AE_K_LFM_ATTN = 26, AE_K_LFM_DWCONV = 27,
  AE_K_COUNT = 28
} ae_kernel_class;

/* Process-wide: from now on, bracket every launch of kernel class `cls`
 * with a pair of HIP events (up to 4096 launches are kept until read);
 * cls = -1 turns timing off. Not for concurrent use from several threads.
 * Unknown classes are AE_ERR_INVALID. */
ae_status ae_timing_enable(int32_t cls);
/* Wait for the recorded events, return the number of timed launches and
 * their summed duration in milliseconds, and clear the record. */
ae_status ae_timing_read(int64_t* launches, double* total_ms);

/* Matrix-core rate probe, a measurement aid beside the timing facility:
 * launches on stream s one kernel whose wavefronts (four 4-wavefront blocks
 * per CU) each run `iters` rounds of eight independent bf16 32x32x16
 * matrix instructions on register operands, with no memory traffic, and
 * stores in *flops (host) the floating-point operations it performs; the
 * caller times it (HIP events on s) for the device's sustained bf16 matrix
 * rate. sink: device float, written only in a case that does not arise
 * (it keeps the products live). iters < 1 or a null pointer:
 * AE_ERR_INVALID. */
ae_status ae_probe_mfma(int32_t iters, float* sink, int64_t* flops, hipStream_t s);

#ifdef __cplusplus
}
#endif
#endif /* AE_H */
