// Internal launchers: one per kernel family. Each returns hipSuccess or the
// launch error; shapes are validated by the caller (the C-ABI layer).
#pragma once

#include "common.h"

namespace ae {

// ----------------------------------------------------------------- GEMM
// C = epilogue(A B^T): A [M][K], B [N][K] row-major, fp32 accumulation.
enum EpiKind {
  EPI_STORE = 0,   // C = clamp(acc, olo, ohi) * colscale[col]       (TO)
  EPI_SILU = 1,    // C = clamp(silu(clamp(acc, olo, ohi)), nlo, nhi) (TO)
  EPI_GLU = 2,     // C[:, j] = a * sigmoid(b), a/b the clamped halves (TO)
  EPI_RESID = 3,   // C (float) += clamp(acc, olo, ohi)
  EPI_BIAS = 4,    // C (float) = acc + bias[col]
  EPI_LNRELU = 5,  // C = relu(LayerNorm_32(acc) * gain)  (conv1, N = 32)
  EPI_ACT = 6      // C = act(acc + bias[col]) (TO), bias optional
};
// Activations of EPI_ACT. EPI_GLU and EPI_RESID also add bias[col] when
// bias is set (GLU: bias[c] to a, bias[glu_d + c] to b), and EPI_RESID
// scales what it adds by rscale.
enum ActKind { ACT_NONE = 0, ACT_RELU = 1, ACT_SILU = 2, ACT_GELU_ERF = 3 };
enum ALoadKind { A_PLAIN = 0, A_CONV1 = 1 };

struct GemmParams {
  int M, N, K;
  // A: plain row-major, one pointer per B segment (qkv may clamp apart)
  const void* A[3];
  int lda;
  // A_CONV1: implicit im2col over conv0 rows y0 [rows][64][128]
  const void* y0;
  const int64_t* row_off;   // conv0 row offsets per clip [B+1]
  const int32_t* tok_pos;   // token -> index in clip
  const int32_t* tok_clip;  // token -> clip
  int n_tok;
  // B: up to 3 row segments of seg_n rows (N = sum), leading dim ldb
  const void* Bm[3];
  int seg_n, ldb;
  int glu_d;                // EPI_GLU: output width; B rows [0,d) = a, [d,2d) = b
  // epilogue
  void* C;
  int ldc;
  float olo[3], ohi[3];
  float nlo, nhi;
  const float* colscale;
  const float* bias;
  const float* gain;
  int act;                  // EPI_ACT: an ActKind
  float rscale;             // EPI_RESID: C += rscale * (acc + bias)
  // float operands: a workspace area for the partial tiles of a K split,
  // at least gemm_f32_part_bytes(M, N, K) bytes; splits is the dispatcher's
  float* part;
  size_t part_bytes;
  int splits;
};

// dtype: AE_F32 or AE_BF16 operands; out_bf16: TO = bf16 (else float).
hipError_t launch_gemm(ae_dtype dt, int epi, int aload, bool out_bf16, const GemmParams& p,
                       hipStream_t s);
// Bytes of the K-split area a float GEMM of this shape needs (0: it runs
// in one pass). The split count follows K alone.
size_t gemm_f32_part_bytes(int64_t M, int N, int K);

// -------------------------------------------------------------- front end
hipError_t mel_tables_init();
hipError_t launch_logmel(const float* wave, const int64_t* sample_off, const int64_t* frame_off,
                         int B, int64_t total_frames, float* mel, hipStream_t s);

// --------------------------------------------------------------- conv0
// float storage only (bf16 models run launch_subsample_fused); the packed
// fragments of the centred taps (8 KB) are the fused subsampler's.
hipError_t launch_conv0(ae_dtype dt, const float* mel, const int64_t* frame_off,
                        const int64_t* row_off, int B, int64_t total_rows, const float* w0,
                        const float* g0, void* y0, hipStream_t s);
constexpr size_t kConv0FragBytes = 4 * 2 * 64 * 16;
hipError_t launch_conv0_pack(const float* w0, void* frag, hipStream_t s);

// ------------------------------------------------- subsampler, bf16 models
// conv0 and conv1 (with their LayerNorms and ReLUs) in one pass, the conv0
// plane kept in LDS: mel [frames][128] float, the per-clip frame and conv0
// row offsets, each token's position and clip, the packed conv0 taps
// (launch_conv0_pack), g0 [128], w1 conv1's weights [32][9 * 128] bf16,
// g1 [32]; x1 [n_tok][32 * 32] bf16, [frequency][channel] per token.
hipError_t launch_subsample_fused(const float* mel, const int64_t* frame_off,
                                  const int64_t* row_off, const int32_t* tok_pos,
                                  const int32_t* tok_clip, int64_t n_tok, const void* w0_frag,
                                  const float* g0, const void* w1, const float* g1, void* x1,
                                  hipStream_t s);

// -------------------------------------------------------------- row norms
// For each row of h [n][d] (float):
//   if y:     h += scale * rms(y) * w_post   (y [n][d] in dtype dt), or
//             h += scale * y when w_post is null
//   if w_out: h  = rms(h) * w_out
//   store h (when y or w_out was applied); if h_copy: also h as dtype dt
//   if w_next: a_i = clamp(rms(h) * w_next, lo_i, hi_i) for i < n_out (dtype dt)
// With w_next = nullptr and h_in_place false, nothing but the a_i are written.
struct RowNormParams {
  int64_t n;
  int d;
  float* h;
  // an earlier residual update whose h the previous launch left unwritten:
  // applied first, the same way as the one below (a post-norm with w_post0,
  // or a plain add when it is null)
  const void* y0;
  float scale0;
  const float* w_post0;
  bool skip_h;           // leave h unwritten (the next launch recomputes it)
  const void* y;
  float scale;
  const float* w_post;
  const float* w_out;
  const float* w_next;   // may be null: then a weightless norm if out_plain
  bool plain_next;       // weightless rms for a_i (head)
  void* a[3];
  float lo[3], hi[3];
  int n_out;
  void* h_copy;          // if set: the final h also stored here in dtype dt
};
hipError_t launch_rownorm(ae_dtype dt, const RowNormParams& p, hipStream_t s);

// ------------------------------------------------------------- attention
// qkv [n][3d] (dtype dt; q, k already scaled), R [left][d] float,
// pos [n] -> o [n][d] (dtype dt) clamped to [lo, hi].
hipError_t launch_attention(ae_dtype dt, const void* qkv, const void* R, const int32_t* pos,
                            int64_t n, int d, int heads, int left, float softcap, float lo,
                            float hi, void* o, hipStream_t s);

// ------------------------------------------------------------ light conv
// u [n][d] (dt) -> c = clamp(silu(rms(dwconv(u)) * w_norm), lo, hi) (dt);
// w_dwt: the depthwise taps transposed, [kernel][d].
hipError_t launch_lconv(ae_dtype dt, const void* u, const float* w_dwt, int kernel,
                        const float* w_norm, const int32_t* pos, int64_t n, int d, float lo,
                        float hi, void* c, hipStream_t s);

// ---------------------------------------------------------- bookkeeping
// Write the packed-offset table (host values passed by value) to `dst`.
hipError_t launch_write_i64(int64_t* dst, const int64_t* host_vals, int count, hipStream_t s);
// tok_pos / tok_clip from token_off [B+1] (device).
hipError_t launch_token_index(const int64_t* token_off, int B, int64_t n_tok, int32_t* tok_pos,
                              int32_t* tok_clip, hipStream_t s);
// Model tables: R = PE rel_k^T ([n_dist][d] float), colscale for q|k|v,
// conv1 weights reordered to [32][(dt*3+df)*128 + ci].
hipError_t launch_relative_keys(ae_dtype dt, const void* rel_k, int d, int n_dist, void* R,
                                hipStream_t s);
hipError_t launch_qkv_scale(const float* pds, int d, int head_dim, float q_scale, float k_scale,
                            float* colscale, hipStream_t s);
hipError_t launch_conv1_reorder(ae_dtype dt, const void* w1, void* w1r, hipStream_t s);
// [d][K] -> [K][d]
hipError_t launch_transpose_taps(const float* w, int d, int K, float* wt, hipStream_t s);

}  // namespace ae
