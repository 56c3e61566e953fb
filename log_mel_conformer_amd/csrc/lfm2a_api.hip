// C ABI of the LFM2A encoder (include/lfm2a.h): sizes, model tables,
// workspace layout and the forward pass in the order of the page
// (cera 0.5.3, audio_encoder_gpu.rs: encode_audio_pcm_gpu ->
// log_mel_spectrogram_gpu -> conv_stem_gpu -> encode_audio_gpu).
//
// The residual stream x is float32 [tokens][512]; every projection runs on
// the bf16 GEMM with its bias, activation or residual add fused into the
// epilogue (SiLU for the feed-forward, the half-weight residual of
// macaron_ffn, GLU with bias for pw1, ReLU for the pointwise stem layers,
// erf GELU for the adapter). Each block's closing LayerNorm is fused with
// the LayerNorm that opens the next block (or the adapter).
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "lfm2a_launch.h"

using namespace ae;
using namespace ae::lfm;

struct lfm2a_model {
  lfm2a_config cfg;
  lfm2a_weights w;
  std::vector<lfm2a_block_weights> blocks;
  int device = 0;
  void* alloc = nullptr;
  bf16* stem_pw[2] = {nullptr, nullptr};    // stem layers 2 and 4, [256][256] bf16
  float* stem_dwt[2] = {nullptr, nullptr};  // stem layers 1 and 3, taps [9][256]
  bf16* pre_w = nullptr;                    // pre_encode_out, columns in (freq, channel) order
  float* qkv_b = nullptr;                   // [n_layer][3 * 512]
  float* dw_t = nullptr;                    // conv-module taps transposed, [n_layer][k][512]
};

namespace {

#define LFM_LAUNCH(cls, stream, expr)                                                  \
  do {                                                                                 \
    timing_begin((cls), (stream));                                                     \
    hipError_t e_ = (expr);                                                            \
    timing_end((cls), (stream));                                                       \
    if (e_ != hipSuccess)                                                              \
      return set_error(AE_ERR_HIP, std::string("launch failed: ") + #expr + ": " +     \
                                       hipGetErrorString(e_));                         \
  } while (0)

constexpr int kFeat = kStemCh * kF3;  // 4096, pre_encode_out input width

size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }
int64_t half_up(int64_t h) { return h > 0 ? (h - 1) / 2 + 1 : 0; }
int64_t frames_of(int64_t n) { return n <= 0 ? 0 : 1 + n / lfm::kHop; }

GemmParams gp(int M, int N, int K, const void* A, const void* Bw, void* C) {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.M = M; p.N = N; p.K = K;
  p.A[0] = p.A[1] = p.A[2] = A;
  p.lda = K;
  p.Bm[0] = p.Bm[1] = p.Bm[2] = Bw;
  p.seg_n = N;
  p.ldb = K;
  p.C = C;
  p.ldc = N;
  for (int i = 0; i < 3; ++i) { p.olo[i] = -INFINITY; p.ohi[i] = INFINITY; }
  p.nlo = -INFINITY; p.nhi = INFINITY;
  p.rscale = 1.0f;
  return p;
}

// Per-batch geometry: offsets of samples, frames, stem rows after the first
// and second stride-2 layers, tokens, and attention query tiles.
struct Geometry {
  int B = 0;
  std::vector<int64_t> so, fo, r1, r2, to, qt;
  int64_t max_t = 0;
  int64_t F() const { return fo[B]; }
  int64_t R1() const { return r1[B]; }
  int64_t R2() const { return r2[B]; }
  int64_t T() const { return to[B]; }
  int64_t QT() const { return qt[B]; }
  void from_frames(const std::vector<int64_t>& fr) {
    B = (int)fr.size();
    fo.assign(B + 1, 0); r1.assign(B + 1, 0); r2.assign(B + 1, 0); to.assign(B + 1, 0);
    qt.assign(B + 1, 0);
    max_t = 0;
    for (int i = 0; i < B; ++i) {
      const int64_t a = half_up(fr[i]), b = half_up(a), t = half_up(b);
      fo[i + 1] = fo[i] + fr[i];
      r1[i + 1] = r1[i] + a;
      r2[i + 1] = r2[i] + b;
      to[i + 1] = to[i] + t;
      qt[i + 1] = qt[i] + (t + kQueriesPerBlock - 1) / kQueriesPerBlock;
      max_t = std::max(max_t, t);
    }
  }
};

// Workspace: the offset tables and token indexes, the front end's
// buffers, the residual stream, then one region shared by the stem's
// planes and the blocks' activations (the stem is done before a block
// starts).
struct Layout {
  size_t tabs, tok_pos, tok_clip, mel, part, stats, x, region;
  size_t y1, y2, pe, P, a, qkv, o, g, c, u;
  size_t total;
  Layout(int B, int64_t F, int64_t R1, int64_t R2, int64_t T, int64_t max_t) {
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t at = off; off += al256(bytes); return at; };
    tabs = take(sizeof(int64_t) * 6 * (size_t)(B + 1));
    tok_pos = take(sizeof(int32_t) * (size_t)T);
    tok_clip = take(sizeof(int32_t) * (size_t)T);
    mel = take(sizeof(float) * kMel * (size_t)F);
    part = take(sizeof(double) * 2 * kMel * kStatSlices * (size_t)B);
    stats = take(sizeof(float) * 2 * kMel * (size_t)B);
    x = take(sizeof(float) * kD * (size_t)T);
    region = off;
    const size_t stem_y1 = al256(2 * (size_t)kStemCh * lfm::kF1 * R1);
    const size_t stem_y3 = al256(2 * (size_t)kStemCh * lfm::kF2 * R2);
    const size_t stem_y5 = al256(2 * (size_t)kFeat * T);
    y1 = region;
    y2 = region + std::max(std::max(stem_y1, stem_y3), stem_y5);
    const size_t stem_end = y2 + al256(2 * (size_t)kStemCh * lfm::kF2 * R2);
    off = region;
    const int64_t prow = max_t > 0 ? 2 * max_t - 1 : 0;
    pe = take(2 * (size_t)kD * prow);
    P = take(2 * (size_t)kD * prow);
    a = take(2 * (size_t)kD * T);
    qkv = take(2 * (size_t)3 * kD * T);
    o = take(2 * (size_t)kD * T);
    g = take(2 * (size_t)kD * T);
    c = take(2 * (size_t)kD * T);
    u = take(2 * (size_t)2048 * T);
    total = std::max(off, stem_end) + 256;
  }
};

struct Bufs {
  char* base;
  int64_t *so, *fo, *r1, *r2, *to, *qt;
  int32_t *tok_pos, *tok_clip;
  float *mel, *stats, *x;
  double* part;
  bf16 *y1, *y2, *pe, *P, *a, *qkv, *o, *g, *c, *u;
  Bufs(void* ws, const Layout& L, int B) {
    base = (char*)ws;
    int64_t* t = (int64_t*)(base + L.tabs);
    so = t; fo = t + (B + 1); r1 = t + 2 * (B + 1); r2 = t + 3 * (B + 1); to = t + 4 * (B + 1);
    qt = t + 5 * (B + 1);
    tok_pos = (int32_t*)(base + L.tok_pos);
    tok_clip = (int32_t*)(base + L.tok_clip);
    mel = (float*)(base + L.mel);
    part = (double*)(base + L.part);
    stats = (float*)(base + L.stats);
    x = (float*)(base + L.x);
    y1 = (bf16*)(base + L.y1); y2 = (bf16*)(base + L.y2);
    pe = (bf16*)(base + L.pe); P = (bf16*)(base + L.P); a = (bf16*)(base + L.a);
    qkv = (bf16*)(base + L.qkv); o = (bf16*)(base + L.o); g = (bf16*)(base + L.g);
    c = (bf16*)(base + L.c); u = (bf16*)(base + L.u);
  }
};

ae_status upload_tables(const Geometry& G, const Bufs& b, bool tokens, hipStream_t s) {
  std::vector<int64_t> all;
  const std::vector<int64_t>* parts[6] = {&G.so, &G.fo, &G.r1, &G.r2, &G.to, &G.qt};
  for (auto* p : parts) {
    if ((int)p->size() == G.B + 1) all.insert(all.end(), p->begin(), p->end());
    else all.insert(all.end(), (size_t)G.B + 1, 0);
  }
  AE_HIP_TRY(launch_write_i64(b.so, all.data(), (int)all.size(), s));
  if (tokens) AE_HIP_TRY(launch_token_index(b.to, G.B, G.T(), b.tok_pos, b.tok_clip, s));
  return AE_OK;
}

bool is_default(const lfm2a_config& c) {
  return c.n_mel == kMel && c.stem_ch == kStemCh && c.n_embd == kD && c.n_head == kHeads &&
         c.n_ff == 2048 && c.n_layer > 0 && c.conv_kernel == kKern && c.pos_dim == kD &&
         c.adapter == 2048 && c.llm_hidden == 2048 && c.eps > 0.f;
}

ae_status check_offsets(const int64_t* off, int32_t B, const char* what) {
  if (!off || B < 0) return set_error(AE_ERR_INVALID, std::string(what) + ": null offsets or B < 0");
  if (off[0] != 0) return set_error(AE_ERR_INVALID, std::string(what) + ": offsets must start at 0");
  for (int i = 0; i < B; ++i)
    if (off[i + 1] < off[i])
      return set_error(AE_ERR_INVALID, std::string(what) + ": offsets must be non-decreasing");
  return AE_OK;
}

// ------------------------------------------------------------- stages
ae_status run_front(const float* wave, const Geometry& G, const Bufs& b, float* feat,
                    hipStream_t s) {
  AE_HIP_TRY(frontend_init());
  LFM_LAUNCH(AE_K_LFM_FRONT, s, launch_logmel_raw(wave, b.so, b.fo, G.B, G.F(), feat, s));
  LFM_LAUNCH(AE_K_LFM_FRONT, s, launch_mel_stats(feat, b.so, b.fo, G.B, b.part, b.stats, s));
  LFM_LAUNCH(AE_K_LFM_FRONT, s, launch_mel_norm(feat, b.so, b.fo, G.B, G.F(), b.stats, s));
  return AE_OK;
}

ae_status run_stem(const lfm2a_model* m, const float* feat, const Geometry& G, const Bufs& b,
                   float* x, hipStream_t s) {
  const lfm2a_weights& w = m->w;
  LFM_LAUNCH(AE_K_LFM_STEM, s, launch_stem01(feat, b.fo, b.r1, b.r2, G.B, G.R2(), w.stem_w[0],
                                             w.stem_b[0], m->stem_dwt[0], w.stem_b[1], b.y2, s));
  {  // pointwise layer 2 + ReLU: y2 -> y3 (in y1's place)
    GemmParams p = gp((int)(G.R2() * lfm::kF2), kStemCh, kStemCh, b.y2, m->stem_pw[0], b.y1);
    p.bias = w.stem_b[2];
    p.act = ACT_RELU;
    LFM_LAUNCH(AE_K_LFM_GEMM_STEM, s, launch_gemm(AE_BF16, EPI_ACT, A_PLAIN, true, p, s));
  }
  LFM_LAUNCH(AE_K_LFM_STEM, s, launch_dw3s2(b.y1, b.r2, b.to, G.B, G.T(), lfm::kF2, m->stem_dwt[1],
                                            w.stem_b[3], b.y2, s));
  {  // pointwise layer 4 + ReLU: y4 -> y5 [T][16 * 256] (in y1's place)
    GemmParams p = gp((int)(G.T() * kF3), kStemCh, kStemCh, b.y2, m->stem_pw[1], b.y1);
    p.bias = w.stem_b[4];
    p.act = ACT_RELU;
    LFM_LAUNCH(AE_K_LFM_GEMM_STEM, s, launch_gemm(AE_BF16, EPI_ACT, A_PLAIN, true, p, s));
  }
  {
    GemmParams p = gp((int)G.T(), kD, kFeat, b.y1, m->pre_w, x);
    p.bias = w.pre_encode_out_b;
    LFM_LAUNCH(AE_K_LFM_GEMM_STEM, s, launch_gemm(AE_BF16, EPI_BIAS, A_PLAIN, false, p, s));
  }
  return AE_OK;
}

ae_status run_ln(float* x, int64_t n, const float* w1, const float* b1, bool write_x,
                 const float* w2, const float* b2, bf16* a, float eps, hipStream_t s) {
  LnParams p;
  p.n = n; p.x = x; p.w1 = w1; p.b1 = b1; p.write_x = write_x; p.w2 = w2; p.b2 = b2; p.a = a;
  p.eps = eps;
  LFM_LAUNCH(AE_K_LFM_LN, s, launch_layernorm(p, s));
  return AE_OK;
}

// x += 0.5 (SiLU(a W_up^T + b_up) W_down^T + b_down), a = LN(x) already
ae_status run_ffn(const lfm2a_model* m, const void* up_w, const float* up_b, const void* down_w,
                  const float* down_b, const Bufs& b, float* x, int64_t T, hipStream_t s) {
  const int ff = m->cfg.n_ff;
  GemmParams p1 = gp((int)T, ff, kD, b.a, up_w, b.u);
  p1.bias = up_b;
  p1.act = ACT_SILU;
  LFM_LAUNCH(AE_K_LFM_GEMM_FFN1, s, launch_gemm(AE_BF16, EPI_ACT, A_PLAIN, true, p1, s));
  GemmParams p2 = gp((int)T, kD, ff, b.u, down_w, x);
  p2.bias = down_b;
  p2.rscale = 0.5f;
  LFM_LAUNCH(AE_K_LFM_GEMM_FFN2, s, launch_gemm(AE_BF16, EPI_RESID, A_PLAIN, false, p2, s));
  return AE_OK;
}

// One block; on entry b.a holds LN(x; ffn_norm). On exit x = LN(x; ln2)
// and, if next_w is set, b.a = LN(x; next_w, next_b).
ae_status run_block(const lfm2a_model* m, int layer, const Geometry& G, const Bufs& b, float* x,
                    const float* next_w, const float* next_b, hipStream_t s) {
  const lfm2a_block_weights& L = m->blocks[layer];
  const int64_t T = G.T();
  const float eps = m->cfg.eps;
  if (ae_status st = run_ffn(m, L.ffn_up_w, L.ffn_up_b, L.ffn_down_w, L.ffn_down_b, b, x, T, s))
    return st;
  if (ae_status st = run_ln(x, T, L.ln1_w, L.ln1_b, false, nullptr, nullptr, b.a, eps, s)) return st;
  {
    GemmParams p = gp((int)T, 3 * kD, kD, b.a, L.attn_q_w, b.qkv);
    p.Bm[1] = L.attn_k_w;
    p.Bm[2] = L.attn_v_w;
    p.seg_n = kD;
    p.bias = m->qkv_b + (size_t)layer * 3 * kD;
    p.act = ACT_NONE;
    LFM_LAUNCH(AE_K_LFM_GEMM_ATTN, s, launch_gemm(AE_BF16, EPI_ACT, A_PLAIN, true, p, s));
  }
  {
    GemmParams p = gp((int)(2 * G.max_t - 1), kD, kD, b.pe, L.linear_pos_w, b.P);
    p.act = ACT_NONE;
    LFM_LAUNCH(AE_K_LFM_GEMM_ATTN, s, launch_gemm(AE_BF16, EPI_ACT, A_PLAIN, true, p, s));
  }
  LFM_LAUNCH(AE_K_LFM_ATTN, s, launch_xl_attention(b.qkv, b.P, G.max_t, L.pos_bias_u,
                                                    L.pos_bias_v, b.to, b.qt, G.B, G.QT(), b.o,
                                                    s));
  {
    GemmParams p = gp((int)T, kD, kD, b.o, L.attn_o_w, x);
    p.bias = L.attn_o_b;
    LFM_LAUNCH(AE_K_LFM_GEMM_ATTN, s, launch_gemm(AE_BF16, EPI_RESID, A_PLAIN, false, p, s));
  }
  if (ae_status st = run_ln(x, T, L.norm_conv_w, L.norm_conv_b, false, nullptr, nullptr, b.a, eps,
                            s))
    return st;
  {
    GemmParams p = gp((int)T, 2 * kD, kD, b.a, L.conv_pw1_w, b.g);
    p.ldc = kD;
    p.glu_d = kD;
    p.bias = L.conv_pw1_b;
    LFM_LAUNCH(AE_K_LFM_GEMM_CONV, s, launch_gemm(AE_BF16, EPI_GLU, A_PLAIN, true, p, s));
  }
  LFM_LAUNCH(AE_K_LFM_DWCONV, s, launch_dwconv(b.g, b.tok_pos, b.tok_clip, b.to, T,
                                               m->dw_t + (size_t)layer * m->cfg.conv_kernel * kD,
                                               m->cfg.conv_kernel, L.conv_dw_b, L.conv_norm_w,
                                               L.conv_norm_b, b.c, s));
  {
    GemmParams p = gp((int)T, kD, kD, b.c, L.conv_pw2_w, x);
    p.bias = L.conv_pw2_b;
    LFM_LAUNCH(AE_K_LFM_GEMM_CONV, s, launch_gemm(AE_BF16, EPI_RESID, A_PLAIN, false, p, s));
  }
  if (ae_status st = run_ln(x, T, L.ffn_norm_1_w, L.ffn_norm_1_b, false, nullptr, nullptr, b.a,
                            eps, s))
    return st;
  if (ae_status st = run_ffn(m, L.ffn_up_1_w, L.ffn_up_1_b, L.ffn_down_1_w, L.ffn_down_1_b, b, x,
                             T, s))
    return st;
  return run_ln(x, T, L.ln2_w, L.ln2_b, true, next_w, next_b, next_w ? b.a : nullptr, eps, s);
}

// adapter from b.a = LN(x; adapter_norm)
ae_status run_adapter(const lfm2a_model* m, const Bufs& b, int64_t T, float* out, hipStream_t s) {
  const lfm2a_weights& w = m->w;
  GemmParams p1 = gp((int)T, m->cfg.adapter, kD, b.a, w.adapter_up_w, b.u);
  p1.bias = w.adapter_up_b;
  p1.act = ACT_GELU_ERF;
  LFM_LAUNCH(AE_K_LFM_GEMM_ADAPTER, s, launch_gemm(AE_BF16, EPI_ACT, A_PLAIN, true, p1, s));
  GemmParams p2 = gp((int)T, m->cfg.llm_hidden, m->cfg.adapter, b.u, w.adapter_down_w, out);
  p2.bias = w.adapter_down_b;
  LFM_LAUNCH(AE_K_LFM_GEMM_ADAPTER, s, launch_gemm(AE_BF16, EPI_BIAS, A_PLAIN, false, p2, s));
  return AE_OK;
}

ae_status check_ws(const lfm2a_model* m, void* ws, size_t ws_bytes, size_t need,
                   const char* what) {
  if (!m) return set_error(AE_ERR_INVALID, std::string(what) + ": null model");
  if (!ws || ws_bytes < need)
    return set_error(AE_ERR_CAPACITY,
                     std::string(what) + ": workspace needs " + std::to_string(need) + " bytes");
  if ((uintptr_t)ws & 255)
    return set_error(AE_ERR_INVALID, std::string(what) + ": workspace must be 256-byte aligned");
  return AE_OK;
}

bool int_range(int64_t v) { return v >= 0 && v <= (int64_t)INT32_MAX / 16; }

}  // namespace

extern "C" {

void lfm2a_config_default(lfm2a_config* c) {
  if (!c) return;
  c->n_mel = kMel;
  c->stem_ch = kStemCh;
  c->n_embd = kD;
  c->n_head = kHeads;
  c->n_ff = 2048;
  c->n_layer = 17;
  c->conv_kernel = kKern;
  c->pos_dim = kD;
  c->adapter = 2048;
  c->llm_hidden = 2048;
  c->eps = 1e-5f;
}

int64_t lfm2a_num_frames(int64_t n) { return frames_of(n); }

int64_t lfm2a_num_tokens(int64_t n) { return half_up(half_up(half_up(frames_of(n)))); }

ae_status lfm2a_plan(const int64_t* n_samples, int32_t B, int64_t* sample_off,
                     int64_t* frame_off, int64_t* token_off) {
  if (B < 0 || (B > 0 && !n_samples)) return set_error(AE_ERR_INVALID, "lfm2a_plan: bad batch");
  int64_t s = 0, f = 0, t = 0;
  if (sample_off) sample_off[0] = 0;
  if (frame_off) frame_off[0] = 0;
  if (token_off) token_off[0] = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t n = n_samples[i];
    if (n < 0) return set_error(AE_ERR_INVALID, "lfm2a_plan: negative clip length");
    if (n > 0 && n < 2 * lfm::kHop)
      return set_error(AE_ERR_SHAPE, "lfm2a_plan: clip " + std::to_string(i) + " has " +
                                         std::to_string(n) +
                                         " samples, fewer than two statistics frames");
    s += n;
    f += frames_of(n);
    t += lfm2a_num_tokens(n);
    if (sample_off) sample_off[i + 1] = s;
    if (frame_off) frame_off[i + 1] = f;
    if (token_off) token_off[i + 1] = t;
  }
  return AE_OK;
}

ae_status lfm2a_plan_frames(const int64_t* frame_off, int32_t B, int64_t* token_off) {
  if (B < 0 || (B > 0 && !frame_off)) return set_error(AE_ERR_INVALID, "lfm2a_plan_frames: bad batch");
  if (B > 0 && frame_off[0] != 0) return set_error(AE_ERR_INVALID, "lfm2a_plan_frames: frame_off[0] != 0");
  int64_t t = 0;
  if (token_off) token_off[0] = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t F = frame_off[i + 1] - frame_off[i];
    if (F < 0) return set_error(AE_ERR_INVALID, "lfm2a_plan_frames: frame_off must be non-decreasing");
    t += half_up(half_up(half_up(F)));
    if (token_off) token_off[i + 1] = t;
  }
  return AE_OK;
}

size_t lfm2a_logmel_workspace_bytes(int32_t B) {
  if (B < 0) return 0;
  return Layout(B, 0, 0, 0, 0, 0).total;
}

ae_status lfm2a_logmel(const float* wave, const int64_t* sample_off, int32_t B, float* feat,
                       void* ws, size_t ws_bytes, ae_stream stream) {
  if (ae_status st = check_offsets(sample_off, B, "lfm2a_logmel")) return st;
  std::vector<int64_t> n(B), fr(B);
  for (int i = 0; i < B; ++i) n[i] = sample_off[i + 1] - sample_off[i];
  if (ae_status st = lfm2a_plan(n.data(), B, nullptr, nullptr, nullptr)) return st;
  for (int i = 0; i < B; ++i) fr[i] = frames_of(n[i]);
  Geometry G;
  G.from_frames(fr);
  G.so.assign(sample_off, sample_off + B + 1);
  if (G.F() == 0) return AE_OK;
  if (!wave || !feat) return set_error(AE_ERR_INVALID, "lfm2a_logmel: null pointer");
  const Layout L(B, 0, 0, 0, 0, 0);
  if (!ws || ws_bytes < L.total)
    return set_error(AE_ERR_CAPACITY,
                     "lfm2a_logmel: workspace needs " + std::to_string(L.total) + " bytes");
  if ((uintptr_t)ws & 255)
    return set_error(AE_ERR_INVALID, "lfm2a_logmel: workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  Bufs b(ws, L, B);
  if (ae_status st = upload_tables(G, b, false, s)) return st;
  return run_front(wave, G, b, feat, s);
}

ae_status lfm2a_model_create(const lfm2a_config* cfg, const lfm2a_weights* w, ae_dtype dtype,
                             ae_stream stream, lfm2a_model** out) {
  if (out) *out = nullptr;
  if (!cfg || !w || !out) return set_error(AE_ERR_INVALID, "lfm2a_model_create: null argument");
  if (!is_default(*cfg))
    return set_error(AE_ERR_UNSUPPORTED,
                     "lfm2a_model_create: only the default widths (128 mel, 256 stem channels, "
                     "512 / 8 heads, 2048 feed-forward, kernel 9, adapter 2048 -> 2048) are "
                     "implemented");
  if (dtype != AE_BF16)
    return set_error(AE_ERR_UNSUPPORTED, "lfm2a_model_create: only AE_BF16 is implemented");
  // every device pointer non-null and 16-byte aligned (the kernels read
  // weights and biases with 16-byte loads)
  auto bad = [](const void* p) { return !p || ((uintptr_t)p & 15) != 0; };
  for (int i = 0; i < 5; ++i)
    if (bad(w->stem_w[i]) || bad(w->stem_b[i]))
      return set_error(AE_ERR_INVALID, "lfm2a_model_create: stem weight NULL or not 16-byte aligned");
  if (!w->blocks)
    return set_error(AE_ERR_INVALID, "lfm2a_model_create: null blocks");
  if (bad(w->pre_encode_out_w) || bad(w->pre_encode_out_b) || bad(w->adapter_norm_w) ||
      bad(w->adapter_norm_b) || bad(w->adapter_up_w) || bad(w->adapter_up_b) ||
      bad(w->adapter_down_w) || bad(w->adapter_down_b))
    return set_error(AE_ERR_INVALID, "lfm2a_model_create: weight NULL or not 16-byte aligned");
  for (int l = 0; l < cfg->n_layer; ++l) {
    const lfm2a_block_weights& L = w->blocks[l];
    const void* ptrs[] = {L.ffn_norm_w, L.ffn_norm_b, L.ffn_up_w, L.ffn_up_b, L.ffn_down_w,
                          L.ffn_down_b, L.ln1_w, L.ln1_b, L.attn_q_w, L.attn_q_b, L.attn_k_w,
                          L.attn_k_b, L.attn_v_w, L.attn_v_b, L.attn_o_w, L.attn_o_b,
                          L.pos_bias_u, L.pos_bias_v, L.linear_pos_w, L.norm_conv_w,
                          L.norm_conv_b, L.conv_pw1_w, L.conv_pw1_b, L.conv_dw_w, L.conv_dw_b,
                          L.conv_norm_w, L.conv_norm_b, L.conv_pw2_w, L.conv_pw2_b,
                          L.ffn_norm_1_w, L.ffn_norm_1_b, L.ffn_up_1_w, L.ffn_up_1_b,
                          L.ffn_down_1_w, L.ffn_down_1_b, L.ln2_w, L.ln2_b};
    for (const void* p : ptrs)
      if (bad(p))
        return set_error(AE_ERR_INVALID, "lfm2a_model_create: block " + std::to_string(l) +
                                             " has a weight NULL or not 16-byte aligned");
  }
  lfm2a_model* m = new lfm2a_model();
  m->cfg = *cfg;
  m->w = *w;
  m->blocks.assign(w->blocks, w->blocks + cfg->n_layer);
  m->w.blocks = nullptr;
  hipStream_t s = (hipStream_t)stream;
  auto fail = [&](ae_status st) {
    if (m->alloc) (void)hipFree(m->alloc);
    delete m;
    return st;
  };
  if (hipGetDevice(&m->device) != hipSuccess)
    return fail(set_error(AE_ERR_HIP, "lfm2a_model_create: hipGetDevice failed"));
  const size_t pw_bytes = al256(2 * (size_t)kStemCh * kStemCh);
  const size_t dwt_bytes = al256(sizeof(float) * 9 * kStemCh);
  const size_t pre_bytes = al256(2 * (size_t)kD * kFeat);
  const size_t qkvb_bytes = al256(sizeof(float) * 3 * kD * (size_t)cfg->n_layer);
  const size_t dwl_bytes = al256(sizeof(float) * kD * (size_t)cfg->conv_kernel * cfg->n_layer);
  const size_t total = 2 * pw_bytes + 2 * dwt_bytes + pre_bytes + qkvb_bytes + dwl_bytes;
  if (hipMalloc(&m->alloc, total) != hipSuccess) {
    m->alloc = nullptr;
    return fail(set_error(AE_ERR_HIP, "lfm2a_model_create: hipMalloc of the model tables failed"));
  }
  char* p = (char*)m->alloc;
  m->stem_pw[0] = (bf16*)p; p += pw_bytes;
  m->stem_pw[1] = (bf16*)p; p += pw_bytes;
  m->stem_dwt[0] = (float*)p; p += dwt_bytes;
  m->stem_dwt[1] = (float*)p; p += dwt_bytes;
  m->pre_w = (bf16*)p; p += pre_bytes;
  m->qkv_b = (float*)p; p += qkvb_bytes;
  m->dw_t = (float*)p;
  hipError_t e = launch_f32_to_bf16(w->stem_w[2], m->stem_pw[0], (int64_t)kStemCh * kStemCh, s);
  if (e == hipSuccess)
    e = launch_f32_to_bf16(w->stem_w[4], m->stem_pw[1], (int64_t)kStemCh * kStemCh, s);
  if (e == hipSuccess) e = launch_transpose_f32(w->stem_w[1], kStemCh, 9, m->stem_dwt[0], s);
  if (e == hipSuccess) e = launch_transpose_f32(w->stem_w[3], kStemCh, 9, m->stem_dwt[1], s);
  if (e == hipSuccess)
    e = launch_flatten_permute((const bf16*)w->pre_encode_out_w, kD, kStemCh, kF3, m->pre_w, s);
  for (int l = 0; l < cfg->n_layer && e == hipSuccess; ++l) {
    e = launch_concat3(m->blocks[l].attn_q_b, m->blocks[l].attn_k_b, m->blocks[l].attn_v_b, kD,
                       m->qkv_b + (size_t)l * 3 * kD, s);
    if (e == hipSuccess)
      e = launch_transpose_f32(m->blocks[l].conv_dw_w, kD, cfg->conv_kernel,
                               m->dw_t + (size_t)l * cfg->conv_kernel * kD, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(set_error(AE_ERR_HIP, std::string("lfm2a_model_create: ") + hipGetErrorString(e)));
  *out = m;
  return AE_OK;
}

void lfm2a_model_destroy(lfm2a_model* m) {
  if (!m) return;
  if (m->alloc) (void)hipFree(m->alloc);
  delete m;
}

size_t lfm2a_workspace_bytes(const lfm2a_model* m, int32_t B, int64_t total_frames,
                             int64_t total_tokens, int64_t max_tokens) {
  if (!m || B < 0 || total_frames < 0 || total_tokens < 0 || max_tokens < 0) return 0;
  // stem rows are bounded by the frame count: R1 <= (F + B) / 2, R2 <= (R1 + B) / 2
  const int64_t R1 = (total_frames + B) / 2 + 1, R2 = (R1 + B) / 2 + 1;
  return Layout(B, total_frames, R1, R2, total_tokens, max_tokens).total;
}

size_t lfm2a_attention_workspace_bytes(int32_t B) {
  if (B < 0) return 0;
  return al256(sizeof(int64_t) * 2 * (size_t)(B + 1)) + 256;
}

ae_status lfm2a_stem(const lfm2a_model* m, const float* feat, const int64_t* frame_off,
                     int32_t B, float* x, void* ws, size_t ws_bytes, ae_stream stream) {
  if (ae_status st = check_offsets(frame_off, B, "lfm2a_stem")) return st;
  std::vector<int64_t> fr(B);
  for (int i = 0; i < B; ++i) fr[i] = frame_off[i + 1] - frame_off[i];
  Geometry G;
  G.from_frames(fr);
  if (!m) return set_error(AE_ERR_INVALID, "lfm2a_stem: null model");
  if (G.T() == 0) return AE_OK;
  if (!feat || !x) return set_error(AE_ERR_INVALID, "lfm2a_stem: null pointer");
  if (!int_range(G.R1() * lfm::kF1))
    return set_error(AE_ERR_CAPACITY, "lfm2a_stem: batch too large for 32-bit row counts");
  const Layout L(B, G.F(), G.R1(), G.R2(), G.T(), G.max_t);
  if (ae_status st = check_ws(m, ws, ws_bytes, L.total, "lfm2a_stem")) return st;
  hipStream_t s = (hipStream_t)stream;
  Bufs b(ws, L, B);
  if (ae_status st = upload_tables(G, b, true, s)) return st;
  return run_stem(m, feat, G, b, x, s);
}

ae_status lfm2a_block(const lfm2a_model* m, int32_t layer, float* x, const int64_t* token_off,
                      int32_t B, void* ws, size_t ws_bytes, ae_stream stream) {
  if (ae_status st = check_offsets(token_off, B, "lfm2a_block")) return st;
  if (!m) return set_error(AE_ERR_INVALID, "lfm2a_block: null model");
  if (layer < 0 || layer >= m->cfg.n_layer)
    return set_error(AE_ERR_INVALID, "lfm2a_block: layer out of range");
  // geometry from the token counts alone
  Geometry G;
  G.B = B;
  G.so.assign(B + 1, 0); G.fo.assign(B + 1, 0); G.r1.assign(B + 1, 0); G.r2.assign(B + 1, 0);
  G.to.assign(token_off, token_off + B + 1);
  G.qt.assign(B + 1, 0);
  for (int i = 0; i < B; ++i) {
    const int64_t t = token_off[i + 1] - token_off[i];
    G.qt[i + 1] = G.qt[i] + (t + kQueriesPerBlock - 1) / kQueriesPerBlock;
    G.max_t = std::max(G.max_t, t);
  }
  if (G.T() == 0) return AE_OK;
  if (!x) return set_error(AE_ERR_INVALID, "lfm2a_block: null x");
  if (!int_range(G.T() * 4) || !int_range(2 * G.max_t))
    return set_error(AE_ERR_CAPACITY, "lfm2a_block: too many tokens for 32-bit row counts");
  const Layout L(B, 0, 0, 0, G.T(), G.max_t);
  if (ae_status st = check_ws(m, ws, ws_bytes, L.total, "lfm2a_block")) return st;
  hipStream_t s = (hipStream_t)stream;
  Bufs b(ws, L, B);
  if (ae_status st = upload_tables(G, b, true, s)) return st;
  AE_HIP_TRY(launch_pos_table(G.max_t, kD, b.pe, s));
  const lfm2a_block_weights& Lw = m->blocks[layer];
  if (ae_status st = run_ln(x, G.T(), Lw.ffn_norm_w, Lw.ffn_norm_b, false, nullptr, nullptr, b.a,
                            m->cfg.eps, s))
    return st;
  return run_block(m, layer, G, b, x, nullptr, nullptr, s);
}

ae_status lfm2a_adapter(const lfm2a_model* m, const float* x, int64_t n, float* out, void* ws,
                        size_t ws_bytes, ae_stream stream) {
  if (!m || n < 0) return set_error(AE_ERR_INVALID, "lfm2a_adapter: null model or n < 0");
  if (n == 0) return AE_OK;
  if (!x || !out) return set_error(AE_ERR_INVALID, "lfm2a_adapter: null pointer");
  if (!int_range(n * 4)) return set_error(AE_ERR_CAPACITY, "lfm2a_adapter: too many rows");
  const Layout L(1, 0, 0, 0, n, 0);
  if (ae_status st = check_ws(m, ws, ws_bytes, L.total, "lfm2a_adapter")) return st;
  hipStream_t s = (hipStream_t)stream;
  Bufs b(ws, L, 1);
  if (ae_status st = run_ln((float*)x, n, m->w.adapter_norm_w, m->w.adapter_norm_b, false,
                            nullptr, nullptr, b.a, m->cfg.eps, s))
    return st;
  return run_adapter(m, b, n, out, s);
}

ae_status lfm2a_encode(const lfm2a_model* m, const float* wave, const int64_t* sample_off,
                       int32_t B, float* out, void* ws, size_t ws_bytes, ae_stream stream) {
  if (ae_status st = check_offsets(sample_off, B, "lfm2a_encode")) return st;
  if (!m) return set_error(AE_ERR_INVALID, "lfm2a_encode: null model");
  std::vector<int64_t> n(B), fr(B);
  for (int i = 0; i < B; ++i) n[i] = sample_off[i + 1] - sample_off[i];
  if (ae_status st = lfm2a_plan(n.data(), B, nullptr, nullptr, nullptr)) return st;
  for (int i = 0; i < B; ++i) fr[i] = frames_of(n[i]);
  Geometry G;
  G.from_frames(fr);
  G.so.assign(sample_off, sample_off + B + 1);
  if (G.T() == 0) return AE_OK;
  if (!wave || !out) return set_error(AE_ERR_INVALID, "lfm2a_encode: null pointer");
  if (!int_range(G.R1() * lfm::kF1) || !int_range(G.T() * 4) || !int_range(2 * G.max_t))
    return set_error(AE_ERR_CAPACITY, "lfm2a_encode: batch too large for 32-bit row counts");
  const Layout L(B, G.F(), G.R1(), G.R2(), G.T(), G.max_t);
  if (ae_status st = check_ws(m, ws, ws_bytes, L.total, "lfm2a_encode")) return st;
  hipStream_t s = (hipStream_t)stream;
  Bufs b(ws, L, B);
  if (ae_status st = upload_tables(G, b, true, s)) return st;
  if (ae_status st = run_front(wave, G, b, b.mel, s)) return st;
  if (ae_status st = run_stem(m, b.mel, G, b, b.x, s)) return st;
  AE_HIP_TRY(launch_pos_table(G.max_t, kD, b.pe, s));
  const int nl = m->cfg.n_layer;
  if (ae_status st = run_ln(b.x, G.T(), m->blocks[0].ffn_norm_w, m->blocks[0].ffn_norm_b, false,
                            nullptr, nullptr, b.a, m->cfg.eps, s))
    return st;
  for (int l = 0; l < nl; ++l) {
    const float* nw = l + 1 < nl ? m->blocks[l + 1].ffn_norm_w : m->w.adapter_norm_w;
    const float* nb = l + 1 < nl ? m->blocks[l + 1].ffn_norm_b : m->w.adapter_norm_b;
    if (ae_status st = run_block(m, l, G, b, b.x, nw, nb, s)) return st;
  }
  return run_adapter(m, b, G.T(), out, s);
}

ae_status lfm2a_xl_attention(const void* qkv, const void* p, int64_t t_max, const float* u,
                             const float* v, const int64_t* token_off, int32_t B, void* o,
                             void* ws, size_t ws_bytes, ae_stream stream) {
  if (ae_status st = check_offsets(token_off, B, "lfm2a_xl_attention")) return st;
  std::vector<int64_t> tab(2 * (size_t)(B + 1), 0);
  int64_t max_t = 0;
  for (int i = 0; i <= B; ++i) tab[i] = token_off[i];
  for (int i = 0; i < B; ++i) {
    const int64_t t = token_off[i + 1] - token_off[i];
    tab[B + 1 + i + 1] = tab[B + 1 + i] + (t + kQueriesPerBlock - 1) / kQueriesPerBlock;
    max_t = std::max(max_t, t);
  }
  if (token_off[B] == 0) return AE_OK;
  if (!qkv || !p || !u || !v || !o) return set_error(AE_ERR_INVALID, "lfm2a_xl_attention: null pointer");
  if (t_max < max_t)
    return set_error(AE_ERR_SHAPE, "lfm2a_xl_attention: t_max below the longest clip");
  if (!int_range(2 * t_max)) return set_error(AE_ERR_CAPACITY, "lfm2a_xl_attention: t_max too large");
  if (!ws || ws_bytes < lfm2a_attention_workspace_bytes(B))
    return set_error(AE_ERR_CAPACITY, "lfm2a_xl_attention: workspace too small");
  if ((uintptr_t)ws & 7) return set_error(AE_ERR_INVALID, "lfm2a_xl_attention: misaligned workspace");
  hipStream_t s = (hipStream_t)stream;
  int64_t* d = (int64_t*)ws;
  AE_HIP_TRY(launch_write_i64(d, tab.data(), (int)tab.size(), s));
  LFM_LAUNCH(AE_K_LFM_ATTN, s, launch_xl_attention((const bf16*)qkv, (const bf16*)p, t_max, u, v,
                                                    d, d + B + 1, B, tab[2 * B + 1], (bf16*)o, s));
  return AE_OK;
}

}  // extern "C"
