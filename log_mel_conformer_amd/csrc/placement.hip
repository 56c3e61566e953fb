// Soft-token placement around the encoder (egemma2_audio.rs, input_ids and
// embed_audio_inputs): the expansion of each audio placeholder in a token-id
// sequence into <|audio> + n x <|audio|> + <audio|> between BOS and EOS
// (host bookkeeping), and the merge that gives the text embedding rows
// whose id is the audio token the soft tokens in order (device).
//
// Merge on the device: the rank of an audio row among audio rows is an
// exclusive prefix count. Pass 1 counts audio ids per 256-id block (wave
// ballots), pass 2 turns the block counts into block offsets and the total
// (one block), pass 3 ranks each block's rows and copies the soft rows into
// the rows with rank < n_soft, float4 moves spread over up to 64 blocks per
// 256 ids.
#include <algorithm>
#include <string>
#include <vector>

#include "launch.h"

namespace ae {
namespace {

constexpr int kIdsPerBlock = 256;

__global__ void __launch_bounds__(256) k_count_audio(const int32_t* __restrict__ ids, int64_t L,
                                                     int32_t audio, int64_t* __restrict__ counts) {
  __shared__ int wc[4];
  const int64_t i = (int64_t)blockIdx.x * kIdsPerBlock + threadIdx.x;
  const bool hit = i < L && ids[i] == audio;
  const uint64_t b = __ballot(hit);
  if ((threadIdx.x & 63) == 0) wc[threadIdx.x >> 6] = __popcll(b);
  __syncthreads();
  if (threadIdx.x == 0) counts[blockIdx.x] = wc[0] + wc[1] + wc[2] + wc[3];
}

// offsets[b] = counts[0] + .. + counts[b - 1]; *total = all of them.
__global__ void __launch_bounds__(256) k_scan_counts(const int64_t* __restrict__ counts, int64_t nb,
                                                     int64_t* __restrict__ offsets,
                                                     int64_t* __restrict__ total) {
  __shared__ int64_t part[256];
  int64_t carry = 0;
  for (int64_t base = 0; base < nb; base += 256) {
    const int64_t i = base + threadIdx.x;
    const int64_t v = i < nb ? counts[i] : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan (Hillis-Steele)
      const int64_t add = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < nb) offsets[i] = carry + part[threadIdx.x] - v;
    carry += part[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

__global__ void __launch_bounds__(256) k_place_rows(const int32_t* __restrict__ ids, int64_t L,
                                                    int32_t audio,
                                                    const int64_t* __restrict__ offsets,
                                                    const float* __restrict__ soft, int64_t n_soft,
                                                    int d, float* __restrict__ x) {
  constexpr int U = 4;  // float4 copies in flight per thread
  __shared__ int wc[4];
  __shared__ int hit_row[kIdsPerBlock];
  __shared__ int64_t hit_rank[kIdsPerBlock];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * kIdsPerBlock + threadIdx.x;
  const bool hit = i < L && ids[i] == audio;
  const uint64_t b = __ballot(hit);
  if (lane == 0) wc[w] = __popcll(b);
  __syncthreads();
  int pos = __popcll(b & (lane ? (~0ull >> (64 - lane)) : 0ull));
  for (int k = 0; k < w; ++k) pos += wc[k];
  if (hit) {
    hit_row[pos] = threadIdx.x;
    hit_rank[pos] = offsets[blockIdx.x] + pos;
  }
  __syncthreads();
  const int n_hit = wc[0] + wc[1] + wc[2] + wc[3];
  // every (audio row, float4 of the row) pair of this block, U at a time
  const int q4 = d / 4;
  const int64_t items = (int64_t)n_hit * q4;
  const float4* s4 = (const float4*)soft;
  float4* x4 = (float4*)x;
  // blockIdx.y takes every gridDim.y-th group of 256 U items
  for (int64_t it = threadIdx.x + (int64_t)blockIdx.y * 256 * U; it < items;
       it += (int64_t)gridDim.y * 256 * U) {
    float4 v[U];
    int64_t dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      dst[u] = -1;
      const int64_t item = it + (int64_t)u * 256;
      if (item < items) {
        const int k = (int)(item / q4), c = (int)(item - (int64_t)k * q4);
        const int64_t rk = hit_rank[k];
        if (rk < n_soft) {
          v[u] = s4[rk * q4 + c];
          dst[u] = ((int64_t)blockIdx.x * kIdsPerBlock + hit_row[k]) * q4 + c;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u] >= 0) x4[dst[u]] = v[u];
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace
}  // namespace ae

using namespace ae;

extern "C" {

ae_status ae_expand_ids(const int32_t* body, int64_t len, const int64_t* n_soft, int32_t clips,
                        const ae_token_ids* tok, int64_t max_tokens, int32_t* out,
                        int64_t out_cap, int64_t* out_len) {
  if (!tok || !out_len || len < 0 || clips < 0 || (len > 0 && !body) ||
      (clips > 0 && !n_soft))
    return set_error(AE_ERR_INVALID, "ae_expand_ids: null pointer or negative size");
  int64_t found = 0;
  for (int64_t i = 0; i < len; ++i) found += body[i] == tok->audio;
  if (found != clips)
    return set_error(AE_ERR_SHAPE, "ae_expand_ids: the body holds " + std::to_string(found) +
                                        " audio placeholder(s) for " + std::to_string(clips) +
                                        " clip(s)");
  int64_t total = len + 2;
  for (int32_t k = 0; k < clips; ++k) {
    if (n_soft[k] < 0) return set_error(AE_ERR_INVALID, "ae_expand_ids: negative token count");
    total += n_soft[k] + 1;  // the placeholder becomes boa, n ids, eoa
  }
  *out_len = total;
  if (total > max_tokens)
    return set_error(AE_ERR_CAPACITY, "ae_expand_ids: " + std::to_string(total) +
                                          " tokens exceed the context of " +
                                          std::to_string(max_tokens));
  if (total > out_cap || !out)
    return set_error(AE_ERR_CAPACITY, "ae_expand_ids: output needs " + std::to_string(total) +
                                          " entries");
  int64_t o = 0;
  int32_t k = 0;
  out[o++] = tok->bos;
  for (int64_t i = 0; i < len; ++i) {
    if (body[i] == tok->audio) {
      out[o++] = tok->boa;
      for (int64_t j = 0; j < n_soft[k]; ++j) out[o++] = tok->audio;
      out[o++] = tok->eoa;
      ++k;
    } else {
      out[o++] = body[i];
    }
  }
  out[o++] = tok->eos;
  return AE_OK;
}

size_t ae_merge_workspace_bytes(int64_t L) {
  if (L < 0) return 0;
  const size_t nb = (size_t)((L + kIdsPerBlock - 1) / kIdsPerBlock);
  return align256(sizeof(int64_t) * nb) * 2 + 256;
}

ae_status ae_merge_soft_tokens(const int32_t* ids, int64_t L, int32_t audio, const float* soft,
                               int64_t n_soft, int32_t d, float* x, int64_t* count, void* ws,
                               size_t ws_bytes, ae_stream stream) {
  if (L < 0 || n_soft < 0 || d <= 0 || d % 4 != 0)
    return set_error(AE_ERR_INVALID, "ae_merge_soft_tokens: L, n_soft >= 0 and d a positive "
                                     "multiple of 4 required");
  if (L == 0) return AE_OK;
  if (!ids || !x || (n_soft > 0 && !soft))
    return set_error(AE_ERR_INVALID, "ae_merge_soft_tokens: null pointer");
  if (((uintptr_t)x | (uintptr_t)soft) & 15)
    return set_error(AE_ERR_INVALID, "ae_merge_soft_tokens: x and soft must be 16-byte aligned");
  const int64_t nb = (L + kIdsPerBlock - 1) / kIdsPerBlock;
  if (nb > INT32_MAX) return set_error(AE_ERR_CAPACITY, "ae_merge_soft_tokens: L too large");
  if (!ws || ws_bytes < ae_merge_workspace_bytes(L))
    return set_error(AE_ERR_CAPACITY, "ae_merge_soft_tokens: workspace needs " +
                                          std::to_string(ae_merge_workspace_bytes(L)) + " bytes");
  int64_t* counts = (int64_t*)ws;
  int64_t* offsets = (int64_t*)((char*)ws + align256(sizeof(int64_t) * nb));
  int64_t* total = (int64_t*)((char*)ws + 2 * align256(sizeof(int64_t) * nb));
  hipStream_t s = (hipStream_t)stream;
  timing_begin(AE_K_MERGE, s);
  hipLaunchKernelGGL(k_count_audio, dim3((unsigned)nb), dim3(256), 0, s, ids, L, audio, counts);
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(256), 0, s, counts, nb, offsets,
                     count ? count : total);
  // copies spread over gridDim.y blocks per 256 ids, so that short id
  // sequences still fill the GPU (each of them ranks the ids again: cheap)
  const unsigned split = (unsigned)std::max<int64_t>(1, std::min<int64_t>(64, 2048 / nb));
  hipLaunchKernelGGL(k_place_rows, dim3((unsigned)nb, split), dim3(256), 0, s, ids, L, audio,
                     offsets, soft, n_soft, d, x);
  timing_end(AE_K_MERGE, s);
  AE_HIP_TRY(hipGetLastError());
  return AE_OK;
}

}  // extern "C"
