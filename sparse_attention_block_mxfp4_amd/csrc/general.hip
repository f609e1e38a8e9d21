// The general selection: any topk, any forced leading / trailing windows,
// and a local page that competes when no trailing window forces it (the vllm
// "indexer_flashinfer" page: MiniMaxM3IndexerFlashInferImpl.forward scores
// the valid pages causally and selects with force_begin leading and
// force_end trailing pages; MiniMaxM3IndexerFlashInferMetadataBuilder.build:
// p // 128 + 1 valid pages per row).
//
// It runs after a score call that wrote every history page's score
// (scores_out).  Two kernels complete it:
//   local_score_kernel: the score of each row's own page over its causal
//     prefix (tokens 0 .. p % 128), one workgroup per row, one thread per
//     token and head group;
//   select_general_kernel: per (row, head), the topk - force_begin -
//     force_end best pages strictly between the two windows (the local page
//     among them when the trailing window is empty), found by an exact radix
//     select over the selection keys, written in ascending id order between
//     the forced windows.
#include <cmath>

#include "common.h"

namespace mi_idx {

constexpr int kLocalThreads = 2 * kPageTokens;   // 128 tokens x 2 head groups
constexpr int kSelThreads = 256;

// E2M1 code -> value (sign in bit 3; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  // 1.5 * 2^(e-1) style closed form: m = 2e + mantissa bit
  const float mag = m < 2u ? 0.5f * (float)m : (m & 1u ? 1.5f : 1.0f) * (float)(1u << ((m >> 1) - 1u));
  return (c & 8u) ? -mag : mag;
}

// E4M3 "fn" byte -> value (bias 7, no infinities, 0x7F / 0xFF NaN).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 15u && m == 7u) mag = __uint_as_float(0x7FC00000u);
  else if (e == 0u) mag = ldexpf((float)m, -9);
  else mag = ldexpf((float)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -mag : mag;
}

// Row t of a score call -> (request, position): decode rows are
// r * query_len + i at seq_lens[r] - query_len + i; prefill rows (cu_seqlens_q
// given) are cu[r] + j at context_lens[r] + j.
__device__ __forceinline__ void row_position(int64_t t, const int32_t *seq_lens,
                                             const int32_t *cu, const int32_t *ctx, int num_reqs,
                                             int query_len, int &r, int &p) {
  if (cu == nullptr) {
    r = (int)(t / query_len);
    p = seq_lens[r] - query_len + (int)(t - (int64_t)r * query_len);
  } else {
    int lo = 0, hi = num_reqs - 1;   // the last r with cu[r] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    r = lo;
    p = ctx[r] + (int)(t - cu[r]);
  }
}

// One workgroup per row: thread (head group hg, token t) decodes token t of
// the row's own page once (its 128 values, scale applied per 32-dim block
// after the block's exact-product sum) and scores it against heads hg, hg +
// 2, ...; tokens past p % 128 score -inf.
template <bool kBf16>
__global__ __launch_bounds__(kLocalThreads) void local_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ ctx, int num_reqs, int query_len, int H, int max_pages,
    float scale, float *__restrict__ out) {
  __shared__ float s_q[MI_IDX_MAX_HEADS][kDim];
  __shared__ float s_max[kLocalThreads / 64][MI_IDX_MAX_HEADS];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = tid & (kPageTokens - 1), hg = tid >> 7;
  int r = 0, p = -1;
  row_position(t, seq_lens, cu, ctx, num_reqs, query_len, r, p);
  const int L = p >> 7;
  int64_t phys = -1;
  if (p >= 0 && L < max_pages) {
    const int32_t v = block_table[(int64_t)r * bt_stride + L];
    if (v >= 0 && (int64_t)v < num_blocks) phys = v;
  }
  float *dst = out + t * H;
  if (phys < 0) {   // no readable local page (the same for the whole workgroup)
    if (tid < H) dst[tid] = __uint_as_float(0x7FC00000u);
    return;
  }
  for (int i = tid; i < H * kDim; i += kLocalThreads) {
    const int h = i / kDim, d = i - h * kDim;
    const int64_t at = (t * H + h) * kDim + d;
    s_q[h][d] = kBf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(q)[at] << 16)
                      : e4m3_value(q[at]);
  }
  const bool causal = tok <= (p & (kPageTokens - 1));   // tokens 0 .. p % 128
  float kv[kDim];
  float f[4];
  if (causal) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(pages + phys * kPageBytes +
                                                           tok * kTokenBytes);
    const uint32_t sw = w[16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t sb = (sw >> (8 * b)) & 0xFFu;
      f[b] = sb == 255u ? __uint_as_float(0x7FC00000u) : ldexpf(1.0f, (int)sb - 127);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = w[i];
#pragma unroll
      for (int k = 0; k < 8; ++k) kv[8 * i + k] = e2m1_value((word >> (4 * k)) & 15u);
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int h = hg; h < H; h += 2) {
    float v = -INFINITY;
    if (causal) {
      v = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < 32; ++d) acc = fmaf(kv[32 * b + d], s_q[h][32 * b + d], acc);
        v += acc * f[b];
      }
    }
    // max over the group's 128 tokens (NaN-propagating, as the page maxima)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = nmax(v, __shfl_xor(v, off, 64));
    if (lane == 0) s_max[wave][h] = v;
  }
  __syncthreads();
  if (tid < H) {
    const int g = tid & 1;   // head h lives in head group h % 2 = waves 2g, 2g + 1
    dst[tid] = scale * nmax(s_max[2 * g][tid], s_max[2 * g + 1][tid]);
  }
}

// Per (row, head): the forced windows and the take best candidates, ascending.
__global__ __launch_bounds__(kSelThreads) void select_general_kernel(
    const float *__restrict__ scores, int64_t stride, const float *__restrict__ local_scores,
    const int32_t *__restrict__ ranked, int topk, int init_blocks, int local_blocks,
    int max_k_tiles, int32_t *__restrict__ out) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_bin, s_rest;
  __shared__ uint32_t s_cnt[kSelThreads];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = ranked[row * kTopk + (kTopk - 1)];   // the row's local page, -1: padding
  int32_t *dst = out + row * topk;
  if (L < 0) {
    for (int i = tid; i < topk; i += kSelThreads) dst[i] = -1;
    return;
  }
  const int nvp = L + 1;
  if (nvp <= topk) {   // every valid page
    for (int i = tid; i < topk; i += kSelThreads) dst[i] = i < nvp ? i : -1;
    return;
  }
  const int fb = min(min(init_blocks, max_k_tiles), topk);
  const int fe = min(local_blocks, topk - fb);
  const int take = topk - fb - fe;
  const int c0 = fb, c1 = nvp - fe;   // candidates [c0, c1), take of them
  for (int i = tid; i < fb; i += kSelThreads) dst[i] = i;
  for (int i = tid; i < fe; i += kSelThreads) dst[fb + take + i] = nvp - fe + i;
  if (take == 0) return;
  const float *srow = scores + row * stride;
  auto key_of = [&](int j) -> uint64_t {
    return make_key(j < L ? srow[j] : local_scores[row], j);
  };
  // Radix select of the take-th largest key, a byte at a time from the top.
  uint64_t prefix = 0, mask = 0;
  uint32_t k = (uint32_t)take;
  for (int byte = 7; byte >= 0; --byte) {
    s_hist[tid] = 0u;
    __syncthreads();
    const int sh = 8 * byte;
    for (int j = c0 + tid; j < c1; j += kSelThreads) {
      const uint64_t key = key_of(j);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(uint32_t)(key >> sh) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {   // wave 0: the bin holding the k-th largest key
      const uint32_t h0 = s_hist[4 * tid], h1 = s_hist[4 * tid + 1], h2 = s_hist[4 * tid + 2],
                     h3 = s_hist[4 * tid + 3];
      const uint32_t mine = h0 + h1 + h2 + h3;
      uint32_t above = mine;   // bins of this lane and every higher lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t x = __shfl_down(above, off, 64);
        above += tid + off < 64 ? x : 0u;
      }
      const uint32_t higher = above - mine;   // keys in higher lanes' bins
      if (higher < k && k <= above) {         // exactly one lane
        uint32_t c = higher;
        const uint32_t hb[4] = {h0, h1, h2, h3};
        int bin = 4 * tid + 3;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if (c + hb[i] >= k) { bin = 4 * tid + i; break; }
          c += hb[i];
        }
        s_bin = (uint32_t)bin;
        s_rest = k - c;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_bin << sh;
    mask |= (uint64_t)255u << sh;
    k = s_rest;
    __syncthreads();
  }
  // prefix is now the take-th largest key: exactly take keys are >= it.
  // Compaction in id order: thread i owns a contiguous run of candidates.
  const int count = c1 - c0;
  const int per = (count + kSelThreads - 1) / kSelThreads;
  const int a = c0 + tid * per, b = min(c1, a + per);
  uint32_t n = 0;
  for (int j = a; j < b; ++j) n += key_of(j) >= prefix ? 1u : 0u;
  s_cnt[tid] = n;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {   // inclusive scan
    const uint32_t x = tid >= off ? s_cnt[tid - off] : 0u;
    __syncthreads();
    s_cnt[tid] += x;
    __syncthreads();
  }
  uint32_t pos = s_cnt[tid] - n;
  for (int j = a; j < b; ++j)
    if (key_of(j) >= prefix) dst[fb + pos++] = j;
}

}  // namespace mi_idx

using namespace mi_idx;

extern "C" int mi_idx_score_local(const void *q, int q_dtype, const uint8_t *pages,
                                  int64_t num_blocks, const int32_t *block_table,
                                  int64_t bt_stride, const int32_t *seq_lens,
                                  const int32_t *cu_seqlens_q, const int32_t *context_lens,
                                  int num_reqs, int query_len, int64_t total_rows, int num_heads,
                                  int max_pages, float scale, float *local_out, void *stream) {
  mi_idx_clear_error();
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "score_local: num_heads %d outside 1..8", num_heads);
  if (q_dtype != MI_IDX_Q_E4M3 && q_dtype != MI_IDX_Q_BF16)
    return mi_idx_fail(MI_IDX_EINVAL, "score_local: q_dtype %d is neither E4M3 (0) nor bf16 (1)",
                       q_dtype);
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return mi_idx_fail(MI_IDX_EINVAL, "score_local: scale must be positive and finite");
  if (num_reqs < 0 || total_rows < 0 || max_pages < 0)
    return mi_idx_fail(MI_IDX_EINVAL, "score_local: negative size");
  const bool prefill = cu_seqlens_q != nullptr;
  if (!prefill) {
    if (query_len < 1 || query_len > MI_IDX_MAX_QUERY_LEN)
      return mi_idx_fail(MI_IDX_EUNSUPPORTED, "score_local: query_len %d outside 1..8",
                         query_len);
    if (total_rows != (int64_t)num_reqs * query_len)
      return mi_idx_fail(MI_IDX_EINVAL, "score_local: decode rows must be num_reqs * query_len");
  } else if (!context_lens) {
    return mi_idx_fail(MI_IDX_EINVAL, "score_local: prefill rows need context_lens");
  }
  if (total_rows == 0 || num_reqs == 0) return MI_IDX_OK;
  if (total_rows > 0x7FFFFFFF) return mi_idx_fail(MI_IDX_EINVAL, "score_local: too many rows");
  if (!q || !pages || !block_table || !local_out || (!prefill && !seq_lens))
    return mi_idx_fail(MI_IDX_EINVAL, "score_local: null pointer");
  if (num_blocks <= 0) return mi_idx_fail(MI_IDX_EINVAL, "score_local: num_blocks <= 0");
  if (bt_stride < max_pages)
    return mi_idx_fail(MI_IDX_EINVAL, "score_local: bt_stride < max_pages");
  const dim3 grid((unsigned)total_rows), block(kLocalThreads);
  const uint8_t *qb = static_cast<const uint8_t *>(q);
  hipStream_t s = (hipStream_t)stream;
  if (q_dtype == MI_IDX_Q_BF16)
    hipLaunchKernelGGL(local_score_kernel<true>, grid, block, 0, s, qb, pages, num_blocks,
                       block_table, bt_stride, seq_lens, cu_seqlens_q, context_lens, num_reqs,
                       query_len, num_heads, max_pages, scale, local_out);
  else
    hipLaunchKernelGGL(local_score_kernel<false>, grid, block, 0, s, qb, pages, num_blocks,
                       block_table, bt_stride, seq_lens, cu_seqlens_q, context_lens, num_reqs,
                       query_len, num_heads, max_pages, scale, local_out);
  return mi_idx_check_launch("score_local");
}

extern "C" int mi_idx_select_topk(const float *scores, int64_t scores_stride,
                                  const float *local_scores, const int32_t *ranked, int64_t n,
                                  int topk, int init_blocks, int local_blocks, int max_k_tiles,
                                  int32_t *out, void *stream) {
  mi_idx_clear_error();
  if (n < 0) return mi_idx_fail(MI_IDX_EINVAL, "select_topk: n < 0");
  if (topk < 1 || topk > MI_IDX_MAX_TOPK)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "select_topk: topk_blocks %d outside 1..%d", topk,
                       MI_IDX_MAX_TOPK);
  if (init_blocks < 0 || local_blocks < 0 || max_k_tiles < 0)
    return mi_idx_fail(MI_IDX_EINVAL, "select_topk: negative init_blocks, local_blocks or "
                                      "max_k_tiles");
  if (n == 0) return MI_IDX_OK;
  if (n > 0x7FFFFFFF) return mi_idx_fail(MI_IDX_EINVAL, "select_topk: too many rows");
  if (!scores || !ranked || !out) return mi_idx_fail(MI_IDX_EINVAL, "select_topk: null pointer");
  // the local page competes when the trailing window can be empty while
  // candidates are taken
  if (local_blocks == 0 && min(init_blocks, max_k_tiles) < topk && !local_scores)
    return mi_idx_fail(MI_IDX_EINVAL, "select_topk: local_blocks 0 makes the local page compete: "
                                      "local_scores (mi_idx_score_local) is needed");
  if (scores_stride < 1) return mi_idx_fail(MI_IDX_EINVAL, "select_topk: scores_stride < 1");
  if ((uintptr_t)ranked % 4 || (uintptr_t)out % 4 || (uintptr_t)scores % 4)
    return mi_idx_fail(MI_IDX_EINVAL, "select_topk: misaligned buffer");
  hipLaunchKernelGGL(select_general_kernel, dim3((unsigned)n), dim3(kSelThreads), 0,
                     (hipStream_t)stream, scores, scores_stride, local_scores, ranked, topk,
                     init_blocks, local_blocks, max_k_tiles, out);
  return mi_idx_check_launch("select_topk");
}
