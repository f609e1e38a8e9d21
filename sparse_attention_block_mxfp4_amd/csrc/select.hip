// General forced-block selection: a leading and a trailing window of pages
// always selected, any topk <= 16, ascending ids and -1 tail padding (the vllm
// "indexer_flashinfer" page, forward and build), derived from the 16-slot
// score-ranked rows the scorers write.
//
// Why the ranked rows are enough: a row's candidates (pages between the two
// windows) are its history pages minus at most force_begin + force_end - 1 of
// them (the trailing window always holds the local page, which is not a
// history page).  The take = topk - force_begin - force_end best candidates
// each have at most (force_begin + force_end - 1) + (take - 1) = topk - 2
// history pages ranked above them, so with topk <= 16 they are all among the
// row's 15 ranked history pages, and the first `take` ranked entries inside
// the candidate range are exactly those pages, in score order.
#include "common.h"

namespace mi_idx {

constexpr int kSelectThreads = 256;

// One thread per (row, head).  The chosen pages are sorted with a 16-input
// bitonic network (unchosen slots hold INT_MAX and sink to the end); the
// row's output is laid out in LDS, where the run of sorted pages starts at
// slot force_begin, and read back whole.
__global__ __launch_bounds__(kSelectThreads) void select_forced_kernel(
    const int32_t *__restrict__ ranked, int64_t n, int topk, int init_blocks, int local_blocks,
    int max_k_tiles, int32_t *__restrict__ out) {
  __shared__ int32_t s_row[kSelectThreads][kTopk + 1];   // +1: rows on distinct banks
  const int64_t i = (int64_t)blockIdx.x * kSelectThreads + threadIdx.x;
  if (i >= n) return;
  int v[kTopk];
  const int4 *src = reinterpret_cast<const int4 *>(ranked + i * kTopk);
#pragma unroll
  for (int q = 0; q < kTopk / 4; ++q) {
    const int4 x = src[q];
    v[4 * q] = x.x;
    v[4 * q + 1] = x.y;
    v[4 * q + 2] = x.z;
    v[4 * q + 3] = x.w;
  }
  const int L = v[kTopk - 1];
  const int nvp = L + 1;                              // pages 0..L are valid
  const bool all = nvp <= topk;                       // every valid page (or none: L < 0)
  const int fb = min(min(init_blocks, max_k_tiles), topk);   // the same for every row
  const int fe = min(local_blocks, topk - fb);
  const int take = topk - fb - fe;
  const int lo = fb, hi = nvp - fe;                   // candidates [lo, hi)
  // the first `take` ranked history entries inside [lo, hi), sorted by id
  int x[kTopk];
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kHist; ++k) {
    const bool c = v[k] >= lo && v[k] < hi && cnt < take;
    cnt += c ? 1 : 0;
    x[k] = c ? v[k] : 0x7FFFFFFF;
  }
  x[kTopk - 1] = 0x7FFFFFFF;
#pragma unroll
  for (int size = 2; size <= kTopk; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int a = 0; a < kTopk; ++a) {
        const int b = a ^ stride;
        if (b > a) {
          const bool up = (a & size) == 0;
          const int lo_v = min(x[a], x[b]), hi_v = max(x[a], x[b]);
          x[a] = up ? lo_v : hi_v;
          x[b] = up ? hi_v : lo_v;
        }
      }
    }
  }
  int32_t *row = s_row[threadIdx.x];
#pragma unroll
  for (int k = 0; k < kTopk; ++k) {
    int val = -1;
    if (k < fb) val = k;                                              // leading window
    if (k >= fb + take && k < fb + take + fe) val = hi + (k - fb - take);   // trailing
    if (all) val = k < nvp ? k : -1;
    row[k] = val;
  }
  if (!all) {
#pragma unroll
    for (int k = 0; k < kTopk; ++k)
      if (k < take) row[fb + k] = x[k];
  }
  int32_t *dst = out + i * topk;
  if (topk == kTopk) {
    int4 *d4 = reinterpret_cast<int4 *>(dst);
#pragma unroll
    for (int q = 0; q < kTopk / 4; ++q)
      d4[q] = make_int4(row[4 * q], row[4 * q + 1], row[4 * q + 2], row[4 * q + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < kTopk; ++k)
      if (k < topk) dst[k] = row[k];
  }
}

}  // namespace mi_idx

using namespace mi_idx;

extern "C" int mi_idx_select_forced(const int32_t *ranked, int64_t n, int topk, int init_blocks,
                                    int local_blocks, int max_k_tiles, int32_t *out,
                                    void *stream) {
  mi_idx_clear_error();
  if (n < 0) return mi_idx_fail(MI_IDX_EINVAL, "select_forced: n < 0");
  if (topk < 1 || topk > MI_IDX_TOPK)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "select_forced: topk_blocks %d outside 1..16", topk);
  if (local_blocks < 1)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED,
                       "select_forced: local_blocks %d < 1 would rank the unscored local page",
                       local_blocks);
  if (init_blocks < 0 || max_k_tiles < 0)
    return mi_idx_fail(MI_IDX_EINVAL, "select_forced: negative init_blocks or max_k_tiles");
  if (n == 0) return MI_IDX_OK;
  if (!ranked || !out) return mi_idx_fail(MI_IDX_EINVAL, "select_forced: null pointer");
  if ((uintptr_t)ranked % 16 || (uintptr_t)out % (topk == MI_IDX_TOPK ? 16 : 4))
    return mi_idx_fail(MI_IDX_EINVAL, "select_forced: ranked (and out when topk is 16) must be "
                                      "16-byte aligned");
  const uintptr_t a0 = (uintptr_t)ranked, a1 = a0 + (uintptr_t)n * MI_IDX_TOPK * 4;
  const uintptr_t b0 = (uintptr_t)out, b1 = b0 + (uintptr_t)n * topk * 4;
  if (a0 < b1 && b0 < a1 && !(b0 == a0 && topk == MI_IDX_TOPK))
    return mi_idx_fail(MI_IDX_EINVAL, "select_forced: out overlaps ranked (only the exact "
                                      "in-place call with topk 16 is allowed)");
  const int64_t grid = (n + kSelectThreads - 1) / kSelectThreads;
  if (grid > 0x7FFFFFFF) return mi_idx_fail(MI_IDX_EINVAL, "select_forced: too many rows");
  hipLaunchKernelGGL(select_forced_kernel, dim3((unsigned)grid), dim3(kSelectThreads), 0,
                     (hipStream_t)stream, ranked, n, topk, init_blocks, local_blocks, max_k_tiles,
                     out);
  return mi_idx_check_launch("select_forced");
}
