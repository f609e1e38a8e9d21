// Decode: device-side work-map plan + fused page scoring and top-16.
//
// Plan (one workgroup): history pages of request r are 0..hist_r-1 with
// hist_r = (seq_len_r - 1) / 128 (the last query's local page bounds every
// row of the request), clamped to max_pages.  A chunk size is picked so that
// the whole batch splits into about kTargetItems equal work items (at least
// kMinChunk pages each); every request gets max(1, ceil(hist_r / chunk))
// items.  Items = (request, first page, end page, first item of the request,
// item count of the request).
//
// Score (one wave per work item): stream the item's pages through the MFMA
// with the request's query rows as the B operand, reduce each page to its max
// over tokens, keep a running top-15 per query column in registers, write the
// list to the workspace, and the LAST item of a request to arrive (an atomic
// counter per request) merges the request's lists and writes the output rows.
#include <cmath>

#include "common.h"

namespace mi_idx {

constexpr int kTargetItems = 2048;
constexpr int kMinChunk = 4;
constexpr int kPlanHeaderInts = 16;
constexpr int kItemInts = 8;
constexpr size_t kWsHeaderBytes = 256;

// Plan header (int32): [0] item count, [1] chunk pages, [2] num_reqs,
// [3] query_len, [4] max_pages, [5] capacity.
struct DecodeItem {
  int r, j0, j1, first, count, pad0, pad1, pad2;
};

__host__ __device__ inline size_t decode_capacity(int max_reqs) {
  return (size_t)max_reqs + kTargetItems;
}

__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t *__restrict__ seq_lens,
                                                           int num_reqs, int max_pages,
                                                           int query_len, int capacity,
                                                           int32_t *__restrict__ plan,
                                                           uint32_t *__restrict__ ws_words) {
  __shared__ long long s_part[1024];
  __shared__ int s_chunk;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  // Contiguous segment of requests per thread.
  const int per = (num_reqs + nt - 1) / nt;
  const int r0 = min(num_reqs, tid * per), r1 = min(num_reqs, r0 + per);
  long long hsum = 0;
  for (int r = r0; r < r1; ++r) {
    int sl = seq_lens[r];
    int h = sl >= 1 ? (sl - 1) >> 7 : 0;
    hsum += min(h, max_pages);
  }
  s_part[tid] = hsum;
  __syncthreads();
  if (tid == 0) {
    long long total = 0;
    for (int i = 0; i < nt; ++i) total += s_part[i];
    long long c = (total + kTargetItems - 1) / kTargetItems;
    s_chunk = (int)max((long long)kMinChunk, c);
  }
  __syncthreads();
  const int chunk = s_chunk;
  // Item counts and their exclusive scan over the thread segments.
  long long cnt = 0;
  for (int r = r0; r < r1; ++r) {
    int sl = seq_lens[r];
    int h = min(sl >= 1 ? (sl - 1) >> 7 : 0, max_pages);
    cnt += max(1, (h + chunk - 1) / chunk);
  }
  __syncthreads();
  s_part[tid] = cnt;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial counts.
  for (int off = 1; off < nt; off <<= 1) {
    long long v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  long long first = s_part[tid] - cnt;
  for (int r = r0; r < r1; ++r) {
    int sl = seq_lens[r];
    int h = min(sl >= 1 ? (sl - 1) >> 7 : 0, max_pages);
    int n = max(1, (h + chunk - 1) / chunk);
    for (int i = 0; i < n; ++i) {
      long long it = first + i;
      if (it < capacity) {
        int4 *dst = reinterpret_cast<int4 *>(plan + kPlanHeaderInts + it * kItemInts);
        dst[0] = make_int4(r, min(h, i * chunk), min(h, (i + 1) * chunk), (int)first);
        dst[1] = make_int4(n, 0, 0, 0);
      }
    }
    first += n;
    ws_words[kWsHeaderBytes / 4 + r] = 0u;   // arrival counter of request r
  }
  if (tid == nt - 1) {
    long long total_items = s_part[nt - 1];
    plan[0] = (int)min(total_items, (long long)capacity);
    plan[1] = chunk;
    plan[2] = num_reqs;
    plan[3] = query_len;
    plan[4] = max_pages;
    plan[5] = capacity;
    ws_words[0] = total_items > capacity ? 2u : 0u;   // error word
  }
}

template <int NCG>
__global__ __launch_bounds__(64) void decode_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, int num_reqs, int query_len, int H, int max_pages,
    float scale, const int32_t *__restrict__ plan, uint8_t *__restrict__ ws,
    int32_t *__restrict__ out, float *__restrict__ scores_out) {
  const int item = blockIdx.x;
  if (item >= plan[0]) return;
  const DecodeItem it = *reinterpret_cast<const DecodeItem *>(plan + kPlanHeaderInts +
                                                                (size_t)item * kItemInts);
  const int lane = threadIdx.x;
  const int t16 = lane & 15, g = lane >> 4;
  const int r = it.r;
  if (r < 0 || r >= num_reqs) return;
  const int rows = query_len * H;
  const int sl = seq_lens[r];
  uint32_t *ws_words = reinterpret_cast<uint32_t *>(ws);
  uint64_t *partial = reinterpret_cast<uint64_t *>(
      ws + kWsHeaderBytes + (((size_t)4 * num_reqs + 255) & ~(size_t)255));

  // Query fragments (B operand) and the causal bound of each column.
  v8i bq[NCG];
  int Lc[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int col = cg * 16 + t16;
    Lc[cg] = -1;
    bq[cg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    if (col < rows) {
      const int i = col / H, h = col - (col / H) * H;
      const int64_t T = (int64_t)r * query_len + i;
      const uint8_t *qp = q + (T * H + h) * kDim;
      const u32x4 lo = *reinterpret_cast<const u32x4 *>(qp + 16 * g);
      const u32x4 hi = *reinterpret_cast<const u32x4 *>(qp + 64 + 16 * g);
      bq[cg] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int p = sl - query_len + i;
      Lc[cg] = p >= 0 ? min(p >> 7, max_pages) : -1;
    }
  }
  TopList top[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) top[cg].clear();

  const int32_t *bt = block_table + (int64_t)r * bt_stride;
  bool bad = false;
  // Page pipeline: the next page's 8 tiles are in flight while the current
  // page goes through the MFMA.  Block-table entries are fetched 64 at a time
  // (one per lane) and broadcast with readlane.
  u32x4 a_cur[8], a_nxt[8];
  uint32_t s_cur[8], s_nxt[8];
  int bt_base = it.j0;
  int bt_lane = (bt_base + lane < it.j1) ? bt[bt_base + lane] : -1;
  auto phys_of = [&](int j) -> int {
    if (j - bt_base >= 64) {
      bt_base += 64;
      bt_lane = (bt_base + lane < it.j1) ? bt[bt_base + lane] : -1;
    }
    return __builtin_amdgcn_readlane(bt_lane, j - bt_base);
  };
  auto issue = [&](int phys, u32x4 *a, uint32_t *sc) {
    const uint8_t *page = pages + (int64_t)phys * kPageBytes;
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      const uint8_t *tp = page + (tile * 16 + t16) * kTokenBytes;
      const u32x4a4 a4 = *reinterpret_cast<const u32x4a4 *>(tp + 16 * g);
      a[tile] = u32x4{a4.x, a4.y, a4.z, a4.w};
      sc[tile] = tp[64 + g];
    }
  };
  int phys_cur = it.j0 < it.j1 ? phys_of(it.j0) : -1;
  bool ok_cur = phys_cur >= 0 && (int64_t)phys_cur < num_blocks;
  if (ok_cur) issue(phys_cur, a_cur, s_cur);
  for (int j = it.j0; j < it.j1; ++j) {
    bool ok_nxt = false;
    if (j + 1 < it.j1) {
      const int phys_nxt = phys_of(j + 1);
      ok_nxt = phys_nxt >= 0 && (int64_t)phys_nxt < num_blocks;
      if (ok_nxt) issue(phys_nxt, a_nxt, s_nxt);
    }
    if (ok_cur) {
      float m[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) m[cg] = -INFINITY;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          m[cg] = fmaxf(m[cg], max4(mfma_fp4_fp8(a_cur[tile], bq[cg], s_cur[tile])));
      }
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        float v = m[cg];
        v = fmaxf(v, __shfl_xor(v, 16, 64));
        v = fmaxf(v, __shfl_xor(v, 32, 64));
        if (j < Lc[cg]) {
          top[cg].insert(make_key(v, j));
          if (scores_out != nullptr && g == 0) {
            const int col = cg * 16 + t16;
            const int i = col / H, h = col - (col / H) * H;
            const int64_t T = (int64_t)r * query_len + i;
            scores_out[(T * H + h) * max_pages + j] = v * scale;
          }
        }
      }
    } else {
      bad = true;
    }
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      a_cur[tile] = a_nxt[tile];
      s_cur[tile] = s_nxt[tile];
    }
    ok_cur = ok_nxt;
  }
  if (bad && lane == 0) atomicOr(&ws_words[0], 1u);

  // Publish this item's lists.
  if (g == 0) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int col = cg * 16 + t16;
      if (col < rows) {
        uint64_t *dst = partial + ((size_t)item * rows + col) * kHist;
#pragma unroll
        for (int k = 0; k < kHist; ++k) dst[k] = top[cg].k[k];
      }
    }
  }
  __threadfence();
  uint32_t old = 0;
  if (lane == 0) old = atomicAdd(&ws_words[kWsHeaderBytes / 4 + r], 1u);
  old = (uint32_t)__shfl((int)old, 0, 64);
  if (old + 1 != (uint32_t)it.count) return;
  __threadfence();

  // Last arrival: merge the request's lists, 4 lane groups over the items.
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int col = cg * 16 + t16;
    TopList acc;
    acc.clear();
    if (col < rows) {
      for (int x = it.first + g; x < it.first + it.count; x += 4) {
        const uint64_t *src = partial + ((size_t)x * rows + col) * kHist;
        for (int k = 0; k < kHist; ++k) {
          const uint64_t key = __builtin_nontemporal_load(src + k);
          if (key <= acc.threshold()) break;
          acc.insert(key);
        }
      }
    }
    merge_xor(acc, 16);
    merge_xor(acc, 32);
    if (g == 0 && col < rows) {
      const int i = col / H, h = col - (col / H) * H;
      const int64_t T = (int64_t)r * query_len + i;
      write_row(out + (T * H + h) * kTopk, acc, Lc[cg]);
    }
  }
  if (lane == 0) ws_words[kWsHeaderBytes / 4 + r] = 0u;   // ready for the next call
}

}  // namespace mi_idx

using namespace mi_idx;

static size_t ws_counters_bytes(int max_reqs) { return ((size_t)4 * max_reqs + 255) & ~(size_t)255; }

extern "C" size_t mi_idx_decode_plan_bytes(int max_reqs) {
  if (max_reqs < 0) return 0;
  return (size_t)kPlanHeaderInts * 4 + decode_capacity(max_reqs) * kItemInts * 4;
}

extern "C" size_t mi_idx_decode_workspace_bytes(int max_reqs, int query_len, int num_heads) {
  if (max_reqs < 0 || query_len < 1 || num_heads < 1) return 0;
  return kWsHeaderBytes + ws_counters_bytes(max_reqs) +
         decode_capacity(max_reqs) * (size_t)query_len * num_heads * kHist * 8;
}

static int plan_capacity(size_t plan_bytes) {
  if (plan_bytes < (size_t)kPlanHeaderInts * 4) return 0;
  size_t c = (plan_bytes - kPlanHeaderInts * 4) / (kItemInts * 4);
  return c > 0x7FFFFFF ? 0x7FFFFFF : (int)c;
}

static int check_decode_sizes(const char *who, int num_reqs, int query_len, int num_heads,
                              int max_pages, size_t plan_bytes, size_t ws_bytes, bool need_heads) {
  if (num_reqs < 0) return mi_idx_fail(MI_IDX_EINVAL, "%s: num_reqs %d < 0", who, num_reqs);
  if (query_len < 1 || query_len > MI_IDX_MAX_QUERY_LEN)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "%s: query_len %d outside 1..8", who, query_len);
  if (need_heads && (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS))
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "%s: num_heads %d outside 1..8", who, num_heads);
  if (max_pages < 0) return mi_idx_fail(MI_IDX_EINVAL, "%s: max_pages %d < 0", who, max_pages);
  const int cap = plan_capacity(plan_bytes);
  if ((size_t)cap < decode_capacity(num_reqs))
    return mi_idx_fail(MI_IDX_ECAPACITY, "%s: plan_bytes %zu < %zu needed for %d requests", who,
                       plan_bytes, mi_idx_decode_plan_bytes(num_reqs), num_reqs);
  size_t need = kWsHeaderBytes + ws_counters_bytes(num_reqs);
  if (need_heads) need += (size_t)cap * query_len * num_heads * kHist * 8;
  if (ws_bytes < need)
    return mi_idx_fail(MI_IDX_ECAPACITY, "%s: ws_bytes %zu < %zu needed", who, ws_bytes, need);
  return MI_IDX_OK;
}

extern "C" int mi_idx_plan_decode(const int32_t *seq_lens, int num_reqs, int query_len,
                                  int max_pages, void *plan, size_t plan_bytes, void *workspace,
                                  size_t ws_bytes, void *stream) {
  mi_idx_clear_error();
  int st = check_decode_sizes("plan_decode", num_reqs, query_len, 1, max_pages, plan_bytes,
                              ws_bytes, false);
  if (st) return st;
  if (!plan || !workspace || (num_reqs > 0 && !seq_lens))
    return mi_idx_fail(MI_IDX_EINVAL, "plan_decode: null pointer");
  if (((uintptr_t)plan % 16) || ((uintptr_t)workspace % 16))
    return mi_idx_fail(MI_IDX_EINVAL, "plan_decode: plan and workspace must be 16-byte aligned");
  const int cap = plan_capacity(plan_bytes);
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, seq_lens,
                     num_reqs, max_pages, query_len, cap, (int32_t *)plan, (uint32_t *)workspace);
  return mi_idx_check_launch("plan_decode");
}

extern "C" int mi_idx_score_topk_decode(const uint8_t *q, const uint8_t *pages,
                                        int64_t num_blocks, const int32_t *block_table,
                                        int64_t bt_stride, const int32_t *seq_lens, int num_reqs,
                                        int query_len, int num_heads, int max_pages, float scale,
                                        const void *plan, size_t plan_bytes, void *workspace,
                                        size_t ws_bytes, int32_t *topk_out, float *scores_out,
                                        void *stream) {
  mi_idx_clear_error();
  int st = check_decode_sizes("score_topk_decode", num_reqs, query_len, num_heads, max_pages,
                              plan_bytes, ws_bytes, true);
  if (st) return st;
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: scale must be positive and finite");
  if (num_reqs == 0) return MI_IDX_OK;
  if (!q || !pages || !block_table || !seq_lens || !plan || !workspace || !topk_out)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: null pointer");
  if (((uintptr_t)q % 16) || ((uintptr_t)pages % 16) || ((uintptr_t)topk_out % 16) ||
      ((uintptr_t)workspace % 16) || ((uintptr_t)plan % 16))
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: q, pages, topk_out, plan and "
                                      "workspace must be 16-byte aligned");
  if (num_blocks <= 0) return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: num_blocks <= 0");
  if (bt_stride < max_pages)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: bt_stride %lld < max_pages %d",
                       (long long)bt_stride, max_pages);
  const int cap = plan_capacity(plan_bytes);
  const int rows = query_len * num_heads;
  const int ncg = (rows + 15) / 16;
  const dim3 grid(cap), block(64);
  hipStream_t s = (hipStream_t)stream;
#define MI_IDX_LAUNCH_DEC(N)                                                                   \
  hipLaunchKernelGGL(decode_score_kernel<N>, grid, block, 0, s, q, pages, num_blocks,          \
                     block_table, bt_stride, seq_lens, num_reqs, query_len, num_heads,         \
                     max_pages, scale, (const int32_t *)plan, (uint8_t *)workspace, topk_out,  \
                     scores_out)
  switch (ncg) {
    case 1: MI_IDX_LAUNCH_DEC(1); break;
    case 2: MI_IDX_LAUNCH_DEC(2); break;
    case 3: MI_IDX_LAUNCH_DEC(3); break;
    default: MI_IDX_LAUNCH_DEC(4); break;
  }
#undef MI_IDX_LAUNCH_DEC
  return mi_idx_check_launch("score_topk_decode");
}
