// Decode: device-side work-map plan, fused page scoring with a per-wave
// top-15, and a per-request merge into the [T, H, 16] output.
//
// Plan (one workgroup): history pages of request r are 0..hist_r-1 with
// hist_r = (seq_len_r - 1) / 128 (the last query's local page bounds every
// row of the request), clamped to max_pages.  A chunk size is picked so that
// the whole batch splits into about kTargetItems equal work items (at least
// kMinChunk pages each); every request gets max(1, ceil(hist_r / chunk_r))
// items, each one wave's worth of work, with chunk_r = chunk raised where
// needed so that no request has more than kMaxItemsPerReq items.  Items = (request, first page, end
// page); the request's first item and item count go to the workspace.
//
// Score (4 independent waves per workgroup, one item each): a wave streams
// its pages through the MFMA with the request's query rows as the B operand,
// reduces each page to its max over tokens, keeps a running top-15 per query
// column in registers and writes the lists to the workspace.
//
// Merge (one workgroup per request, a second launch on the same stream, so
// the lists written by every XCD are visible without device-wide fences):
// merges the request's item lists into the 16 output slots of every row.
#include <cmath>

#include "common.h"

namespace mi_idx {

constexpr int kTargetItems = 2048;    // ~8 waves per CU
constexpr int kMinChunk = 4;
constexpr int kPlanHeaderInts = 16;
constexpr int kItemInts = 4;
constexpr size_t kWsHeaderBytes = 256;
constexpr int kListKeys = 16;         // 15 keys + an empty slot: 128-byte lists
constexpr int kDepth = 3;             // pages in flight per wave (register ring)
constexpr int kMergeKeys = 2048;      // LDS head keys of one merge pass
constexpr int kCandKeys = 2048;       // LDS candidate keys of one merge pass
constexpr int kMaxItemsPerReq = 256;  // bounds the merge's O(n^2) ranking

// Plan header (int32): [0] item count, [1] chunk pages, [2] num_reqs,
// [3] query_len, [4] max_pages, [5] capacity.  Items follow (int4 each).
// Workspace: [0, 256) header (word 0: error bits), then (first item, item
// count) int2 per request, padded to 256 bytes, then the item lists
// [capacity][rows][kListKeys] uint64.

__host__ __device__ inline size_t decode_capacity(int max_reqs) {
  return (size_t)max_reqs + kTargetItems;
}

__host__ __device__ inline size_t lists_bytes(size_t capacity, int rows) {
  return capacity * (size_t)rows * kListKeys * 8;
}

__host__ __device__ inline size_t lists_offset(int num_reqs) {
  return kWsHeaderBytes + (((size_t)8 * num_reqs + 255) & ~(size_t)255);
}

__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t *__restrict__ seq_lens,
                                                           int num_reqs, int max_pages,
                                                           int query_len, int capacity, int rows,
                                                           int32_t *__restrict__ plan,
                                                           uint8_t *__restrict__ ws) {
  __shared__ long long s_part[1024];
  __shared__ int s_chunk;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  int2 *req_info = reinterpret_cast<int2 *>(ws + kWsHeaderBytes);
  // Contiguous segment of requests per thread.
  const int per = (num_reqs + nt - 1) / nt;
  const int r0 = min(num_reqs, tid * per), r1 = min(num_reqs, r0 + per);
  long long hsum = 0;
  for (int r = r0; r < r1; ++r) {
    const int sl = seq_lens[r];
    hsum += min(sl >= 1 ? (sl - 1) >> 7 : 0, max_pages);
  }
  s_part[tid] = hsum;
  __syncthreads();
  if (tid == 0) {
    long long total = 0;
    for (int i = 0; i < nt; ++i) total += s_part[i];
    const long long c = (total + kTargetItems - 1) / kTargetItems;
    s_chunk = (int)max((long long)kMinChunk, c);
  }
  __syncthreads();
  const int chunk = s_chunk;
  auto chunk_of = [&](int h) {
    return max(chunk, (h + kMaxItemsPerReq - 1) / kMaxItemsPerReq);
  };
  // Item counts and their exclusive scan over the thread segments.
  long long cnt = 0;
  for (int r = r0; r < r1; ++r) {
    const int sl = seq_lens[r];
    const int h = min(sl >= 1 ? (sl - 1) >> 7 : 0, max_pages);
    const int c = chunk_of(h);
    cnt += max(1, (h + c - 1) / c);
  }
  __syncthreads();
  s_part[tid] = cnt;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial counts.
  for (int off = 1; off < nt; off <<= 1) {
    const long long v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  long long first = s_part[tid] - cnt;
  for (int r = r0; r < r1; ++r) {
    const int sl = seq_lens[r];
    const int h = min(sl >= 1 ? (sl - 1) >> 7 : 0, max_pages);
    const int c = chunk_of(h);
    const int n = max(1, (h + c - 1) / c);
    for (int i = 0; i < n; ++i) {
      const long long it = first + i;
      if (it < capacity)
        reinterpret_cast<int4 *>(plan + kPlanHeaderInts)[it] =
            make_int4(r, min(h, i * c), min(h, (i + 1) * c), 0);
    }
    req_info[r] = make_int2((int)first, n);
    first += n;
  }
  if (tid == nt - 1) {
    const long long total_items = s_part[nt - 1];
    plan[0] = (int)min(total_items, (long long)capacity);
    plan[1] = chunk;
    plan[2] = num_reqs;
    plan[3] = query_len;
    plan[4] = max_pages;
    plan[5] = capacity;
    reinterpret_cast<uint32_t *>(ws)[0] = total_items > capacity ? 2u : 0u;   // error bits
  }
}

__device__ __forceinline__ uint64_t *item_list(uint64_t *lists, int item, int rows, int col) {
  return lists + ((size_t)item * rows + col) * kListKeys;
}

template <int NCG, bool kScores>
__global__ __launch_bounds__(256) void decode_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, int num_reqs, int query_len, int H, int max_pages,
    float scale, const int32_t *__restrict__ plan, uint8_t *__restrict__ ws,
    float *__restrict__ scores_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int item = blockIdx.x * 4 + (tid >> 6);
  if (item >= plan[0]) return;
  const int4 it = reinterpret_cast<const int4 *>(plan + kPlanHeaderInts)[item];
  const int r = it.x, j0 = it.y, j1 = it.z;
  if (r < 0 || r >= num_reqs) return;
  const int t16 = lane & 15, g = lane >> 4;
  const int rows = query_len * H;
  const int sl = seq_lens[r];
  uint64_t *lists = reinterpret_cast<uint64_t *>(ws + lists_offset(num_reqs));

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

  // The item's pages are walked in segments of 64: one vector load brings
  // the segment's block-table entries (one per lane) and readlane hands
  // them out.  Inside a segment a ring of kDepth pages lives in registers:
  // kDepth-1 pages are in flight while one goes through the MFMA.  Ring
  // indices are compile-time (the ring loop is unrolled), so there are no
  // register copies, and every page load is unconditional -- a position past
  // the segment re-loads its last page (a cache hit) and an invalid page id
  // loads page 0 and is skipped -- so the wait counts stay exact.
  const int32_t *bt = block_table + (int64_t)r * bt_stride;
  bool bad = false;
  u32x4 a[kDepth][8];
  uint32_t s[kDepth][8];
  bool okb[kDepth];
  for (int seg = j0; seg < j1; seg += 64) {
    const int ns = min(64, j1 - seg);
    const int bt_lane = lane < ns ? bt[seg + lane] : -1;
    auto issue = [&](int i, u32x4 *ab, uint32_t *sb) -> bool {
      const int phys = __builtin_amdgcn_readlane(bt_lane, min(i, ns - 1));
      const bool valid = phys >= 0 && (int64_t)phys < num_blocks;
      const uint8_t *page = pages + (int64_t)(valid ? phys : 0) * kPageBytes;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
        const uint8_t *tp = page + (tile * 16 + t16) * kTokenBytes;
        const u32x4a4 a4 = *reinterpret_cast<const u32x4a4 *>(tp + 16 * g);
        ab[tile] = u32x4{a4.x, a4.y, a4.z, a4.w};
        sb[tile] = tp[64 + g];
      }
      if (i < ns && !valid) bad = true;
      return i < ns && valid;
    };
    // Keep the prologue's pages in ring order (no interleaving), as in the
    // steady state, so the wait counts at the loop head stay exact.
#pragma unroll
    for (int d = 0; d < kDepth - 1; ++d) {
      okb[d] = issue(d, a[d], s[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int ib = 0; ib < ns; ib += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int i = ib + u;
        const int j = seg + i;
        const int un = (u + kDepth - 1) % kDepth;
        okb[un] = issue(i + kDepth - 1, a[un], s[un]);
        __builtin_amdgcn_sched_barrier(0);
        if (okb[u]) {
          float m[NCG];
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) m[cg] = -INFINITY;
#pragma unroll
          for (int tile = 0; tile < 8; ++tile) {
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg)
              m[cg] = fmaxf(m[cg], max4(mfma_fp4_fp8(a[u][tile], bq[cg], s[u][tile])));
          }
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            float v = m[cg];
            v = fmaxf(v, __shfl_xor(v, 16, 64));
            v = fmaxf(v, __shfl_xor(v, 32, 64));
            if (j < Lc[cg]) {
              top[cg].insert(make_key(v, j));
              if (kScores && g == 0) {
                const int col = cg * 16 + t16;
                const int qi = col / H, h = col - (col / H) * H;
                const int64_t T = (int64_t)r * query_len + qi;
                scores_out[(T * H + h) * max_pages + j] = v * scale;
              }
            }
          }
        }
      }
    }
  }
  if (bad && lane == 0) atomicOr(reinterpret_cast<uint32_t *>(ws), 1u);

  // This item's lists (16 keys each, the last one empty).
  if (g == 0) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int col = cg * 16 + t16;
      if (col < rows) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(item_list(lists, item, rows, col));
#pragma unroll
        for (int k2 = 0; k2 < kListKeys / 2; ++k2) {
          const uint64_t x0 = top[cg].k[2 * k2];
          const uint64_t x1 = 2 * k2 + 1 < kHist ? top[cg].k[2 * k2 + 1] : 0ull;
          dst[k2] = u32x4{(uint32_t)x0, (uint32_t)(x0 >> 32), (uint32_t)x1, (uint32_t)(x1 >> 32)};
        }
      }
    }
  }
}

constexpr int kHead = 4;              // keys per list the merge reads up front

struct MergeSmem {
  uint64_t head[kMergeKeys];  // the lists' first kHead keys
  uint64_t cand[kCandKeys];   // keys at or above a column's bound
  uint64_t thr[64];
  uint32_t ncand[64];
  uint32_t over[64];
};

// One workgroup per request: merge the request's n item lists, for every
// column (row x head), into its 16 output slots.
//
// Any 15 distinct keys bound the 15th best key of the union from below; the
// 15th largest of the lists' top-K keys (K = ceil(15 / n), so 1 once there
// are 15 lists or more) is such a bound, and every key of the final top-15
// is at or above it.  The keys at or above the bound are gathered and ranked
// by counting (keys are distinct).  The first kHead keys of every list come
// in with two 16-byte loads; deeper keys are read only from a list whose
// kHead-th key still reaches the bound.  Columns go in batches that fit the
// LDS arrays; a column whose candidates overflow its share is merged by
// per-lane insertion and a butterfly instead (slower, same result).
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const int32_t *__restrict__ seq_lens, int num_reqs, int query_len, int H, int max_pages,
    const uint8_t *__restrict__ ws, int32_t *__restrict__ out) {
  __shared__ MergeSmem sm;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int rows = query_len * H;
  const uint64_t *lists = reinterpret_cast<const uint64_t *>(ws + lists_offset(num_reqs));
  const int2 info = reinterpret_cast<const int2 *>(ws + kWsHeaderBytes)[r];
  const int first = info.x, n = info.y;
  const int sl = seq_lens[r];
  auto list_ptr = [&](int c, int x) -> const uint64_t * {
    return lists + ((size_t)(first + x) * rows + c) * kListKeys;
  };
  auto emit = [&](int c, int slot, uint64_t v) {
    const int qi = c / H, h = c - (c / H) * H;
    const int64_t T = (int64_t)r * query_len + qi;
    const int p = sl - query_len + qi;
    const int L = p >= 0 ? min(p >> 7, max_pages) : -1;
    out[(T * H + h) * kTopk + slot] = (L >= 0 && v != 0ull) ? key_id(v) : -1;
  };
  const int K = n >= kHist ? 1 : min(kHead, (kHist + n - 1) / max(n, 1));
  const int per_col = max(n * kHead, 1);
  const int batch = max(1, min(rows, min(kMergeKeys / per_col, 64)));
  for (int c0 = 0; c0 < rows; c0 += batch) {
    const int nc = min(batch, rows - c0);
    const int cand_cap = kCandKeys / nc;
    // 1. the first kHead keys of every list
    for (int p = tid; p < nc * n; p += nt) {
      const int cl = p / n, x = p - cl * n;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(list_ptr(c0 + cl, x));
      const u32x4 a = src[0], b = src[1];
      uint64_t *h = sm.head + (size_t)p * kHead;
      h[0] = ((uint64_t)a.y << 32) | a.x;
      h[1] = ((uint64_t)a.w << 32) | a.z;
      h[2] = ((uint64_t)b.y << 32) | b.x;
      h[3] = ((uint64_t)b.w << 32) | b.z;
    }
    for (int c = tid; c < nc; c += nt) {
      sm.thr[c] = 0ull;
      sm.ncand[c] = 0u;
      sm.over[c] = 0u;
    }
    __syncthreads();
    // 2. the bound: the 15th largest of the lists' top-K keys (none if
    // there are fewer than 15 of them)
    for (int p = tid; p < nc * n * K; p += nt) {
      const int cl = p / (n * K), i = p - cl * (n * K);
      const uint64_t *hc = sm.head + (size_t)cl * n * kHead;
      const uint64_t me = hc[(i / K) * kHead + i % K];
      if (me == 0ull) continue;
      int rank = 0;
      for (int x = 0; x < n; ++x)
        for (int k = 0; k < K; ++k) rank += hc[x * kHead + k] > me ? 1 : 0;
      if (rank == kHist - 1) sm.thr[cl] = me;
    }
    __syncthreads();
    // 3. gather every key at or above the bound
    for (int p = tid; p < nc * n; p += nt) {
      const int cl = p / n, x = p - cl * n;
      const uint64_t thr = sm.thr[cl] ? sm.thr[cl] : 1ull;
      const uint64_t *h = sm.head + (size_t)p * kHead;
      int k = 0;
      for (; k < kHead; ++k) {
        const uint64_t v = h[k];
        if (v < thr) break;
        const uint32_t pos = atomicAdd(&sm.ncand[cl], 1u);
        if (pos < (uint32_t)cand_cap) sm.cand[cl * cand_cap + pos] = v;
        else sm.over[cl] = 1u;
      }
      if (k == kHead) {
        const uint64_t *src = list_ptr(c0 + cl, x);
        for (; k < kHist; ++k) {
          const uint64_t v = src[k];
          if (v < thr) break;
          const uint32_t pos = atomicAdd(&sm.ncand[cl], 1u);
          if (pos < (uint32_t)cand_cap) sm.cand[cl * cand_cap + pos] = v;
          else sm.over[cl] = 1u;
        }
      }
    }
    __syncthreads();
    // 4. rank them; slots past the candidates are empty
    for (int p = tid; p < nc * kHist; p += nt) {
      const int cl = p / kHist, k = p - cl * kHist;
      if (!sm.over[cl] && k >= (int)sm.ncand[cl]) emit(c0 + cl, k, 0ull);
    }
    for (int p = tid; p < nc * cand_cap; p += nt) {
      const int cl = p / cand_cap, i = p - cl * cand_cap;
      const int m = (int)sm.ncand[cl];
      if (sm.over[cl] || i >= m) continue;
      const uint64_t *cc = sm.cand + cl * cand_cap;
      const uint64_t me = cc[i];
      int rank = 0;
      for (int b = 0; b < m; ++b) rank += cc[b] > me ? 1 : 0;
      if (rank < kHist) emit(c0 + cl, rank, me);
    }
    // Overflowed columns: one wave, per-lane insertion, then a butterfly.
    if (tid < 64) {
      for (int cl = 0; cl < nc; ++cl) {
        if (!sm.over[cl]) continue;
        TopList acc;
        acc.clear();
        for (int x = tid; x < n; x += 64) {
          const uint64_t *src = list_ptr(c0 + cl, x);
          for (int k = 0; k < kHist; ++k) {
            const uint64_t v = src[k];
            if (v <= acc.threshold()) break;
            acc.insert(v);
          }
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) merge_xor(acc, m);
        if (tid < kHist) {
          uint64_t v = 0ull;
#pragma unroll
          for (int k = 0; k < kHist; ++k) v = (k == tid) ? acc.k[k] : v;
          emit(c0 + cl, tid, v);
        }
      }
    }
    __syncthreads();
  }
  // Slot 15: the local page (-1 for a padding row).
  for (int c = tid; c < rows; c += nt) {
    const int qi = c / H, h = c - (c / H) * H;
    const int64_t T = (int64_t)r * query_len + qi;
    const int p = sl - query_len + qi;
    out[(T * H + h) * kTopk + kHist] = p >= 0 ? min(p >> 7, max_pages) : -1;
  }
}

}  // namespace mi_idx

using namespace mi_idx;

extern "C" size_t mi_idx_decode_plan_bytes(int max_reqs) {
  if (max_reqs < 0) return 0;
  return (size_t)kPlanHeaderInts * 4 + decode_capacity(max_reqs) * kItemInts * 4;
}

extern "C" size_t mi_idx_decode_workspace_bytes(int max_reqs, int query_len, int num_heads) {
  if (max_reqs < 0 || query_len < 1 || num_heads < 1) return 0;
  return lists_offset(max_reqs) + lists_bytes(decode_capacity(max_reqs), query_len * num_heads);
}

static int plan_capacity(size_t plan_bytes) {
  if (plan_bytes < (size_t)kPlanHeaderInts * 4) return 0;
  const size_t c = (plan_bytes - kPlanHeaderInts * 4) / (kItemInts * 4);
  return c > 0x7FFFFFF ? 0x7FFFFFF : (int)c;
}

static int check_decode_sizes(const char *who, int num_reqs, int query_len, int num_heads,
                              int max_pages, size_t plan_bytes, size_t ws_bytes) {
  if (num_reqs < 0) return mi_idx_fail(MI_IDX_EINVAL, "%s: num_reqs %d < 0", who, num_reqs);
  if (query_len < 1 || query_len > MI_IDX_MAX_QUERY_LEN)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "%s: query_len %d outside 1..8", who, query_len);
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "%s: num_heads %d outside 1..8", who, num_heads);
  if (max_pages < 0) return mi_idx_fail(MI_IDX_EINVAL, "%s: max_pages %d < 0", who, max_pages);
  const int cap = plan_capacity(plan_bytes);
  if ((size_t)cap < decode_capacity(num_reqs))
    return mi_idx_fail(MI_IDX_ECAPACITY, "%s: plan_bytes %zu < %zu needed for %d requests", who,
                       plan_bytes, mi_idx_decode_plan_bytes(num_reqs), num_reqs);
  const size_t need = lists_offset(num_reqs) + lists_bytes(cap, query_len * num_heads);
  if (ws_bytes < need)
    return mi_idx_fail(MI_IDX_ECAPACITY, "%s: ws_bytes %zu < %zu needed", who, ws_bytes, need);
  return MI_IDX_OK;
}

extern "C" int mi_idx_plan_decode(const int32_t *seq_lens, int num_reqs, int query_len,
                                  int num_heads, int max_pages, void *plan, size_t plan_bytes,
                                  void *workspace, size_t ws_bytes, void *stream) {
  mi_idx_clear_error();
  int st = check_decode_sizes("plan_decode", num_reqs, query_len, num_heads, max_pages,
                              plan_bytes, ws_bytes);
  if (st) return st;
  if (!plan || !workspace || (num_reqs > 0 && !seq_lens))
    return mi_idx_fail(MI_IDX_EINVAL, "plan_decode: null pointer");
  if (((uintptr_t)plan % 16) || ((uintptr_t)workspace % 16))
    return mi_idx_fail(MI_IDX_EINVAL, "plan_decode: plan and workspace must be 16-byte aligned");
  const int cap = plan_capacity(plan_bytes);
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, seq_lens,
                     num_reqs, max_pages, query_len, cap, query_len * num_heads, (int32_t *)plan,
                     (uint8_t *)workspace);
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
                              plan_bytes, ws_bytes);
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
  const dim3 grid((cap + 3) / 4), block(256);
  hipStream_t s = (hipStream_t)stream;
#define MI_IDX_LAUNCH_DEC(N)                                                                   \
  if (scores_out)                                                                              \
    hipLaunchKernelGGL((decode_score_kernel<N, true>), grid, block, 0, s, q, pages, num_blocks, \
                       block_table, bt_stride, seq_lens, num_reqs, query_len, num_heads,       \
                       max_pages, scale, (const int32_t *)plan, (uint8_t *)workspace,          \
                       scores_out);                                                            \
  else                                                                                         \
    hipLaunchKernelGGL((decode_score_kernel<N, false>), grid, block, 0, s, q, pages,            \
                       num_blocks, block_table, bt_stride, seq_lens, num_reqs, query_len,      \
                       num_heads, max_pages, scale, (const int32_t *)plan,                     \
                       (uint8_t *)workspace, scores_out)
  switch (ncg) {
    case 1: MI_IDX_LAUNCH_DEC(1); break;
    case 2: MI_IDX_LAUNCH_DEC(2); break;
    case 3: MI_IDX_LAUNCH_DEC(3); break;
    default: MI_IDX_LAUNCH_DEC(4); break;
  }
#undef MI_IDX_LAUNCH_DEC
  st = mi_idx_check_launch("score_topk_decode");
  if (st) return st;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(num_reqs), dim3(256), 0, s, seq_lens, num_reqs,
                     query_len, num_heads, max_pages, (const uint8_t *)workspace, topk_out);
  return mi_idx_check_launch("score_topk_decode (merge)");
}
