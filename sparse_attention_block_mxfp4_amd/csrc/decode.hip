// Decode: device-side work-map plan, fused page scoring with a per-wave
// top-15, and a per-request merge into the [T, H, 16] output.
//
// Plan (one workgroup): history pages of request r are 0..hist_r-1 with
// hist_r = (seq_len_r - 1) / 128 (the last query's local page bounds every
// row of the request), clamped to max_pages.  A chunk size is picked so that
// the whole batch splits into at most as many equal work items (at least
// kMinChunk pages each) as the scorer can hold resident at once -- a second
// round of items would double the tail; every request gets max(1,
// ceil(hist_r / chunk_r)) items, each one wave's worth of work, with chunk_r
// = chunk raised where needed so that no request has more than
// kMaxItemsPerReq items.  Items = (request, first page, end
// page); the request's first item and item count go to the workspace.
//
// Score (8 or 4 independent waves per workgroup, one item each): a wave streams
// its pages through the MFMA with the request's query rows as the B operand,
// reduces each page to its max over tokens, keeps a running top-15 per query
// column in registers and writes the lists to the workspace.
//
// Merge (one wave per request column, a second launch on the same stream, so
// the lists written by every XCD are visible without device-wide fences):
// merges the request's item lists into the 16 output slots of every row.
#include <atomic>
#include <cmath>
#include <mutex>

#include "common.h"

namespace mi_idx {

constexpr int kTargetItems = 2048;    // ~8 waves per CU
constexpr int kMinChunk = 4;
constexpr int kPlanHeaderInts = 16;
constexpr int kItemInts = 4;
constexpr size_t kWsHeaderBytes = 256;
constexpr int kListKeys = 16;         // 15 keys + an empty slot: 128-byte lists
constexpr int kDepth = 2;             // pages in flight per wave (register ring)
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

constexpr int kPlanThreads = 256;

__device__ __forceinline__ long long wave_sum(long long v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ long long wave_inclusive_scan(long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long u = __shfl_up(v, off, 64);
    v += lane >= off ? u : 0;
  }
  return v;
}

__device__ __forceinline__ int history_of(const int32_t *seq_lens, int r, int max_pages) {
  const int sl = seq_lens[r];
  return min(sl >= 1 ? (sl - 1) >> 7 : 0, max_pages);
}

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(
    const int32_t *__restrict__ seq_lens, int num_reqs, int max_pages, int query_len,
    int capacity, int rows, int resident, int32_t *__restrict__ plan, uint8_t *__restrict__ ws) {
  constexpr int kWaves = kPlanThreads / 64;
  __shared__ long long s_wave[2][kWaves];
  __shared__ long long s_first[kPlanThreads];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int2 *req_info = reinterpret_cast<int2 *>(ws + kWsHeaderBytes);
  // Contiguous segment of requests per thread.
  const int per = (num_reqs + kPlanThreads - 1) / kPlanThreads;
  const int r0 = min(num_reqs, tid * per), r1 = min(num_reqs, r0 + per);
  long long hsum = 0;
  int over = 0;   // a request whose history goes past max_pages block-table columns
  for (int r = r0; r < r1; ++r) {
    hsum += history_of(seq_lens, r, max_pages);
    const int sl = seq_lens[r];
    over |= sl >= 1 && ((sl - 1) >> 7) > max_pages;
  }
  hsum = wave_sum(hsum);
  if (lane == 0) s_wave[0][wave] = hsum;
  over = __syncthreads_or(over);
  long long total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += s_wave[0][w];
  // each request rounds its item count up by less than one, so aiming at
  // resident - num_reqs items keeps the total within what runs at once
  const long long aim = max((long long)resident / 2, (long long)resident - num_reqs);
  const int chunk = (int)max((long long)kMinChunk, (total + aim - 1) / aim);
  auto chunk_of = [&](int h) {
    return max(chunk, (h + kMaxItemsPerReq - 1) / kMaxItemsPerReq);
  };
  // Item counts and their exclusive scan over the thread segments.
  long long cnt = 0;
  for (int r = r0; r < r1; ++r) {
    const int h = history_of(seq_lens, r, max_pages);
    const int c = chunk_of(h);
    cnt += max(1, (h + c - 1) / c);
  }
  const long long incl = wave_inclusive_scan(cnt);
  if (lane == 63) s_wave[1][wave] = incl;
  __syncthreads();
  long long first = incl - cnt, total_items = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    first += w < wave ? s_wave[1][w] : 0;
    total_items += s_wave[1][w];
  }
  int4 *items = reinterpret_cast<int4 *>(plan + kPlanHeaderInts);
  if (per == 1) {
    // One request per thread: the request's items are written by a team of
    // tpr threads (consecutive threads, consecutive items), so the stores
    // are spread over every wave and coalesced.
    if (tid < num_reqs) {
      const int h = history_of(seq_lens, tid, max_pages);
      const int c = chunk_of(h);
      const int n = max(1, (h + c - 1) / c);
      s_first[tid] = first;
      req_info[tid] = make_int2((int)first, n);
    }
    __syncthreads();
    int tpr = 1;
    while (tpr * 2 * num_reqs <= kPlanThreads) tpr *= 2;
    const int r = tid / tpr, sub = tid - r * tpr;
    if (r < num_reqs) {
      const int h = history_of(seq_lens, r, max_pages);
      const int c = chunk_of(h);
      const int n = max(1, (h + c - 1) / c);
      const long long f = s_first[r];
      for (int i = sub; i < n; i += tpr) {
        const long long it = f + i;
        if (it < capacity) items[it] = make_int4(r, min(h, i * c), min(h, (i + 1) * c), 0);
      }
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      const int h = history_of(seq_lens, r, max_pages);
      const int c = chunk_of(h);
      const int n = max(1, (h + c - 1) / c);
      for (int i = 0; i < n; ++i) {
        const long long it = first + i;
        if (it < capacity) items[it] = make_int4(r, min(h, i * c), min(h, (i + 1) * c), 0);
      }
      req_info[r] = make_int2((int)first, n);
      first += n;
    }
  }
  if (tid == 0) {
    plan[0] = (int)min(total_items, (long long)capacity);
    plan[1] = chunk;
    plan[2] = num_reqs;
    plan[3] = query_len;
    plan[4] = max_pages;
    plan[5] = capacity;
    // error bits: 1 = plan overflow, 2 = rows refused for a history past max_pages
    reinterpret_cast<uint32_t *>(ws)[0] = (total_items > capacity ? 2u : 0u) | (over ? 4u : 0u);
  }
}

__device__ __forceinline__ uint64_t *item_list(uint64_t *lists, int item, int rows, int col) {
  return lists + ((size_t)item * rows + col) * kListKeys;
}

// kBf16: the query is bfloat16 (256 bytes per row and head) and the tiles run
// on the bf16 MFMA (see mfma_fp4_bf16); otherwise E4M3 (128 bytes).
// Waves per scorer workgroup: with up to 2 column groups a wave fits in half
// a SIMD's registers and a CU holds 8 waves, launched as one workgroup of 8
// (half the workgroups of two 4-wave ones; the decode batch's phase measured
// 3 % faster); with more, a CU holds 4, one workgroup.
template <int NCG>
constexpr int score_wg_waves() { return NCG <= 2 ? 8 : 4; }

template <int NCG, bool kScores, bool kBf16>
__global__ __launch_bounds__(64 * score_wg_waves<NCG>()) void decode_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, int num_reqs, int query_len, int H, int max_pages,
    float scale, const int32_t *__restrict__ plan, uint8_t *__restrict__ ws,
    float *__restrict__ scores_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int item = blockIdx.x * score_wg_waves<NCG>() + (tid >> 6);
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
  u32x4 bqh[kBf16 ? NCG : 1][4];
  int Lc[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int col = cg * 16 + t16;
    Lc[cg] = -1;
    bq[cg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (kBf16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) bqh[cg][k] = u32x4{0u, 0u, 0u, 0u};
    }
    if (col < rows) {
      const int i = col / H, h = col - (col / H) * H;
      const int64_t T = (int64_t)r * query_len + i;
      if constexpr (kBf16) {
        load_q_bf16(q + (T * H + h) * (2 * kDim), g, bqh[cg]);
      } else {
        const uint8_t *qp = q + (T * H + h) * kDim;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(qp + 16 * g);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(qp + 64 + 16 * g);
        bq[cg] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      const int p = sl - query_len + i;
      Lc[cg] = local_page(p, max_pages);
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
              m[cg] = nmax(m[cg], max4(kBf16 ? mfma_fp4_bf16(a[u][tile], bqh[kBf16 ? cg : 0], s[u][tile])
                                              : mfma_fp4_fp8(a[u][tile], bq[cg], s[u][tile])));
          }
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            float v = m[cg];
            v = nmax(v, __shfl_xor(v, 16, 64));
            v = nmax(v, __shfl_xor(v, 32, 64));
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

constexpr int kHead = 4;                              // keys per list read up front
constexpr int kMergeWaves = 4;                        // columns per merge workgroup
constexpr int kListsPerLane = kMaxItemsPerReq / 64;   // a request's lists over 64 lanes
constexpr int kFlatKeys = 256;                        // >= n * K for every n <= 256
constexpr int kCandCap = 256;                         // > 15 lists x 15 keys

struct __align__(16) MergeWaveSmem {   // 16-byte aligned pair reads
  uint64_t flat[kFlatKeys + 2];   // top-K keys of every list (+ zero padding)
  uint64_t cand[kCandCap + 2];    // keys at or above the bound (+ zero padding)
  uint64_t thr;
  uint32_t ncand;
};

__device__ __forceinline__ uint64_t key_lo(const u32x4 &q) {
  return ((uint64_t)q.y << 32) | q.x;
}
__device__ __forceinline__ uint64_t key_hi(const u32x4 &q) {
  return ((uint64_t)q.w << 32) | q.z;
}

// Orders one wave's LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Number of keys in flat[0, n2) (n2 even, zero padded) greater than me.
__device__ __forceinline__ int rank_in(const uint64_t *flat, int n2, uint64_t me) {
  int rank = 0;
#pragma unroll 4
  for (int j = 0; j < n2; j += 2) {
    const u32x4 q = *reinterpret_cast<const u32x4 *>(flat + j);
    rank += (key_lo(q) > me ? 1 : 0) + (key_hi(q) > me ? 1 : 0);
  }
  return rank;
}

// One wave per column (row x head) of request blockIdx.x: merge the
// request's n item lists (n <= 256, sorted, keys distinct across lists
// because the items cover disjoint pages) into the 16 output slots.
//
// Any 15 distinct keys bound the 15th best key of the union from below; the
// 15th largest of the lists' top-K keys (K = 4 for up to 16 lists, else 1)
// is such a bound, and every key of the final top-15 is at or above it.
// Only lists whose first key reaches the bound hold such keys, and there are
// at most 15 of them (their first keys are among the 15 largest of the
// top-K keys), so at most 225 candidates exist; they are gathered and ranked by counting.  When fewer
// than 15 of the top-K keys are non-empty, every non-empty key is gathered
// (at most 14 non-empty lists x 15).  Lane x holds lists x, x+64, ...: their
// first four keys come in with two 16-byte loads, the rest only for a list
// whose fourth key still reaches the bound.
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(
    const int32_t *__restrict__ seq_lens, int num_reqs, int query_len, int H, int max_pages,
    const uint8_t *__restrict__ ws, int32_t *__restrict__ out) {
  __shared__ MergeWaveSmem smem[kMergeWaves];
  const int r = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = query_len * H;
  const int c = blockIdx.y * kMergeWaves + wave;
  if (c >= rows) return;   // whole waves only; no workgroup barrier follows
  MergeWaveSmem &sm = smem[wave];
  const int qi = c / H, h = c - qi * H;
  const int64_t T = (int64_t)r * query_len + qi;
  // The request's item range is read together with its length (one round
  // trip, not two); it is used only for a row with a local page.
  const int2 info = reinterpret_cast<const int2 *>(ws + kWsHeaderBytes)[r];
  const int sl = seq_lens[r];
  asm volatile("" :: "s"(info.x), "s"(info.y), "s"(sl));
  const int p = sl - query_len + qi;
  const int L = local_page(p, max_pages);
  int32_t *dst = out + (T * H + h) * kTopk;
  if (L < 0) {   // a padding or refused row: every slot empty
    if (lane < kTopk) dst[lane] = -1;
    return;
  }
  const uint64_t *lists = reinterpret_cast<const uint64_t *>(ws + lists_offset(num_reqs));
  const int first = info.x, n = max(1, min(info.y, kMaxItemsPerReq));
  auto list_of = [&](int x) -> const u32x4 * {
    return reinterpret_cast<const u32x4 *>(lists + ((size_t)(first + x) * rows + c) * kListKeys);
  };
  // 1. the first four keys of every list
  u32x4 a[kListsPerLane], b[kListsPerLane];
#pragma unroll
  for (int j = 0; j < kListsPerLane; ++j) {
    const u32x4 *src = list_of(min(lane + 64 * j, n - 1));
    a[j] = src[0];
    b[j] = src[1];
  }
  // Keys per list behind the bound: all four loaded ones for up to 16 lists
  // (a tight bound: few candidates, few lists read further), the first for
  // more (the bound's own ranking would cost more than it saves).
  const int K = n <= 16 ? kHead : 1;
  const int nK = n * K;
#pragma unroll
  for (int j = 0; j < kListsPerLane; ++j) {
    const int x = lane + 64 * j;
    if (x < n) {
      uint64_t *f = sm.flat + x * K;
      f[0] = key_lo(a[j]);
      if (K > 1) f[1] = key_hi(a[j]);
      if (K > 2) f[2] = key_lo(b[j]);
      if (K > 3) f[3] = key_hi(b[j]);
    }
  }
  if (lane == 0) {
    sm.flat[nK] = 0ull;
    sm.thr = 0ull;
    sm.ncand = 0u;
  }
  wave_lds_sync();
  // 2. the bound: the key of rank 14 among the top-K keys, if non-empty
  const int nK2 = (nK + 1) & ~1;
  for (int i = lane; i < nK; i += 64) {
    const uint64_t me = sm.flat[i];
    if (me != 0ull && rank_in(sm.flat, nK2, me) == kHist - 1) sm.thr = me;
  }
  wave_lds_sync();
  const uint64_t thr = sm.thr ? sm.thr : 1ull;
  // 3. gather every key at or above the bound
  auto push = [&](uint64_t v) {
    const uint32_t pos = atomicAdd(&sm.ncand, 1u);
    if (pos < (uint32_t)kCandCap) sm.cand[pos] = v;
  };
#pragma unroll
  for (int j = 0; j < kListsPerLane; ++j) {
    const int x = lane + 64 * j;
    bool live = x < n;
    const uint64_t head[kHead] = {key_lo(a[j]), key_hi(a[j]), key_lo(b[j]), key_hi(b[j])};
#pragma unroll
    for (int k = 0; k < kHead; ++k) {
      live = live && head[k] >= thr;
      if (live) push(head[k]);
    }
    if (live) {
      const u32x4 *src = list_of(x) + 2;   // keys 4..15
      u32x4 w[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) w[i] = src[i];
#pragma unroll
      for (int k = 0; k < kHist - kHead; ++k) {
        const uint64_t v = (k & 1) ? key_hi(w[k >> 1]) : key_lo(w[k >> 1]);
        live = live && v >= thr;
        if (live) push(v);
      }
    }
  }
  wave_lds_sync();
  const int m = min((int)sm.ncand, kCandCap);
  if (lane == 0) sm.cand[m] = 0ull;
  wave_lds_sync();
  // 4. rank the candidates; slots past them are empty; slot 15 is the local page
  const int m2 = (m + 1) & ~1;
  for (int i = lane; i < m; i += 64) {
    const uint64_t me = sm.cand[i];
    const int rank = rank_in(sm.cand, m2, me);
    if (rank < kHist) dst[rank] = key_id(me);
  }
  if (lane >= m && lane < kHist) dst[lane] = -1;
  if (lane == kHist) dst[kHist] = L;
}

}  // namespace mi_idx

using namespace mi_idx;

extern "C" size_t mi_idx_decode_plan_bytes(int max_reqs) {
  if (max_reqs < 0) return 0;
  return (size_t)kPlanHeaderInts * 4 + decode_capacity(max_reqs) * kItemInts * 4;
}

extern "C" size_t mi_idx_decode_plan_capacity(int max_reqs, int max_pages, int query_len,
                                              int num_heads) {
  if (max_reqs < 0 || max_pages < 0 || query_len < 1 || query_len > MI_IDX_MAX_QUERY_LEN ||
      num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return 0;
  return decode_capacity(max_reqs);
}

extern "C" size_t mi_idx_decode_workspace_bytes(int max_reqs, int query_len, int num_heads) {
  if (max_reqs < 0 || query_len < 1 || num_heads < 1) return 0;
  return lists_offset(max_reqs) + lists_bytes(decode_capacity(max_reqs), query_len * num_heads);
}

// Waves of the decode scorer (one item each) that the device holds at once
// for `rows` query columns, capped at kTargetItems (the plan capacity per
// batch).  The plan knows neither the query dtype nor whether scores are
// written, so it takes the lowest occupancy of the four instantiations for
// the column group count; once per device and count.
template <int N>
static hipError_t min_score_blocks(int *blocks) {
  int b[4] = {0, 0, 0, 0};
  constexpr int kT = 64 * score_wg_waves<N>();
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[0], decode_score_kernel<N, false, false>, kT, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[1], decode_score_kernel<N, true, false>, kT, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[2], decode_score_kernel<N, false, true>, kT, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[3], decode_score_kernel<N, true, true>, kT, 0);
  // waves per CU
  *blocks = min(min(b[0], b[1]), min(b[2], b[3])) * score_wg_waves<N>();
  return e;
}

static int resident_items(int rows) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][5];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kTargetItems;
  }
  const int ncg = min(max((rows + 15) / 16, 1), 4);
  const int hit = cache[dev][ncg].load(std::memory_order_relaxed);
  if (hit > 0) return hit;
  int blocks = 0, cus = 0;
  hipError_t e = hipSuccess;
  switch (ncg) {
    case 1: e = min_score_blocks<1>(&blocks); break;
    case 2: e = min_score_blocks<2>(&blocks); break;
    case 3: e = min_score_blocks<3>(&blocks); break;
    default: e = min_score_blocks<4>(&blocks); break;
  }
  if (e != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return kTargetItems;
  }
  const long long waves = (long long)blocks * cus;
  const int r = waves > 0 ? (int)min(waves, (long long)kTargetItems) : kTargetItems;
  cache[dev][ncg].store(r, std::memory_order_relaxed);
  return r;
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

// The decode plan kernel on `plan` (capacity items) and `ws`; arguments
// already checked.
static int launch_plan(const int32_t *seq_lens, int num_reqs, int query_len, int num_heads,
                       int max_pages, int32_t *plan, int cap, uint8_t *ws, hipStream_t s) {
  const int resident = resident_items(query_len * num_heads);
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, seq_lens, num_reqs,
                     max_pages, query_len, cap, query_len * num_heads, resident, plan, ws);
  return mi_idx_check_launch("plan_decode");
}

// The scorer and the merge on a plan of `cap` items; arguments already
// checked.
static int launch_score(const uint8_t *qb, int q_dtype, const uint8_t *pages,
                        int64_t num_blocks, const int32_t *block_table, int64_t bt_stride,
                        const int32_t *seq_lens, int num_reqs, int query_len, int num_heads,
                        int max_pages, float scale, const int32_t *plan, int cap, uint8_t *ws,
                        int32_t *topk_out, float *scores_out, hipStream_t s) {
  const int rows = query_len * num_heads;
  const int ncg = (rows + 15) / 16;
#define MI_IDX_LAUNCH_DEC1(N, SC, BF)                                                          \
  hipLaunchKernelGGL((decode_score_kernel<N, SC, BF>),                                         \
                     dim3((cap + score_wg_waves<N>() - 1) / score_wg_waves<N>()),              \
                     dim3(64 * score_wg_waves<N>()), 0, s, qb, pages,                          \
                     num_blocks, block_table, bt_stride, seq_lens, num_reqs, query_len,        \
                     num_heads, max_pages, scale, plan, ws, scores_out)
#define MI_IDX_LAUNCH_DEC(N)                                                                   \
  if (q_dtype == MI_IDX_Q_BF16) {                                                              \
    if (scores_out) MI_IDX_LAUNCH_DEC1(N, true, true);                                         \
    else MI_IDX_LAUNCH_DEC1(N, false, true);                                                   \
  } else {                                                                                     \
    if (scores_out) MI_IDX_LAUNCH_DEC1(N, true, false);                                        \
    else MI_IDX_LAUNCH_DEC1(N, false, false);                                                  \
  }
  switch (ncg) {
    case 1: MI_IDX_LAUNCH_DEC(1); break;
    case 2: MI_IDX_LAUNCH_DEC(2); break;
    case 3: MI_IDX_LAUNCH_DEC(3); break;
    default: MI_IDX_LAUNCH_DEC(4); break;
  }
#undef MI_IDX_LAUNCH_DEC
#undef MI_IDX_LAUNCH_DEC1
  int st = mi_idx_check_launch("score_topk_decode");
  if (st) return st;
  hipLaunchKernelGGL(decode_merge_kernel,
                     dim3(num_reqs, (rows + kMergeWaves - 1) / kMergeWaves),
                     dim3(64 * kMergeWaves), 0, s, seq_lens, num_reqs, query_len, num_heads,
                     max_pages, ws, topk_out);
  return mi_idx_check_launch("score_topk_decode (merge)");
}

// Checks of a score call's own arguments (the plan and workspace sizes are
// checked by the caller).
static int check_score_args(const char *who, const void *q, int q_dtype, const uint8_t *pages,
                            int64_t num_blocks, const int32_t *block_table, int64_t bt_stride,
                            const int32_t *seq_lens, int max_pages, float scale,
                            const int32_t *topk_out) {
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return mi_idx_fail(MI_IDX_EINVAL, "%s: scale must be positive and finite", who);
  if (q_dtype != MI_IDX_Q_E4M3 && q_dtype != MI_IDX_Q_BF16)
    return mi_idx_fail(MI_IDX_EINVAL, "%s: q_dtype %d is neither E4M3 (0) nor bf16 (1)", who,
                       q_dtype);
  if (!q || !pages || !block_table || !seq_lens || !topk_out)
    return mi_idx_fail(MI_IDX_EINVAL, "%s: null pointer", who);
  if (((uintptr_t)q % 16) || ((uintptr_t)pages % 16) || ((uintptr_t)topk_out % 16))
    return mi_idx_fail(MI_IDX_EINVAL, "%s: q, pages and topk_out must be 16-byte aligned", who);
  if (num_blocks <= 0) return mi_idx_fail(MI_IDX_EINVAL, "%s: num_blocks <= 0", who);
  if (bt_stride < max_pages)
    return mi_idx_fail(MI_IDX_EINVAL, "%s: bt_stride %lld < max_pages %d", who,
                       (long long)bt_stride, max_pages);
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
  return launch_plan(seq_lens, num_reqs, query_len, num_heads, max_pages, (int32_t *)plan,
                     plan_capacity(plan_bytes), (uint8_t *)workspace, (hipStream_t)stream);
}

extern "C" int mi_idx_score_topk_decode(const void *q, int q_dtype, const uint8_t *pages,
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
  if (q_dtype != MI_IDX_Q_E4M3 && q_dtype != MI_IDX_Q_BF16)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: q_dtype %d is neither E4M3 (0) nor "
                                      "bf16 (1)", q_dtype);
  if (num_reqs == 0) return MI_IDX_OK;
  st = check_score_args("score_topk_decode", q, q_dtype, pages, num_blocks, block_table,
                        bt_stride, seq_lens, max_pages, scale, topk_out);
  if (st) return st;
  if (!plan || !workspace)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: null pointer");
  if (((uintptr_t)workspace % 16) || ((uintptr_t)plan % 16))
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_decode: plan and workspace must be 16-byte "
                                      "aligned");
  return launch_score(static_cast<const uint8_t *>(q), q_dtype, pages, num_blocks, block_table,
                      bt_stride, seq_lens, num_reqs, query_len, num_heads, max_pages, scale,
                      (const int32_t *)plan, plan_capacity(plan_bytes), (uint8_t *)workspace,
                      topk_out, scores_out, (hipStream_t)stream);
}

// ------------------------------------------------------- allocation-free --
// Plan + score + merge with the plan and the workspace in one file-scope
// device array instead of caller buffers.  Host code never passes the
// array's name to a kernel (in host code it is a host-side stand-in, not a
// device address): the device address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) uint8_t scratch[MI_IDX_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64];

static int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return mi_idx_fail(MI_IDX_EHIP, "decode_noalloc: no current device: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= 64)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "decode_noalloc: device %d beyond the 64 served", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return mi_idx_fail(MI_IDX_EHIP, "decode_noalloc: hipGetSymbolAddress failed: %s",
                         hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MI_IDX_OK;
}

extern "C" int mi_idx_decode_noalloc(const void *q, int q_dtype, const uint8_t *pages,
                                     int64_t num_blocks, const int32_t *block_table,
                                     int64_t bt_stride, const int32_t *seq_lens, int num_reqs,
                                     int query_len, int num_heads, int max_pages, float scale,
                                     int32_t *topk_out, float *scores_out, void *stream) {
  mi_idx_clear_error();
  if (num_reqs < 0) return mi_idx_fail(MI_IDX_EINVAL, "decode_noalloc: num_reqs %d < 0", num_reqs);
  if (query_len < 1 || query_len > MI_IDX_MAX_QUERY_LEN)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "decode_noalloc: query_len %d outside 1..8", query_len);
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "decode_noalloc: num_heads %d outside 1..8", num_heads);
  if (max_pages < 0) return mi_idx_fail(MI_IDX_EINVAL, "decode_noalloc: max_pages %d < 0", max_pages);
  const size_t plan_bytes = mi_idx_decode_plan_bytes(num_reqs);
  const size_t plan_region = (plan_bytes + 255) & ~(size_t)255;
  const size_t ws_bytes = mi_idx_decode_workspace_bytes(num_reqs, query_len, num_heads);
  if (plan_region + ws_bytes > (size_t)MI_IDX_NOALLOC_SCRATCH_BYTES)
    return mi_idx_fail(MI_IDX_ECAPACITY, "decode_noalloc: %d requests x %d query columns need "
                       "%zu scratch bytes, above the %d-byte static scratch", num_reqs,
                       query_len * num_heads, plan_region + ws_bytes,
                       MI_IDX_NOALLOC_SCRATCH_BYTES);
  int st = check_score_args("decode_noalloc", q, q_dtype, pages, num_blocks, block_table,
                            bt_stride, seq_lens, max_pages, scale, topk_out);
  if (st) return st;
  if (num_reqs == 0) return MI_IDX_OK;
  void *base = nullptr;
  st = scratch_address(&base);
  if (st) return st;
  int32_t *plan = static_cast<int32_t *>(base);
  uint8_t *ws = static_cast<uint8_t *>(base) + plan_region;
  const int cap = plan_capacity(plan_bytes);
  hipStream_t s = (hipStream_t)stream;
  st = launch_plan(seq_lens, num_reqs, query_len, num_heads, max_pages, plan, cap, ws, s);
  if (st) return st;
  return launch_score(static_cast<const uint8_t *>(q), q_dtype, pages, num_blocks, block_table,
                      bt_stride, seq_lens, num_reqs, query_len, num_heads, max_pages, scale, plan,
                      cap, ws, topk_out, scores_out, s);
}
