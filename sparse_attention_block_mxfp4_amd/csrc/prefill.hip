// Prefill: host-side tile plan + fused page scoring and top-16.
//
// A workgroup owns a tile of M consecutive query rows of one request and all
// H heads: 256 query columns (column = row * H + head), 64 per wave, so each
// wave holds four 16-column MFMA B operands in registers for the whole tile.
// The tile walks its causal pages 0..L_max-1 in two interleaved page
// streams of four waves each; each page (8704 bytes) is staged once into LDS
// -- a ring of four buffers per stream, two pages per barrier, the next two
// pages' global loads in flight while the current two are consumed -- and
// re-read by the stream's four waves as the MFMA A operand.  At the end the
// two streams' lists are merged in LDS; rows never cross workgroups, so a
// column's top-15 is final then: no merge pass.
#include <algorithm>
#include <cmath>
#include <vector>

#include "common.h"

namespace mi_idx {

constexpr int kTileCols = 256;          // query columns per workgroup
constexpr int kPreHeaderInts = 16;
constexpr int kChunks = kPageBytes / 16;                    // 544 16-byte chunks
constexpr int kXcds = 8;                // MI355X accelerator complex dies
constexpr int kPrefillCgw = 4;          // 16-column groups per wave
constexpr int kPrefillStreams = 2;      // page streams per workgroup
constexpr int kQueue = 16;              // per-column key queue (LDS)
constexpr int kBufs = 4;                // LDS page buffers per stream

inline int rows_per_tile(int H) { return kTileCols / H; }

// Plan header (int32): [0] tile count, [1] rows per tile, [2] num_heads,
// [3] chunk count.  Tile (int4): request, first row (in the request), row
// count, page upper bound.

// Token of a page that MFMA row t16 of tile tl reads.  A page's score is a
// max over its tokens, so any assignment that covers the 128 tokens once is
// correct; the one chosen spreads a tile's LDS reads (dword 17*token + 4*g)
// over distinct banks.
__device__ __forceinline__ int page_token(int tl, int t16) {
  return 32 * (tl >> 1) + 8 * (t16 >> 2) + 4 * (tl & 1) + (t16 & 3);
}

// CGW = 16-column MFMA groups per wave: 16 / CGW waves cover the tile's
// kTileCols = 256 query columns.  NS page streams of such wave sets share the
// workgroup: stream s walks pages s, s + NS, s + 2 NS, ... with LDS buffers of
// its own, so a SIMD holds NS waves that interleave MFMA, VALU and waits.  At
// the end the streams' lists are merged through LDS by stream 0.
// kBf16: bfloat16 query (256 bytes per row and head) on the bf16 MFMA (see
// mfma_fp4_bf16); otherwise E4M3.
template <int CGW, int NS, bool kScores, bool kBf16>
__global__ __launch_bounds__(64 * NS * (16 / CGW)) void prefill_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ cu_seqlens_q, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ context_lens, int num_reqs, int64_t total_q, int H,
    int max_pages, float scale, const int32_t *__restrict__ plan, int32_t *__restrict__ out,
    float *__restrict__ scores_out) {
  constexpr int NW = 16 / CGW;                       // waves per stream
  constexpr int NT = 64 * NW;                        // threads per stream
  constexpr int kLoads = (kChunks + NT - 1) / NT;    // 16-byte chunks per thread
  static_assert(NS >= 1 && NS <= 2, "one or two page streams");
  static_assert(NS == 1 || kHist * NT * 8 <= NS * kBufs * kPageBytes,
                "the stream merge reuses the page buffers");
  // kBufs LDS page buffers per stream (a ring: two pages read per block while
  // the next two are written), each in the page's global byte layout (token
  // t at 68*t; +16 bytes: the landing slot of the threads that have no chunk
  // to write).
  __shared__ __attribute__((aligned(16))) uint8_t s_page[NS][kBufs][kPageBytes + 16];
  // Each stream's current 15th key per column, double-buffered by block
  // parity: block b writes slot b & 1 and reads the partner's slot written in
  // block b-1 (a barrier apart).  Keys are distinct, so a key at or below the
  // partner's 15th key has 15 better keys there and cannot be in the final
  // top-15: the partner's bound filters this stream's pushes.
  __shared__ uint64_t s_floor[NS == 2 ? 2 : 1][NS][NS == 2 ? 64 * (16 / CGW) : 1];
  // Keys waiting to enter a column's list: a queue per thread, entry i of
  // thread t at [i][t] (consecutive lanes, consecutive words).
  __shared__ uint64_t s_queue[kQueue][NS * 64 * (16 / CGW)];
  // Drain requests, double-buffered by block parity: at the end of a block a
  // wave whose queues may fill up in the next block posts a flag byte; at the
  // start of that block every wave of the workgroup drains, so one slow
  // block serves all waves (the block barrier would make the others wait
  // anyway).  The 8 bytes of a parity are read as one word.
  static_assert(NS * (16 / CGW) <= 8, "one flag byte per wave");
  __shared__ __attribute__((aligned(8))) uint8_t s_need[2][8];

  if ((int)blockIdx.x >= plan[0]) return;
  const int4 tile = reinterpret_cast<const int4 *>(plan + kPreHeaderInts)[blockIdx.x];
  const int r = tile.x, row0 = tile.y, nrows = tile.z;
  if (r < 0 || r >= num_reqs) return;
  // wave-uniform (page indices derived from it stay scalar)
  const int stream = NS == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
  const int tid = (int)threadIdx.x - stream * NT;    // thread within its stream
  const int wave = tid >> 6, lane = tid & 63;
  const int t16 = lane & 15, g = lane >> 4;
  const int ctx = context_lens[r];
  const int sl = seq_lens[r];
  const int64_t q0 = cu_seqlens_q[r];

  // B operands: columns (wave*CGW + cg)*16 + t16.
  v8i bq[kBf16 ? 1 : CGW];
  u32x4 bqh[kBf16 ? CGW : 1][4];
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    const int col = (wave * CGW + cg) * 16 + t16;
    const int rl = col / H, h = col - rl * H;
    if constexpr (kBf16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) bqh[cg][k] = u32x4{0u, 0u, 0u, 0u};
    } else {
      bq[cg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (rl < nrows) {
      const int64_t T = q0 + row0 + rl;
      if (T < total_q) {
        if constexpr (kBf16) {
          load_q_bf16(q + (T * H + h) * (2 * kDim), g, bqh[cg]);
        } else {
          const uint8_t *qp = q + (T * H + h) * kDim;
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(qp + 16 * g);
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(qp + 64 + 16 * g);
          bq[cg] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
    }
  }
  // One 16x16x128 tile of column group cg.
  auto tile_mfma = [&](const u32x4 &a, int cg, uint32_t sc) -> v4f {
    if constexpr (kBf16) return mfma_fp4_bf16(a, bqh[cg], sc);
    else return mfma_fp4_fp8(a, bq[cg], sc);
  };
  // The column this lane owns after the page-max reduction: with 4 groups
  // per wave each lane group owns one; with 2, lane groups g and g^1 both
  // hold group g>>1 (the even one writes it); with 1, all hold it.
  const int my_cg = CGW == 4 ? g : (CGW == 2 ? (g >> 1) : 0);
  const bool writer = CGW == 4 ? true : (CGW == 2 ? (g & 1) == 0 : g == 0);
  const int mycol = (wave * CGW + my_cg) * 16 + t16;
  const int my_rl = mycol / H, my_h = mycol - my_rl * H;
  const int64_t myT = q0 + row0 + my_rl;
  int myL = -1;
  if (my_rl < nrows && myT < total_q) {
    const int p = ctx + row0 + my_rl;
    myL = (p >= 0 && p < sl) ? min(p >> 7, max_pages) : -1;
  }
  // Pages walked by the tile: every row's history is a prefix of 0..J-1.
  int J = 0;
  {
    const int plast = ctx + row0 + nrows - 1;
    J = plast >= 0 ? min(plast >> 7, max_pages) : 0;
    J = max(J, 0);
  }
  // The column's top-15 (registers) and its queue (LDS): a key that beats
  // the list's 15th key (and the partner stream's) is appended to the queue
  // with no branch -- the write always happens, the count moves only for a
  // qualifying key -- and queues are drained into the lists rarely, each
  // wave running as many insertions as its fullest queue holds.
  TopList top;
  top.clear();
  int nq = 0;
  const int qslot = stream * NT + tid;

  // Page pipeline (per stream; step s is the stream's s-th page).  The
  // 16-byte chunks of step s are loaded into register slot s & 1 (kLoads
  // chunks per thread), copied into LDS buffer s & 3 a block later, and read
  // there by the stream's four waves in the block after that: while a block
  // consumes two pages, the next two sit in registers (then LDS) and the two
  // after them are in flight.  Every load is unconditional (chunk and page
  // indices are clamped, an invalid page id reads page 0 and is skipped), and
  // the barriers order LDS only, so the global loads stay in flight across
  // them.
  const int32_t *bt = block_table + (int64_t)r * bt_stride;
  const int jlast = J - 1;
  static_assert(kLoads >= 1 && kLoads <= 3, "page staging takes 1..3 chunks per thread");
  // slot 0 (even pages): e0..e2, slot 1 (odd pages): o0..o2
  uint4 e0, e1, e2, o0, o1, o2;
  // Validity of the page of step s (bit s & 63), recorded when the page is
  // issued; a step's page is taken 4 steps after its issue, long before the
  // bit is reused 64 steps later.  Wave-uniform, so it lives in SGPRs.
  uint64_t vmask = 0;
  // This thread's chunks of a page: byte offsets in global memory (the last
  // chunk re-read by threads past it) and in an LDS buffer (the landing slot
  // for those threads); loop-invariant.
  const uint32_t goff0 = 16u * (uint32_t)min(tid, kChunks - 1);
  const uint32_t goff1 = 16u * (uint32_t)min(tid + NT, kChunks - 1);
  const uint32_t goff2 = 16u * (uint32_t)min(tid + 2 * NT, kChunks - 1);
  const uint32_t loff0 = 16u * (uint32_t)min(tid, kChunks);
  const uint32_t loff1 = 16u * (uint32_t)min(tid + NT, kChunks);
  const uint32_t loff2 = 16u * (uint32_t)min(tid + 2 * NT, kChunks);
  // Block-table entry of a step (clamped like the page index).
  auto bt_entry = [&](int step) { return bt[min(NS * step + stream, jlast)]; };
  // The entries of steps step and step + 1 as one vector load (even lanes the
  // first, odd lanes the second), fetched a block before they are used: a
  // vector load waits on the in-order load counter, which the page loads of
  // the block in between have already drained, whereas a scalar load here
  // would be waited for together with every outstanding LDS access.
  auto bt_fetch = [&](int step) -> int { return bt_entry(step + (lane & 1)); };
  auto pf_issue = [&](int step, int phys, uint4 &R0, uint4 &R1, uint4 &R2) {
    const bool valid = phys >= 0 && (int64_t)phys < num_blocks;
    const uint64_t bit = 1ull << (step & 63);
    vmask = valid ? (vmask | bit) : (vmask & ~bit);
    // wave-uniform page base + this thread's 32-bit chunk offsets
    const uint8_t *base = pages + (int64_t)(valid ? phys : 0) * kPageBytes;
    R0 = *reinterpret_cast<const uint4 *>(base + goff0);
    if (kLoads > 1) R1 = *reinterpret_cast<const uint4 *>(base + goff1);
    if (kLoads > 2) R2 = *reinterpret_cast<const uint4 *>(base + goff2);
  };
  auto pf_commit = [&](int buf, const uint4 &R0, const uint4 &R1, const uint4 &R2) {
    // No branches: a thread without a chunk writes the landing slot.
    uint8_t *d = s_page[stream][buf];
    *reinterpret_cast<uint4 *>(d + loff0) = R0;
    if (kLoads > 1) *reinterpret_cast<uint4 *>(d + loff1) = R1;
    if (kLoads > 2) *reinterpret_cast<uint4 *>(d + loff2) = R2;
  };
  // Partial page maxima of the page in LDS buffer buf: 8 token tiles x CGW
  // MFMAs, tile tl's MFMAs into one accumulator set while tile tl-1's are
  // folded into m[cg] (this lane's 4 tokens of every tile).  No branches.
  auto page_fold = [&](int buf, float (&m)[CGW]) {
    const uint8_t *pg = s_page[stream][buf];
    if constexpr (kBf16) {
      // bf16 query: each tile's codes are read and converted once (four
      // bf16 k-steps), then every column group runs its four-MFMA chain;
      // tile tl's chains go into one accumulator set while tile tl-1's are
      // folded, as in the E4M3 path.
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) m[cg] = -INFINITY;
      v4f cx[CGW], cy[CGW];
#pragma unroll
      for (int tl = 0; tl < 8; ++tl) {
        const uint8_t *tp = pg + page_token(tl, t16) * kTokenBytes;
        const uint32_t *a32 = reinterpret_cast<const uint32_t *>(tp + 16 * g);
        const float sf = e8m0_scale(tp[64 + g]);
        bf16x8 av[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) av[k] = fp4x8_to_bf16(a32[k], sf);
#pragma unroll
        for (int cg = 0; cg < CGW; ++cg) {
          v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < 4; ++k)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], __builtin_bit_cast(bf16x8, bqh[cg][k]),
                                                        c, 0, 0, 0);
          if (tl & 1) {
            cy[cg] = c;
            m[cg] = fold4(m[cg], cx[cg]);
          } else {
            cx[cg] = c;
            if (tl > 0) m[cg] = fold4(m[cg], cy[cg]);
          }
        }
      }
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) m[cg] = fold4(m[cg], cy[cg]);
      return;
    }
    u32x4 A[8];
    uint32_t S[8];
#pragma unroll
    for (int tl = 0; tl < 8; ++tl) {
      const uint8_t *tp = pg + page_token(tl, t16) * kTokenBytes;
      const u32x4a4 a4 = *reinterpret_cast<const u32x4a4 *>(tp + 16 * g);
      A[tl] = u32x4{a4.x, a4.y, a4.z, a4.w};
      S[tl] = tp[64 + g];
    }
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) m[cg] = -INFINITY;
    v4f cx[CGW], cy[CGW];
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) cx[cg] = tile_mfma(A[0], cg, S[0]);
#pragma unroll
    for (int tl = 1; tl < 8; ++tl) {
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) {
        if (tl & 1) {
          cy[cg] = tile_mfma(A[tl], cg, S[tl]);
          m[cg] = fold4(m[cg], cx[cg]);
        } else {
          cx[cg] = tile_mfma(A[tl], cg, S[tl]);
          m[cg] = fold4(m[cg], cy[cg]);
        }
      }
    }
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) m[cg] = fold4(m[cg], cy[cg]);
  };
  // The reduction over the 4 lane groups (token quarters) with VALU lane
  // swaps: afterwards the lane holds the page max of its own column.
  // Keeps a step's MFMA chain inside the step: the empty asm consumes the
  // folded maxima, so the compiler cannot sink the chain past the barrier
  // into the next step (where it would stay live across a queue drain).
  auto pin = [&](float (&m)[CGW]) {
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) asm volatile("" : "+v"(m[cg]));
  };
  auto page_reduce = [&](const float (&m)[CGW]) -> float {
    if constexpr (CGW == 4) {
      // reduce-scatter: lane group g ends with column group g's max
      const float k0 = max_split32(m[0], m[2]);   // groups 0,1: cg 0; groups 2,3: cg 2
      const float k1 = max_split32(m[1], m[3]);   // groups 0,1: cg 1; groups 2,3: cg 3
      return max_split16(k0, k1);                 // group g: cg g
    } else if constexpr (CGW == 2) {
      return max_xor16(max_split32(m[0], m[1]));  // groups 0,1: cg 0; 2,3: cg 1
    } else {
      return max_xor16(max_xor32(m[0]));
    }
  };
  const int wave_id = stream * NW + wave;
  // Insert every queued key into its column's list; each wave runs as many
  // insertions as its fullest queue holds.
  auto drain = [&]() {
#pragma unroll 1
    for (int i = 0; i < kQueue; ++i) {
      if (!__any(i < nq)) break;
      const uint64_t v = s_queue[i][qslot];
      top.insert_nb(i < nq ? v : 0ull);
    }
    nq = 0;
  };
  // At the start of a block (parity = the block's): drain every queue if
  // any wave posted a flag at the end of the previous block.
  auto need_flags = [&](int parity) -> uint64_t {
    return *reinterpret_cast<const uint64_t *>(&s_need[parity ^ 1][0]);
  };
  auto drain_if = [&](uint64_t flags) {
    if (__builtin_amdgcn_readfirstlane(flags != 0ull ? 1 : 0)) drain();   // same for every lane
  };
  auto maybe_drain = [&](int parity) { drain_if(need_flags(parity)); };
  // Offer page j's max to the column's list (j < 0, past the row's history
  // or an invalid page: nothing).  Branch-free: the queue write always
  // happens, the count moves only for a key above the filter bound.
  auto take = [&](float v, int step, int parity) {
    const int j = NS * step + stream;
    const bool ok = (j >= 0) & (j < myL) & (((vmask >> (step & 63)) & 1ull) != 0ull);
    const uint64_t key = ok ? make_key(v, j) : 0ull;
    uint64_t bound = top.k[kHist - 1];
    if constexpr (NS == 2) {
      const uint64_t floor = s_floor[parity ^ 1][stream ^ 1][tid];
      bound = floor > bound ? floor : bound;
      s_floor[parity][stream][tid] = top.k[kHist - 1];
    }
    // A queue whose wave posted no flag held at most kQueue - 4 keys at the
    // block's start (a flag is posted at kQueue - 3), so with the block's two
    // pushes the write index stays below kQueue - 2.
    s_queue[nq][qslot] = key;
    nq += key > bound ? 1 : 0;
    if (kScores && writer && ok) scores_out[(myT * H + my_h) * max_pages + j] = v * scale;
  };
  // End of a block (two pushes per queue): without a posted flag every queue
  // holds at most kQueue - 4 keys, so the next block's two writes stay
  // inside the queue.
  auto post = [&](int parity) {
    const bool need = __any(nq >= kQueue - 3);
    if (lane == 0) s_need[parity][wave_id] = need ? 1 : 0;
  };

  // Step k of the stream handles page NS * k + stream; a page index at or
  // past J re-reads page J - 1 and is not taken (J >= every row's L).  The
  // walk is software-pipelined: step k runs the MFMAs of its page and the
  // reduction and selection of step k-1's page.  The two streams do these
  // in opposite orders, so the two waves that share a SIMD (one per stream)
  // overlap one's MFMA chain with the other's selection work.
  const int K = (J + NS - 1) / NS;
  if (K > 0) {
    float ma[CGW], mb[CGW];
#pragma unroll
    for (int cg = 0; cg < CGW; ++cg) mb[cg] = -INFINITY;
    if constexpr (NS == 2) {
      s_floor[0][stream][tid] = 0ull;
      s_floor[1][stream][tid] = 0ull;
    }
    if (threadIdx.x < 16) (&s_need[0][0])[threadIdx.x] = 0;
    pf_issue(0, bt_entry(0), e0, e1, e2);
    __builtin_amdgcn_sched_barrier(0);
    pf_issue(1, bt_entry(1), o0, o1, o2);
    __builtin_amdgcn_sched_barrier(0);
    pf_commit(0, e0, e1, e2);
    pf_commit(1, o0, o1, o2);
    __builtin_amdgcn_sched_barrier(0);
    pf_issue(2, bt_entry(2), e0, e1, e2);
    __builtin_amdgcn_sched_barrier(0);
    pf_issue(3, bt_entry(3), o0, o1, o2);
    __builtin_amdgcn_sched_barrier(0);
    int bt_a = bt_fetch(4), bt_b = 0;
    lds_barrier();
    // Blocks of two steps, one barrier each.  Block b reads steps 2b, 2b+1
    // from buffers (2b) & 3, (2b+1) & 3, commits steps 2b+2, 2b+3 (loaded
    // during block b-1) into the other two buffers, and issues the loads of
    // steps 2b+4, 2b+5.  A buffer is rewritten one barrier after its reads.
    // bt_use holds the block-table entries of steps k+4, k+5 (fetched one
    // block earlier); bt_next receives those of steps k+6, k+7.
    // The staging (commit of steps k+2, k+3, issue of k+4, k+5) sits where
    // the stream's LDS traffic is light: stream 1 stages after its opening
    // selection step, before its first page's operand reads; stream 0 opens
    // with those reads (which would queue behind the staging writes) and
    // stages after its first page.
    auto block = [&](int k, int rb, int parity, int bt_use, int &bt_next) {
      auto stage = [&]() {
        pf_commit(rb ^ 2, e0, e1, e2);
        pf_commit((rb ^ 2) + 1, o0, o1, o2);
        bt_next = bt_fetch(k + 6);
        pf_issue(k + 4, __builtin_amdgcn_readlane(bt_use, 0), e0, e1, e2);
        pf_issue(k + 5, __builtin_amdgcn_readlane(bt_use, 1), o0, o1, o2);
      };
      maybe_drain(parity);
      if (stream == 0) {
        page_fold(rb, ma);
        pin(ma);
        take(page_reduce(mb), k - 1, parity);
        stage();
        page_fold(rb + 1, mb);
        pin(mb);
        take(page_reduce(ma), k, parity);
      } else {
        take(page_reduce(mb), k - 1, parity);
        pin(mb);
        stage();
        page_fold(rb, ma);
        pin(ma);
        take(page_reduce(ma), k, parity);
        pin(ma);
        page_fold(rb + 1, mb);
        pin(mb);
      }
      post(parity);
      lds_barrier();
    };
    int k = 0;
    for (; k < K; k += 4) {
      block(k, 0, 0, bt_a, bt_b);
      block(k + 2, 2, 1, bt_b, bt_a);
    }
    maybe_drain(0);
    take(page_reduce(mb), k - 1, 0);
  }
  drain();
  if constexpr (NS == 2) {
    // Stream 1 hands its lists to stream 0 through the (now idle) page
    // buffers: key i of thread t at [i * NT + t].  The streams saw disjoint
    // pages, so inserting one list into the other gives the top-15 of both.
    uint64_t *s_lists = reinterpret_cast<uint64_t *>(&s_page[0][0][0]);
    if (stream == 1) {
#pragma unroll
      for (int i = 0; i < kHist; ++i) s_lists[i * NT + tid] = top.k[i];
    }
    lds_barrier();
    if (stream == 0) {
#pragma unroll
      for (int i = 0; i < kHist; ++i) top.insert_nb(s_lists[i * NT + tid]);
    }
  }
  if (stream == 0 && writer && my_rl < nrows && myT < total_q)
    write_row(out + (myT * H + my_h) * kTopk, top, myL);
}

}  // namespace mi_idx

using namespace mi_idx;

extern "C" size_t mi_idx_prefill_plan_bytes(int num_reqs, int64_t total_q, int num_heads) {
  if (num_reqs < 0 || total_q < 0 || num_heads < 1 || num_heads > MI_IDX_MAX_HEADS) return 0;
  const int M = rows_per_tile(num_heads);
  const size_t tiles = (size_t)(total_q / M) + (size_t)num_reqs + 1;
  return (size_t)kPreHeaderInts * 4 + tiles * 16;
}

extern "C" int mi_idx_plan_prefill(const int32_t *cu_seqlens_q_host, const int32_t *seq_lens_host,
                                   int num_reqs, int num_heads, int gather_budget_pages,
                                   void *staging_host_pinned, void *plan, size_t plan_bytes,
                                   int *num_chunks_out_host, int *num_tiles_out_host,
                                   void *stream) {
  mi_idx_clear_error();
  if (num_reqs < 0) return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: num_reqs < 0");
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "plan_prefill: num_heads %d outside 1..8", num_heads);
  if (!staging_host_pinned || !plan || !num_tiles_out_host ||
      (num_reqs > 0 && (!cu_seqlens_q_host || !seq_lens_host)))
    return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: null pointer");
  if ((uintptr_t)plan % 16) return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: plan must be 16-byte aligned");
  if (num_reqs > 0 && cu_seqlens_q_host[0] != 0)
    return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: cu_seqlens_q[0] must be 0");
  for (int r = 0; r < num_reqs; ++r) {
    const int qn = cu_seqlens_q_host[r + 1] - cu_seqlens_q_host[r];
    if (qn < 0) return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: cu_seqlens_q decreases at %d", r);
    if (seq_lens_host[r] < qn)
      return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: seq_lens[%d]=%d < %d query rows", r,
                         seq_lens_host[r], qn);
  }
  const int64_t total_q = num_reqs > 0 ? cu_seqlens_q_host[num_reqs] : 0;
  const size_t need = mi_idx_prefill_plan_bytes(num_reqs, total_q, num_heads);
  if (plan_bytes < need)
    return mi_idx_fail(MI_IDX_ECAPACITY, "plan_prefill: plan_bytes %zu < %zu", plan_bytes, need);
  const int M = rows_per_tile(num_heads);
  // Greedy chunks of consecutive requests under the page budget.
  std::vector<int> chunk_of(num_reqs, 0);
  int nchunks = 0;
  {
    int first = 0;
    while (first < num_reqs) {
      int64_t total = std::max((seq_lens_host[first] - 1) / 128, 0);
      int end = first + 1;
      while (end < num_reqs) {
        const int64_t h = std::max((seq_lens_host[end] - 1) / 128, 0);
        if (gather_budget_pages > 0 && total + h > gather_budget_pages) break;
        total += h;
        ++end;
      }
      for (int r = first; r < end; ++r) chunk_of[r] = nchunks;
      ++nchunks;
      first = end;
    }
  }
  struct Tile { int r, row0, nrows, pages, chunk; };
  std::vector<Tile> tiles;
  for (int r = 0; r < num_reqs; ++r) {
    const int qn = cu_seqlens_q_host[r + 1] - cu_seqlens_q_host[r];
    const int ctx_ub = seq_lens_host[r] - qn;
    for (int row0 = 0; row0 < qn; row0 += M) {
      const int n = std::min(M, qn - row0);
      const int pages_ub = std::max((ctx_ub + row0 + n - 1) / 128, 0);
      tiles.push_back({r, row0, n, pages_ub, chunk_of[r]});
    }
  }
  // Launch order.  Workgroup b runs on XCD b % kXcds, and each XCD has its
  // own L2, so tiles that read the same pages (those of one request) should
  // share an XCD.  Chunk by chunk: the chunk's tiles, in request order, fill
  // the XCD queues one after another up to an equal share of the page work
  // each; every queue is sorted longest first; the queues are interleaved so
  // that position b takes the next tile of queue b % kXcds.
  std::vector<Tile> order;
  order.reserve(tiles.size());
  {
    size_t t0 = 0;
    while (t0 < tiles.size()) {
      size_t t1 = t0;
      int64_t work = 0;
      while (t1 < tiles.size() && tiles[t1].chunk == tiles[t0].chunk) {
        work += (int64_t)tiles[t1].pages + 1;
        ++t1;
      }
      std::vector<std::vector<Tile>> queue(kXcds);
      const int64_t share = (work + kXcds - 1) / kXcds;
      int x = 0;
      int64_t filled = 0;
      for (size_t i = t0; i < t1; ++i) {
        if (filled >= share && x < kXcds - 1) {
          ++x;
          filled = 0;
        }
        queue[x].push_back(tiles[i]);
        filled += (int64_t)tiles[i].pages + 1;
      }
      for (auto &qx : queue)
        std::stable_sort(qx.begin(), qx.end(),
                         [](const Tile &a, const Tile &b) { return a.pages > b.pages; });
      std::vector<size_t> head(kXcds, 0);
      size_t left = t1 - t0;
      int xi = (int)(order.size() % kXcds);   // the XCD of the next position
      while (left > 0) {
        if (head[xi] < queue[xi].size()) {
          order.push_back(queue[xi][head[xi]++]);
          --left;
        }
        xi = (xi + 1) % kXcds;
      }
      t0 = t1;
    }
  }
  tiles.swap(order);
  int32_t *st = static_cast<int32_t *>(staging_host_pinned);
  const size_t bytes = (size_t)kPreHeaderInts * 4 + tiles.size() * 16;
  if (bytes > plan_bytes)
    return mi_idx_fail(MI_IDX_ECAPACITY, "plan_prefill: %zu tiles exceed the plan", tiles.size());
  std::fill(st, st + kPreHeaderInts, 0);
  st[0] = (int32_t)tiles.size();
  st[1] = M;
  st[2] = num_heads;
  st[3] = nchunks;
  for (size_t i = 0; i < tiles.size(); ++i) {
    int32_t *t = st + kPreHeaderInts + 4 * i;
    t[0] = tiles[i].r;
    t[1] = tiles[i].row0;
    t[2] = tiles[i].nrows;
    t[3] = tiles[i].pages;
  }
  *num_tiles_out_host = (int)tiles.size();
  if (num_chunks_out_host) *num_chunks_out_host = nchunks;
  hipError_t e = hipMemcpyAsync(plan, staging_host_pinned, bytes, hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess)
    return mi_idx_fail(MI_IDX_EHIP, "plan_prefill: copy failed: %s", hipGetErrorString(e));
  return MI_IDX_OK;
}

extern "C" int mi_idx_score_topk_prefill(const void *q, int q_dtype, const uint8_t *pages,
                                         int64_t num_blocks, const int32_t *block_table,
                                         int64_t bt_stride, const int32_t *cu_seqlens_q,
                                         const int32_t *seq_lens, const int32_t *context_lens,
                                         int num_reqs, int64_t total_q, int num_heads,
                                         int max_pages, float scale, const void *plan,
                                         size_t plan_bytes, int num_tiles, int32_t *topk_out,
                                         float *scores_out, void *stream) {
  mi_idx_clear_error();
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "score_topk_prefill: num_heads %d outside 1..8",
                       num_heads);
  if (num_reqs < 0 || total_q < 0 || max_pages < 0 || num_tiles < 0)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: negative size");
  if (q_dtype != MI_IDX_Q_E4M3 && q_dtype != MI_IDX_Q_BF16)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: q_dtype %d is neither E4M3 (0) nor "
                                      "bf16 (1)", q_dtype);
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: scale must be positive and finite");
  if (num_tiles == 0 || total_q == 0) return MI_IDX_OK;
  if (!q || !pages || !block_table || !cu_seqlens_q || !seq_lens || !context_lens || !plan ||
      !topk_out)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: null pointer");
  if (((uintptr_t)q % 16) || ((uintptr_t)pages % 16) || ((uintptr_t)topk_out % 16) ||
      ((uintptr_t)plan % 16))
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: q, pages, topk_out and plan must be "
                                      "16-byte aligned");
  if (num_blocks <= 0) return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: num_blocks <= 0");
  if (bt_stride < max_pages)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: bt_stride < max_pages");
  if ((size_t)kPreHeaderInts * 4 + (size_t)num_tiles * 16 > plan_bytes)
    return mi_idx_fail(MI_IDX_ECAPACITY, "score_topk_prefill: num_tiles %d exceeds plan_bytes",
                       num_tiles);
  const dim3 grid(num_tiles), block(64 * kPrefillStreams * (16 / kPrefillCgw));
  const uint8_t *qb = static_cast<const uint8_t *>(q);
#define MI_IDX_LAUNCH_PRE(SC, BF)                                                              \
  hipLaunchKernelGGL((prefill_score_kernel<kPrefillCgw, kPrefillStreams, SC, BF>), grid, block, \
                     0, (hipStream_t)stream, qb, pages, num_blocks, block_table, bt_stride,    \
                     cu_seqlens_q, seq_lens, context_lens, num_reqs, total_q, num_heads,       \
                     max_pages, scale, (const int32_t *)plan, topk_out, scores_out)
  if (q_dtype == MI_IDX_Q_BF16) {
    if (scores_out) MI_IDX_LAUNCH_PRE(true, true);
    else MI_IDX_LAUNCH_PRE(false, true);
  } else {
    if (scores_out) MI_IDX_LAUNCH_PRE(true, false);
    else MI_IDX_LAUNCH_PRE(false, false);
  }
#undef MI_IDX_LAUNCH_PRE
  return mi_idx_check_launch("score_topk_prefill");
}
