// Prefill: host-side work plan + fused page scoring and top-16.
//
// A row tile is M consecutive query rows of one request and all H heads: 256
// query columns (column = row * H + head), 64 per wave, so each wave holds
// four 16-column MFMA B operands in registers while it works on the tile.
// The tile's causal pages 0..L_max-1 are walked in two interleaved page
// streams of four waves each; each page (8704 bytes) is staged once into LDS,
// rearranged so that the MFMA operand reads are aligned and few (below) --
// a ring of four buffers per stream, two pages per barrier, the next two
// pages' global loads in flight while the current two are consumed -- and
// re-read by the stream's four waves as the MFMA A operand.  At the end of a
// walk the two streams' lists are merged in LDS.
//
// Load balance.  Row tiles of one launch can differ a hundredfold in length
// (a ragged batch mixes short and long histories), and one workgroup fills a
// CU, so the host cuts the total page work into one equal work list per
// resident workgroup (persistent workgroups): a list holds whole tiles and
// page ranges of tiles.  A workgroup walks its pieces in turn; a whole tile
// writes its output rows, a page range of a split tile writes its columns'
// partial top-15 lists to the workspace, and a second small launch merges
// each split tile's lists into its output rows (on the same stream, so no
// device-wide fence is needed).
#include <algorithm>
#include <atomic>
#include <queue>
#include <cmath>
#include <vector>

#include "common.h"

namespace mi_idx {

constexpr int kTileCols = 256;          // query columns per row tile
constexpr int kPreHeaderInts = 16;
constexpr int kPreErrWord = 9;          // plan header word of the error bits
constexpr int kXcds = 8;                // MI355X accelerator complex dies
constexpr int kPrefillCgw = 4;          // 16-column groups per wave
constexpr int kPrefillStreams = 2;      // page streams per workgroup
constexpr int kQueue = 16;              // per-column key queue (LDS)
constexpr int kBufs = 4;                // LDS page buffers per stream
constexpr int kMaxLists = 512;          // work lists (scorer workgroups) per plan
constexpr int kPieceCost = 24;          // planning cost of a piece's set-up, in pages
constexpr int kMinSplit = 4;            // fewest pages a split piece gets
constexpr int kListKeys = 16;           // 15 keys + an empty slot: 128-byte lists
constexpr int kMaxSlots = 2 * kMaxLists;   // partial lists (one per split piece)

inline int rows_per_tile(int H) { return kTileCols / H; }

// Plan (int32 words).  Header: [0] work lists, [1] rows per tile,
// [2] num_heads, [3] chunk count, [4] pieces, [5] word offset of the pieces,
// [6] split tiles, [7] word offset of the split tiles, [8] partial-list slots,
// [9] error bits of the score calls on this plan (written 0 by the plan's
// copy; bit 0: a block-table id outside the pool was skipped, bit 2: a row
// whose history runs past max_pages was refused).
// Work list i (int4 at word 16 + 4 i): first piece, piece count.  Piece (8
// words): request, first row (in the request), row count, first page, end
// page (an upper bound; the kernel clamps it to the device lengths), slot
// (-1: a whole tile, which writes its output rows; else the partial-list
// slot).  Split tile (8 words): request, first row, row count, first slot,
// slot count.
// Workspace: partial lists [slot][256 columns][kListKeys] uint64 keys.

// LDS layout of a staged page (8704 bytes, rearranged from the global token
// records while staging).  Token tile tl of an MFMA chain is tokens 16 tl ..
// 16 tl + 15; MFMA lane (r, g) = r + 16 g takes token 16 tl + r, dims 32 g ..
// 32 g + 31 (16 code bytes) and that block's E8M0 scale.
//   codes: chunk g of token t at 16-byte slot 4 t + (g ^ lds_swz(t & 15)), so
//     lane (r, g) reads tile tl with one aligned 16-byte read at 1024 tl +
//     64 r + 16 (g ^ lds_swz(r)); the swizzle puts the chunks of any 8, and
//     of any 16, consecutive lanes of a read on distinct banks;
//   scales: after the 8192 code bytes, byte 8 (r + 16 g) + tl holds the scale
//     of token 16 tl + r, block g, so one 8-byte read gives a lane the scales
//     of all eight tiles, which the MFMA takes by byte select.
__device__ __forceinline__ int lds_swz(int r) { return (r >> 2) ^ (r & 2); }
constexpr int kLdsScales = kPageTokens * 64;   // 8192

// CGW = 16-column MFMA groups per wave: 16 / CGW waves cover the tile's
// kTileCols = 256 query columns.  NS page streams of such wave sets share the
// workgroup: stream s walks pages s, s + NS, s + 2 NS, ... with LDS buffers of
// its own, so a SIMD holds NS waves that interleave MFMA, VALU and waits.  At
// the end the streams' lists are merged through LDS by stream 0.
// kBf16: bfloat16 query (256 bytes per row and head) on the bf16 MFMA (see
// mfma_fp4_bf16); otherwise E4M3.
// kOne: every work list of the plan holds one whole tile (the piece loop is
// then a single pass over pages 0..J-1 that writes its rows, compiled
// without the loop).
template <int CGW, int NS, bool kScores, bool kBf16, bool kOne>
__global__ __launch_bounds__(64 * NS * (16 / CGW)) void prefill_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ cu_seqlens_q, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ context_lens, int num_reqs, int64_t total_q, int H,
    int max_pages, float scale, const int32_t *__restrict__ plan, uint64_t *__restrict__ ws_lists,
    int32_t *__restrict__ out, float *__restrict__ scores_out, uint32_t *err) {
  constexpr int NW = 16 / CGW;                       // waves per stream
  constexpr int NT = 64 * NW;                        // threads per stream
  static_assert(NS >= 1 && NS <= 2, "one or two page streams");
  static_assert(NS == 1 || kHist * NT * 8 <= NS * kBufs * kPageBytes,
                "the stream merge reuses the page buffers");
  // kBufs LDS page buffers per stream (a ring: two pages read per block while
  // the next two are written), each in the staged layout above.
  static_assert(NT == 256, "staging: two code chunks and two scale bytes per thread");
  __shared__ __attribute__((aligned(16))) uint8_t s_page[NS][kBufs][kPageBytes];
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
  const int4 wl = reinterpret_cast<const int4 *>(plan + kPreHeaderInts)[blockIdx.x];
  const int4 *pieces = reinterpret_cast<const int4 *>(plan + plan[5]);
  // wave-uniform (page indices derived from it stay scalar)
  const int stream = NS == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
  const int tid = (int)threadIdx.x - stream * NT;    // thread within its stream
  const int wave = tid >> 6, lane = tid & 63;
  const int t16 = lane & 15, g = lane >> 4;
  const int pend = kOne ? wl.x + 1 : wl.x + wl.y;
  // The next piece's record, read ahead while this piece walks its pages:
  // lane i < 6 of vrec holds word i (request, first row, row count, first
  // page, end page, slot).  A vector load: the page walk's LDS waits do not
  // wait for it, as they would for a scalar load.
  int vrec = 0;
#pragma unroll 1
  for (int pi = wl.x; pi < pend; ++pi) {
    int r, row0, nrows, pw, px, slot;
    if (kOne || pi == wl.x) {
      const int4 pc0 = pieces[2 * pi], pc1 = pieces[2 * pi + 1];
      r = pc0.x, row0 = pc0.y, nrows = pc0.z, pw = pc0.w, px = pc1.x, slot = pc1.y;
    } else {
      r = __builtin_amdgcn_readlane(vrec, 0), row0 = __builtin_amdgcn_readlane(vrec, 1);
      nrows = __builtin_amdgcn_readlane(vrec, 2), pw = __builtin_amdgcn_readlane(vrec, 3);
      px = __builtin_amdgcn_readlane(vrec, 4), slot = __builtin_amdgcn_readlane(vrec, 5);
    }
    if (!kOne) {
      const int32_t *nrec = reinterpret_cast<const int32_t *>(pieces) + 8 * (pi + 1);
      vrec = (pi + 1 < pend && lane < 6) ? nrec[lane] : 0;
    }
    if (r < 0 || r >= num_reqs) continue;   // the same for every thread
    const int ctx = context_lens[r];
    const int sl = seq_lens[r];
    const int64_t q0 = cu_seqlens_q[r];
    // What the end of the piece needs, kept in one register through the page
    // walk (lane i: request, first row, row count, slot, context length,
    // sequence length, first query row); the empty asm keeps the compiler
    // from holding the scalar originals instead.
    int vcur = lane == 0 ? r : lane == 1 ? row0 : lane == 2 ? nrows : lane == 3 ? slot
             : lane == 4 ? ctx : lane == 5 ? sl : (int)q0;
    asm volatile("" : "+v"(vcur));

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
    // This lane's code chunk of token tile 0 in a staged page (tile tl at
    // +1024 tl).
    const uint32_t code_off = 64u * (uint32_t)t16 + 16u * (uint32_t)(g ^ lds_swz(t16));
    // One 16x16x128 E4M3 tile of column group cg, token tile tl (its scale:
    // byte tl & 3 of sc.x or sc.y).
    auto tile_mfma_sel = [&](const u32x4 &a, int cg, const uint2 &sc, int tl) -> v4f {
      const uint32_t w = tl < 4 ? sc.x : sc.y;
      switch (tl & 3) {
        case 0: return mfma_fp4_fp8_sel<0>(a, bq[cg], w);
        case 1: return mfma_fp4_fp8_sel<1>(a, bq[cg], w);
        case 2: return mfma_fp4_fp8_sel<2>(a, bq[cg], w);
        default: return mfma_fp4_fp8_sel<3>(a, bq[cg], w);
      }
    };
    // The column this lane owns after the page-max reduction: with 4 groups
    // per wave each lane group owns one; with 2, lane groups g and g^1 both
    // hold group g>>1 (the even one writes it); with 1, all hold it.
    const int my_cg = CGW == 4 ? g : (CGW == 2 ? (g >> 1) : 0);
    const bool writer = CGW == 4 ? true : (CGW == 2 ? (g & 1) == 0 : g == 0);
    const int mycol = (wave * CGW + my_cg) * 16 + t16;
    const int my_rl = mycol / H, my_h = mycol - my_rl * H;
    const int64_t myT = q0 + row0 + my_rl;
    int myL = -1;   // -1 also for a row refused because its history runs past max_pages
    if (my_rl < nrows && myT < total_q) {
      const int p = ctx + row0 + my_rl;
      myL = p < sl ? local_page(p, max_pages) : -1;
    }
    // Pages of the tile: every row's history is a prefix of 0..J-1.  This
    // piece walks pages jb..je-1 of them; a column takes page j < myLe.
    int J = 0;
    {
      const int plast = ctx + row0 + nrows - 1;
      J = plast >= 0 ? min(plast >> 7, max_pages) : 0;
      J = max(J, 0);
    }
    const int jb = kOne ? 0 : max(pw, 0);
    const int je = kOne ? J : max(min(px, J), jb);
    const int myLe = kOne ? myL : min(myL, je);
    // The column's top-15 (registers) and its queue (LDS): a key that beats
    // the list's 15th key (and the partner stream's) is appended to the queue
    // with no branch -- the write always happens, the count moves only for a
    // qualifying key -- and queues are drained into the lists rarely, each
    // wave running as many insertions as its fullest queue holds.
    TopList top;
    top.clear();
    int nq = 0;
    const int qslot = stream * NT + tid;

    // Page pipeline (per stream; step s is the stream's s-th page).  This
    // thread's share of step s (two code chunks and a scale word) is loaded
    // into register slot s & 1, written into LDS buffer s & 3 a block later
    // (rearranged into the staged layout), and read
    // there by the stream's four waves in the block after that: while a block
    // consumes two pages, the next two sit in registers (then LDS) and the two
    // after them are in flight.  Every load is unconditional (chunk and page
    // indices are clamped, an invalid page id reads page 0 and is skipped), and
    // the barriers order LDS only, so the global loads stay in flight across
    // them.
    const int32_t *bt = block_table + (int64_t)r * bt_stride;
    const int jlast = je - 1;
    // slot 0 (even pages): e0, e1, es; slot 1 (odd pages): o0, o1, os
    uint4 e0, e1, o0, o1;
    uint32_t es, os;
    // Validity of the page of step s (bit s & 63), recorded when the page is
    // issued; a step's page is taken 4 steps after its issue, long before the
    // bit is reused 64 steps later.  Wave-uniform, so it lives in SGPRs.
    uint64_t vmask = 0;
    // This thread's share of a page (loop-invariant byte offsets): code chunks
    // q = tid and tid + 256 (token q >> 2, block q & 3; global 68 (q >> 2) +
    // 16 (q & 3)), and the scale bytes of blocks gs, gs + 1 of token tid >> 1
    // (its scale word at global 68 (tid >> 1) + 64).
    auto code_goff = [](int q) { return 68u * (uint32_t)(q >> 2) + 16u * (uint32_t)(q & 3); };
    auto code_loff = [](int q) {
      const int t = q >> 2;
      return 16u * (uint32_t)(4 * t + ((q & 3) ^ lds_swz(t & 15)));
    };
    const uint32_t goff0 = code_goff(tid), goff1 = code_goff(tid + NT);
    const uint32_t loff0 = code_loff(tid), loff1 = code_loff(tid + NT);
    const int ts = tid >> 1, gs = 2 * (tid & 1);
    const uint32_t goffs = 68u * (uint32_t)ts + 64u;
    const uint32_t loffs = (uint32_t)kLdsScales + 8u * (uint32_t)((ts & 15) + 16 * gs) +
                           (uint32_t)(ts >> 4);   // block gs; block gs + 1 at +128
    const uint32_t sshift = 8u * (uint32_t)gs;
    // Block-table entry of a step (clamped like the page index).
    auto bt_entry = [&](int step) { return bt[min(jb + NS * step + stream, jlast)]; };
    // The entries of steps step and step + 1 as one vector load (even lanes the
    // first, odd lanes the second), fetched a block before they are used: a
    // vector load waits on the in-order load counter, which the page loads of
    // the block in between have already drained, whereas a scalar load here
    // would be waited for together with every outstanding LDS access.
    auto bt_fetch = [&](int step) -> int { return bt_entry(step + (lane & 1)); };
    // an issued page id outside the pool (every issued page lies inside the
    // piece's range): skipped, reported in the plan's error word
    bool bad = false;
    auto pf_issue = [&](int step, int phys, uint4 &R0, uint4 &R1, uint32_t &RS) {
      const bool valid = phys >= 0 && (int64_t)phys < num_blocks;
      bad |= !valid;
      const uint64_t bit = 1ull << (step & 63);
      vmask = valid ? (vmask | bit) : (vmask & ~bit);
      // wave-uniform page base + this thread's 32-bit offsets (the code chunks
      // are 4-byte aligned in global memory)
      const uint8_t *base = pages + (int64_t)(valid ? phys : 0) * kPageBytes;
      const u32x4a4 c0 = *reinterpret_cast<const u32x4a4 *>(base + goff0);
      const u32x4a4 c1 = *reinterpret_cast<const u32x4a4 *>(base + goff1);
      R0 = uint4{c0.x, c0.y, c0.z, c0.w};
      R1 = uint4{c1.x, c1.y, c1.z, c1.w};
      RS = *reinterpret_cast<const uint32_t *>(base + goffs);
    };
    auto pf_commit = [&](int buf, const uint4 &R0, const uint4 &R1, uint32_t RS) {
      uint8_t *d = s_page[stream][buf];
      *reinterpret_cast<uint4 *>(d + loff0) = R0;
      *reinterpret_cast<uint4 *>(d + loff1) = R1;
      d[loffs] = (uint8_t)(RS >> sshift);
      d[loffs + 128u] = (uint8_t)(RS >> (sshift + 8u));
    };
    // Partial page maxima of the page in LDS buffer buf: 8 token tiles x CGW
    // MFMAs, tile tl's MFMAs into one accumulator set while tile tl-1's are
    // folded into m[cg] (this lane's 4 tokens of every tile).  No branches.
    // (pre: the scale word and tile 0's operand, psc and pa0, were read ahead)
    auto page_fold = [&](int buf, float (&m)[CGW], bool pre = false, uint2 psc = uint2{0u, 0u},
                         u32x4 pa0 = u32x4{0u, 0u, 0u, 0u}) {
      const uint8_t *pg = s_page[stream][buf];
      if constexpr (kBf16) {
        // bf16 query: each tile's codes are read and converted once (four
        // bf16 k-steps), then every column group runs its four-MFMA chain;
        // tile tl's chains go into one accumulator set while tile tl-1's are
        // folded, as in the E4M3 path.
#pragma unroll
        for (int cg = 0; cg < CGW; ++cg) m[cg] = -INFINITY;
        v4f cx[CGW], cy[CGW];
        const uint2 sc = *reinterpret_cast<const uint2 *>(pg + kLdsScales + 8 * lane);
#pragma unroll
        for (int tl = 0; tl < 8; ++tl) {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(pg + code_off + 1024 * tl);
          const float sf = e8m0_scale(((tl < 4 ? sc.x : sc.y) >> (8 * (tl & 3))) & 0xFFu);
          bf16x8 av[4];
          av[0] = fp4x8_to_bf16(a.x, sf);
          av[1] = fp4x8_to_bf16(a.y, sf);
          av[2] = fp4x8_to_bf16(a.z, sf);
          av[3] = fp4x8_to_bf16(a.w, sf);
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
      // the scales first: the chain's first MFMA then waits for two reads, not nine
      const uint2 sc = pre ? psc : *reinterpret_cast<const uint2 *>(pg + kLdsScales + 8 * lane);
      u32x4 A[8];
      A[0] = pre ? pa0 : *reinterpret_cast<const u32x4 *>(pg + code_off);
#pragma unroll
      for (int tl = 1; tl < 8; ++tl)
        A[tl] = *reinterpret_cast<const u32x4 *>(pg + code_off + 1024 * tl);
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) m[cg] = -INFINITY;
      v4f cx[CGW], cy[CGW];
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) cx[cg] = tile_mfma_sel(A[0], cg, sc, 0);
#pragma unroll
      for (int tl = 1; tl < 8; ++tl) {
#pragma unroll
        for (int cg = 0; cg < CGW; ++cg) {
          if (tl & 1) {
            cy[cg] = tile_mfma_sel(A[tl], cg, sc, tl);
            m[cg] = fold4(m[cg], cx[cg]);
          } else {
            cx[cg] = tile_mfma_sel(A[tl], cg, sc, tl);
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
    // Drain every queue into its list.  With 6 or more keys queued in some
    // lane, by sorting networks: the (zero-padded) 16 queued keys sorted
    // descending (bitonic sort), then max(list[i], queue[15 - i]) -- the best
    // 16 of both, as a bitonic sequence -- and one bitonic merge: 112
    // compare-exchanges against 15 per inserted key.  With fewer, one
    // insertion per key.
    auto drain = [&]() {
      if (__any(nq >= 6)) {
        uint64_t q[kQueue];
#pragma unroll
        for (int i = 0; i < kQueue; ++i) q[i] = i < nq ? s_queue[i][qslot] : 0ull;
        auto cas = [](uint64_t &a, uint64_t &b) {   // a >= b afterwards
          const bool sw = a < b;
          const uint64_t t = a;
          a = sw ? b : a;
          b = sw ? t : b;
        };
#pragma unroll
        for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
          for (int j = k >> 1; j >= 1; j >>= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int l = i ^ j;
              if (l > i) {
                if ((i & k) == 0) cas(q[i], q[l]);
                else cas(q[l], q[i]);
              }
            }
        uint64_t c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint64_t a = i < kHist ? top.k[i] : 0ull, b = q[15 - i];
          c[i] = a > b ? a : b;
        }
#pragma unroll
        for (int j = 8; j >= 1; j >>= 1)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) cas(c[i], c[l]);
          }
#pragma unroll
        for (int i = 0; i < kHist; ++i) top.k[i] = c[i];
      } else {
#pragma unroll 1
        for (int i = 0; i < kQueue; ++i) {
          if (!__any(i < nq)) break;
          const uint64_t v = s_queue[i][qslot];
          top.insert_nb(i < nq ? v : 0ull);
        }
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
    // Offer page j's max to the column's list (step < 0, past the row's
    // history or the piece, or an invalid page: nothing).  Branch-free: the
    // queue write always happens, the count moves only for a key above the
    // filter bound.  Both selection steps of a block compare against the same
    // partner bound (written a block earlier), so the block reads it once and
    // passes it in (have_floor, floor_pre).
    auto take = [&](float v, int step, int parity, bool have_floor = false,
                    uint64_t floor_pre = 0ull) {
      const int j = jb + NS * step + stream;
      const bool ok = (step >= 0) & (j < myLe) & (((vmask >> (step & 63)) & 1ull) != 0ull);
      const uint64_t key = ok ? make_key(v, j) : 0ull;
      uint64_t bound = top.k[kHist - 1];
      if constexpr (NS == 2) {
        const uint64_t floor = have_floor ? floor_pre : s_floor[parity ^ 1][stream ^ 1][tid];
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

    // Step k of the stream handles page jb + NS * k + stream; a page index at
    // or past je re-reads page je - 1 and is not taken.  The
    // walk is software-pipelined: step k runs the MFMAs of its page and the
    // reduction and selection of step k-1's page.  The two streams do these
    // in opposite orders, so the two waves that share a SIMD (one per stream)
    // overlap one's MFMA chain with the other's selection work.
    const int K = (je - jb + NS - 1) / NS;
    if (K > 0) {
      float ma[CGW], mb[CGW];
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) mb[cg] = -INFINITY;
      if constexpr (NS == 2) {
        s_floor[0][stream][tid] = 0ull;
        s_floor[1][stream][tid] = 0ull;
      }
      if (threadIdx.x < 16) (&s_need[0][0])[threadIdx.x] = 0;
      pf_issue(0, bt_entry(0), e0, e1, es);
      __builtin_amdgcn_sched_barrier(0);
      pf_issue(1, bt_entry(1), o0, o1, os);
      __builtin_amdgcn_sched_barrier(0);
      pf_commit(0, e0, e1, es);
      pf_commit(1, o0, o1, os);
      __builtin_amdgcn_sched_barrier(0);
      pf_issue(2, bt_entry(2), e0, e1, es);
      __builtin_amdgcn_sched_barrier(0);
      pf_issue(3, bt_entry(3), o0, o1, os);
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
          __builtin_amdgcn_s_setprio(1);
          pf_commit(rb ^ 2, e0, e1, es);
          pf_commit((rb ^ 2) + 1, o0, o1, os);
          bt_next = bt_fetch(k + 6);
          pf_issue(k + 4, __builtin_amdgcn_readlane(bt_use, 0), e0, e1, es);
          pf_issue(k + 5, __builtin_amdgcn_readlane(bt_use, 1), o0, o1, os);
          __builtin_amdgcn_s_setprio(0);
        };
        // A wave issuing its MFMA chain, or staging the next pages, runs at
        // raised priority, so that the SIMD's other wave (in its selection
        // step) does not delay the next MFMA or load (about 1.7 % faster on
        // the mixed step in A/B).
        // The block's first page's scale word and first operand tile, and the
        // partner stream's bound for both selection steps, are read together
        // with the drain flags: stream 0's chain on that page then
        // does not wait for a second LDS round trip after the check, and
        // stream 1's starts after its selection step and staging with them in
        // registers.
        const uint8_t *pg0 = s_page[stream][rb];
        const uint2 sc0 = *reinterpret_cast<const uint2 *>(pg0 + kLdsScales + 8 * lane);
        const u32x4 a00 = *reinterpret_cast<const u32x4 *>(pg0 + code_off);
        const uint64_t fl = s_floor[parity ^ 1][stream ^ 1][tid];
        maybe_drain(parity);
        if (stream == 0) {
          __builtin_amdgcn_s_setprio(1);
          page_fold(rb, ma, true, sc0, a00);
          __builtin_amdgcn_s_setprio(0);
          pin(ma);
          take(page_reduce(mb), k - 1, parity, true, fl);
          stage();
          __builtin_amdgcn_s_setprio(1);
          page_fold(rb + 1, mb);
          __builtin_amdgcn_s_setprio(0);
          pin(mb);
          take(page_reduce(ma), k, parity, true, fl);
        } else {
          take(page_reduce(mb), k - 1, parity, true, fl);
          pin(mb);
          stage();
          __builtin_amdgcn_s_setprio(1);
          page_fold(rb, ma, true, sc0, a00);
          __builtin_amdgcn_s_setprio(0);
          pin(ma);
          take(page_reduce(ma), k, parity, true, fl);
          pin(ma);
          __builtin_amdgcn_s_setprio(1);
          page_fold(rb + 1, mb);
          __builtin_amdgcn_s_setprio(0);
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
    if (bad && lane == 0) atomicOr(err, 1u);
    if constexpr (NS == 2) {
      // Stream 1 hands its lists to stream 0 through the (now idle) page
      // buffers: key i of thread t at [i * NT + t].  The streams saw disjoint
      // pages, so the best 15 of both lists are the tile's top-15.
      uint64_t *s_lists = reinterpret_cast<uint64_t *>(&s_page[0][0][0]);
      if (stream == 1) {
#pragma unroll
        for (int i = 0; i < kHist; ++i) s_lists[i * NT + tid] = top.k[i];
      }
      lds_barrier();
      if (stream == 0) {
        // max(a[i], b[15 - i]) of the two sorted lists (each padded with an
        // empty 16th key) holds the best 16 of both as a bitonic sequence,
        // which one bitonic merge sorts.
        uint64_t c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint64_t a = i < kHist ? top.k[i] : 0ull;
          const uint64_t b = i >= 1 ? s_lists[(15 - i) * NT + tid] : 0ull;
          c[i] = a > b ? a : b;
        }
#pragma unroll
        for (int j = 8; j >= 1; j >>= 1)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) {
              const bool sw = c[i] < c[l];
              const uint64_t t = c[i];
              c[i] = sw ? c[l] : c[i];
              c[l] = sw ? t : c[l];
            }
          }
#pragma unroll
        for (int i = 0; i < kHist; ++i) top.k[i] = c[i];
      }
    }
    if (stream == 0 && writer) {
      const int frow0 = __builtin_amdgcn_readlane(vcur, 1);
      const int fnrows = __builtin_amdgcn_readlane(vcur, 2);
      const int fslot = __builtin_amdgcn_readlane(vcur, 3);
      const int fctx = __builtin_amdgcn_readlane(vcur, 4);
      const int fsl = __builtin_amdgcn_readlane(vcur, 5);
      const int fq0 = __builtin_amdgcn_readlane(vcur, 6);
      const int rl = mycol / H, h = mycol - rl * H;
      const int64_t T = (int64_t)fq0 + frow0 + rl;
      if (rl < fnrows && T < total_q) {
        if (kOne || fslot < 0) {
          const int p = fctx + frow0 + rl;
          const int L = p < fsl ? local_page(p, max_pages) : -1;
          write_row(out + (T * H + h) * kTopk, top, L);
          if (L < 0 && p >= 0 && p < fsl) atomicOr(err, 4u);   // refused row
        } else if (ws_lists != nullptr && fslot < kMaxSlots) {
          u32x4 *dst = reinterpret_cast<u32x4 *>(
              ws_lists + ((size_t)fslot * kTileCols + mycol) * kListKeys);
#pragma unroll
          for (int k2 = 0; k2 < kListKeys / 2; ++k2) {
            const uint64_t x0 = top.k[2 * k2];
            const uint64_t x1 = 2 * k2 + 1 < kHist ? top.k[2 * k2 + 1] : 0ull;
            dst[k2] = u32x4{(uint32_t)x0, (uint32_t)(x0 >> 32), (uint32_t)x1,
                            (uint32_t)(x1 >> 32)};
          }
        }
      }
    }
    // The next piece's staging rewrites the page buffers read just above.
    if constexpr (!kOne) __syncthreads();
  }
}

// One workgroup per split tile, one thread per column: the top-15 of the
// tile's partial lists (their pages are disjoint, so their keys are
// distinct) goes to the column's output row with the -1 padding and the
// local page, as a whole tile writes it.
__global__ __launch_bounds__(kTileCols) void prefill_merge_kernel(
    const int32_t *__restrict__ cu_seqlens_q, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ context_lens, int num_reqs, int64_t total_q, int H,
    int max_pages, const int32_t *__restrict__ plan, const uint64_t *__restrict__ ws_lists,
    int32_t *__restrict__ out, uint32_t *err) {
  if ((int)blockIdx.x >= plan[6]) return;
  const int4 *splits = reinterpret_cast<const int4 *>(plan + plan[7]);
  const int4 m0 = splits[2 * blockIdx.x], m1 = splits[2 * blockIdx.x + 1];
  const int r = m0.x, row0 = m0.y, nrows = m0.z, s0 = m0.w, ns = m1.x;
  if (r < 0 || r >= num_reqs || s0 < 0 || ns < 0 || s0 + ns > kMaxSlots) return;
  const int c = (int)threadIdx.x;
  const int rl = c / H, h = c - rl * H;
  if (rl >= nrows) return;
  const int64_t T = (int64_t)cu_seqlens_q[r] + row0 + rl;
  if (T >= total_q) return;
  const int p = context_lens[r] + row0 + rl;
  const int L = p < seq_lens[r] ? local_page(p, max_pages) : -1;
  if (L < 0 && p >= 0 && p < seq_lens[r]) atomicOr(err, 4u);   // refused row
  // The pieces' lists (16 keys each, sorted, the last one empty) are loaded
  // four at a time, all in flight together, and folded in with sorting
  // networks: max(a[i], b[15 - i]) holds the best 16 of the running list a
  // and list b as a bitonic sequence, which one bitonic merge sorts.
  uint64_t a[kListKeys];
#pragma unroll
  for (int i = 0; i < kListKeys; ++i) a[i] = 0ull;
  auto cas = [](uint64_t &x, uint64_t &y) {   // x >= y afterwards
    const bool sw = x < y;
    const uint64_t t = x;
    x = sw ? y : x;
    y = sw ? t : y;
  };
#pragma unroll 1
  for (int sb = s0; sb < s0 + ns; sb += 4) {
    u32x4 v[4][kListKeys / 2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = min(sb + j, s0 + ns - 1);   // past the last list: re-read it, not merged
      const u32x4 *src = reinterpret_cast<const u32x4 *>(
          ws_lists + ((size_t)sl * kTileCols + c) * kListKeys);
#pragma unroll
      for (int k2 = 0; k2 < kListKeys / 2; ++k2) v[j][k2] = src[k2];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sb + j >= s0 + ns) break;
      uint64_t cmb[kListKeys];
#pragma unroll
      for (int i = 0; i < kListKeys; ++i) {
        const u32x4 w = v[j][(kListKeys - 1 - i) >> 1];
        const uint64_t b = ((kListKeys - 1 - i) & 1) ? (((uint64_t)w.w << 32) | w.z)
                                                     : (((uint64_t)w.y << 32) | w.x);
        cmb[i] = a[i] > b ? a[i] : b;
      }
#pragma unroll
      for (int d = kListKeys / 2; d >= 1; d >>= 1)
#pragma unroll
        for (int i = 0; i < kListKeys; ++i)
          if ((i ^ d) > i) cas(cmb[i], cmb[i ^ d]);
#pragma unroll
      for (int i = 0; i < kListKeys; ++i) a[i] = cmb[i];
    }
  }
  TopList top;
#pragma unroll
  for (int i = 0; i < kHist; ++i) top.k[i] = a[i];
  write_row(out + (T * H + h) * kTopk, top, L);
}

}  // namespace mi_idx

using namespace mi_idx;

// Row tiles of a plan: at most one per M rows plus one partial tile per request.
static size_t max_tiles(int num_reqs, int64_t total_q, int M) {
  return (size_t)(total_q / M) + (size_t)num_reqs + 1;
}

static size_t plan_words(size_t lists, size_t pieces, size_t splits) {
  return (size_t)kPreHeaderInts + 4 * lists + 8 * pieces + 8 * splits;
}

// Scorer workgroups the device holds at once (the lowest occupancy of the
// four instantiations times the CU count), capped at kMaxLists; once per
// device.  Without a device (host-only use) the MI355X figure, 256.
static int resident_lists() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  const int hit = cache[dev].load(std::memory_order_relaxed);
  if (hit > 0) return hit;
  const int threads = 64 * kPrefillStreams * (16 / kPrefillCgw);
  int b[4] = {0, 0, 0, 0}, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &b[0], prefill_score_kernel<kPrefillCgw, kPrefillStreams, false, false, false>, threads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b[1], prefill_score_kernel<kPrefillCgw, kPrefillStreams, true, false, false>, threads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b[2], prefill_score_kernel<kPrefillCgw, kPrefillStreams, false, true, false>, threads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b[3], prefill_score_kernel<kPrefillCgw, kPrefillStreams, true, true, false>, threads, 0);
  if (e != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  const long long n = (long long)std::max(std::min(std::min(b[0], b[1]), std::min(b[2], b[3])), 1) * cus;
  const int v = (int)std::max(1LL, std::min(n, (long long)kMaxLists));
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

extern "C" size_t mi_idx_prefill_plan_bytes(int num_reqs, int64_t total_q, int num_heads) {
  if (num_reqs < 0 || total_q < 0 || num_heads < 1 || num_heads > MI_IDX_MAX_HEADS) return 0;
  const size_t tiles = max_tiles(num_reqs, total_q, rows_per_tile(num_heads));
  // each split closes a work list: pieces <= tiles + lists - 1, split tiles <= lists - 1
  return 4 * plan_words(kMaxLists, tiles + kMaxLists, kMaxLists);
}

extern "C" size_t mi_idx_prefill_workspace_bytes(void) {
  return (size_t)kMaxSlots * kTileCols * kListKeys * 8;
}

extern "C" int mi_idx_plan_prefill(const int32_t *cu_seqlens_q_host, const int32_t *seq_lens_host,
                                   int num_reqs, int num_heads, int gather_budget_pages,
                                   void *staging_host_pinned, void *plan, size_t plan_bytes,
                                   mi_idx_prefill_launch *launch_out_host, void *stream) {
  mi_idx_clear_error();
  if (num_reqs < 0) return mi_idx_fail(MI_IDX_EINVAL, "plan_prefill: num_reqs < 0");
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "plan_prefill: num_heads %d outside 1..8", num_heads);
  if (!staging_host_pinned || !plan || !launch_out_host ||
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
  // Chunk by chunk and request by request, longest tile first inside a
  // request (requests are numbered in chunk order).
  std::stable_sort(tiles.begin(), tiles.end(), [](const Tile &a, const Tile &b) {
    return a.r != b.r ? a.r < b.r : a.pages > b.pages;
  });
  // Work lists, one per resident scorer workgroup (S), of equal planning cost
  // (pages + kPieceCost per piece).  Near-equal tiles (the longest within 5 %
  // above the balanced share), no more than S of them, stay whole, one per
  // list.  Otherwise the tiles go longest first to the least-loaded list, and
  // then, while it lowers the maximum, the largest piece of the most-loaded
  // list gives a page range from its end to the least-loaded list (at most S
  // such splits, each piece at least kMinSplit pages).  Lists are ordered by
  // the request of their first piece, for the placement below; empty lists
  // are dropped.
  const int S = resident_lists();
  struct Piece { int tile, pa, pe; };
  std::vector<Piece> pieces;     // grouped by list, lists in launch order
  std::vector<int> list_first;
  std::vector<int> slot;
  struct Split { int tile, first_slot, nslots; };
  std::vector<Split> splits;
  int nslots = 0;
  int nlists = 0;
  {
    int64_t work = 0, longest = 0;
    for (const Tile &t : tiles) {
      work += (int64_t)t.pages + kPieceCost;
      longest = std::max(longest, (int64_t)t.pages + kPieceCost);
    }
    const int64_t share = std::max<int64_t>((work + S - 1) / S, kPieceCost + kMinSplit);
    const bool whole = (longest <= share || longest * 20 <= share * 21) && (int)tiles.size() <= S;
    struct P { int tile, pa, pe, list; };
    std::vector<P> ps;
    ps.reserve(tiles.size() + S);
    std::vector<int> head(S, -1);      // a list's first (largest) piece
    if (whole) {
      for (int ti = 0; ti < (int)tiles.size(); ++ti) {
        head[ti] = (int)ps.size();
        ps.push_back({ti, 0, tiles[ti].pages, ti});
      }
    } else {
      std::vector<int64_t> load(S, 0);
      std::vector<int> order(tiles.size());
      for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
      std::stable_sort(order.begin(), order.end(),
                       [&](int x, int y) { return tiles[x].pages > tiles[y].pages; });
      using LI = std::pair<int64_t, int>;
      std::priority_queue<LI, std::vector<LI>, std::greater<LI>> lo;   // least-loaded first
      for (int i = 0; i < S; ++i) lo.push({0, i});
      for (int ti : order) {
        const int i = lo.top().second;
        lo.pop();
        if (head[i] < 0) head[i] = (int)ps.size();
        ps.push_back({ti, 0, tiles[ti].pages, i});
        load[i] += (int64_t)tiles[ti].pages + kPieceCost;
        lo.push({load[i], i});
      }
      // Rebalance with two heaps over (load, list); an entry whose load is
      // no longer the list's is stale and skipped.
      std::priority_queue<LI> hi;                                   // most-loaded first
      for (int i = 0; i < S; ++i) hi.push({load[i], i});
      auto top_of = [&](auto &h) {
        while (h.top().first != load[h.top().second]) h.pop();
        return h.top().second;
      };
      for (int it = 0; it < S; ++it) {
        const int mx = top_of(hi), mn = top_of(lo);
        if (mx == mn || head[mx] < 0) break;
        P &pc = ps[head[mx]];
        int64_t X = (load[mx] - load[mn] - kPieceCost) / 2;
        X = std::min<int64_t>(X, (int64_t)(pc.pe - pc.pa) - kMinSplit);
        if (X < kMinSplit) break;
        const int cut = pc.pe - (int)X;
        if (head[mn] < 0) head[mn] = (int)ps.size();
        ps.push_back({pc.tile, cut, ps[head[mx]].pe, mn});
        ps[head[mx]].pe = cut;
        load[mx] -= X;
        load[mn] += X + kPieceCost;
        hi.push({load[mx], mx});
        hi.push({load[mn], mn});
        lo.push({load[mx], mx});
        lo.push({load[mn], mn});
      }
    }
    // Launch order of the non-empty lists: by the request of their first
    // piece (stable), then each list's pieces in the order they were added.
    std::vector<int> lorder;
    for (int i = 0; i < S; ++i)
      if (head[i] >= 0) lorder.push_back(i);
    std::stable_sort(lorder.begin(), lorder.end(), [&](int x, int y) {
      return tiles[ps[head[x]].tile].r < tiles[ps[head[y]].tile].r;
    });
    nlists = (int)lorder.size();
    std::vector<int> pos(S, -1), count(nlists + 1, 0);
    for (int k = 0; k < nlists; ++k) pos[lorder[k]] = k;
    for (const P &q : ps) ++count[pos[q.list] + 1];
    for (int k = 0; k < nlists; ++k) count[k + 1] += count[k];
    list_first.assign(count.begin(), count.begin() + nlists);
    pieces.resize(ps.size());
    std::vector<int> at(ps.size());
    for (int i = 0; i < (int)ps.size(); ++i) {
      const int k = count[pos[ps[i].list]]++;
      pieces[k] = {ps[i].tile, ps[i].pa, ps[i].pe};
      at[i] = k;
    }
    // Slots: consecutive per split tile, in page order.
    std::vector<int> by_tile(ps.size());
    for (int i = 0; i < (int)ps.size(); ++i) by_tile[i] = i;
    std::sort(by_tile.begin(), by_tile.end(), [&](int x, int y) {
      return ps[x].tile != ps[y].tile ? ps[x].tile < ps[y].tile : ps[x].pa < ps[y].pa;
    });
    slot.assign(pieces.size(), -1);
    for (size_t i = 0; i < by_tile.size();) {
      size_t j = i + 1;
      while (j < by_tile.size() && ps[by_tile[j]].tile == ps[by_tile[i]].tile) ++j;
      if (j - i > 1) {
        splits.push_back({ps[by_tile[i]].tile, nslots, (int)(j - i)});
        for (size_t k = i; k < j; ++k) slot[at[by_tile[k]]] = nslots++;
      }
      i = j;
    }
  }
  // Placement.  Workgroup b runs on XCD b % kXcds, each XCD with its own L2,
  // and lists in request order put a request's tiles (which read the same
  // pages) close together, so consecutive lists go to one XCD: XCD x takes
  // the next count(x) lists as workgroups x, x + kXcds, ...
  std::vector<int> list_at(nlists);
  {
    int i = 0;
    for (int x = 0; x < kXcds; ++x)
      for (int b = x; b < nlists; b += kXcds) list_at[b] = i++;
  }
  if (nlists > kMaxLists || nslots > kMaxSlots || splits.size() > (size_t)kMaxLists ||
      pieces.size() > tiles.size() + kMaxLists)
    return mi_idx_fail(MI_IDX_ECAPACITY, "plan_prefill: %d lists, %d slots exceed the plan",
                       nlists, nslots);
  const size_t piece_off = plan_words(nlists, 0, 0);
  const size_t split_off = plan_words(nlists, pieces.size(), 0);
  const size_t words = plan_words(nlists, pieces.size(), splits.size());
  if (4 * words > plan_bytes)
    return mi_idx_fail(MI_IDX_ECAPACITY, "plan_prefill: %zu pieces exceed the plan", pieces.size());
  int32_t *st = static_cast<int32_t *>(staging_host_pinned);
  std::fill(st, st + words, 0);
  st[0] = nlists;
  st[1] = M;
  st[2] = num_heads;
  st[3] = nchunks;
  st[4] = (int32_t)pieces.size();
  st[5] = (int32_t)piece_off;
  st[6] = (int32_t)splits.size();
  st[7] = (int32_t)split_off;
  st[8] = nslots;
  for (int b = 0; b < nlists; ++b) {
    const int i = list_at[b];
    const int end = i + 1 < nlists ? list_first[i + 1] : (int)pieces.size();
    st[kPreHeaderInts + 4 * b] = list_first[i];
    st[kPreHeaderInts + 4 * b + 1] = end - list_first[i];
  }
  for (size_t i = 0; i < pieces.size(); ++i) {
    int32_t *w = st + piece_off + 8 * i;
    const Tile &t = tiles[pieces[i].tile];
    w[0] = t.r;
    w[1] = t.row0;
    w[2] = t.nrows;
    w[3] = pieces[i].pa;
    w[4] = pieces[i].pe;
    w[5] = slot[i];
  }
  for (size_t i = 0; i < splits.size(); ++i) {
    int32_t *w = st + split_off + 8 * i;
    const Tile &t = tiles[splits[i].tile];
    w[0] = t.r;
    w[1] = t.row0;
    w[2] = t.nrows;
    w[3] = splits[i].first_slot;
    w[4] = splits[i].nslots;
  }
  launch_out_host->num_lists = nlists;
  launch_out_host->num_pieces = (int32_t)pieces.size();
  launch_out_host->num_merges = (int32_t)splits.size();
  launch_out_host->num_chunks = nchunks;
  hipError_t e = hipMemcpyAsync(plan, staging_host_pinned, 4 * words, hipMemcpyHostToDevice,
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
                                         int max_pages, float scale, void *plan,
                                         size_t plan_bytes, const mi_idx_prefill_launch *launch,
                                         void *workspace, size_t ws_bytes, int32_t *topk_out,
                                         float *scores_out, void *stream) {
  mi_idx_clear_error();
  if (num_heads < 1 || num_heads > MI_IDX_MAX_HEADS)
    return mi_idx_fail(MI_IDX_EUNSUPPORTED, "score_topk_prefill: num_heads %d outside 1..8",
                       num_heads);
  if (!launch) return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: null launch");
  const int num_tiles = launch->num_lists, num_pieces = launch->num_pieces,
            num_merges = launch->num_merges;
  if (num_reqs < 0 || total_q < 0 || max_pages < 0 || num_tiles < 0 || num_merges < 0 ||
      num_pieces < num_tiles)
    return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: negative size or fewer pieces than "
                                      "work lists");
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
  if (num_tiles > kMaxLists || num_merges > kMaxLists ||
      4 * plan_words(num_tiles, num_pieces, num_merges) > plan_bytes)
    return mi_idx_fail(MI_IDX_ECAPACITY, "score_topk_prefill: %d lists, %d pieces, %d merges "
                       "exceed the plan", num_tiles, num_pieces, num_merges);
  if (num_merges > 0) {
    if (!workspace || ((uintptr_t)workspace % 16))
      return mi_idx_fail(MI_IDX_EINVAL, "score_topk_prefill: the plan splits tiles and needs a "
                                        "16-byte aligned workspace");
    if (ws_bytes < mi_idx_prefill_workspace_bytes())
      return mi_idx_fail(MI_IDX_ECAPACITY, "score_topk_prefill: ws_bytes %zu < %zu", ws_bytes,
                         mi_idx_prefill_workspace_bytes());
  }
  const dim3 grid(num_tiles), block(64 * kPrefillStreams * (16 / kPrefillCgw));
  uint32_t *err = static_cast<uint32_t *>(plan) + kPreErrWord;
  const uint8_t *qb = static_cast<const uint8_t *>(q);
  uint64_t *lists = static_cast<uint64_t *>(workspace);
#define MI_IDX_LAUNCH_PRE(SC, BF)                                                              \
  hipLaunchKernelGGL((prefill_score_kernel<kPrefillCgw, kPrefillStreams, SC, BF, MI_IDX_ONE>), grid, block, \
                     0, (hipStream_t)stream, qb, pages, num_blocks, block_table, bt_stride,    \
                     cu_seqlens_q, seq_lens, context_lens, num_reqs, total_q, num_heads,       \
                     max_pages, scale, (const int32_t *)plan, lists, topk_out, scores_out,      \
                     err)
  // one whole tile per work list: the single-pass instantiation
  const bool one = num_pieces == num_tiles && num_merges == 0;
  if (one) {
#define MI_IDX_ONE true
    if (q_dtype == MI_IDX_Q_BF16) {
      if (scores_out) MI_IDX_LAUNCH_PRE(true, true);
      else MI_IDX_LAUNCH_PRE(false, true);
    } else {
      if (scores_out) MI_IDX_LAUNCH_PRE(true, false);
      else MI_IDX_LAUNCH_PRE(false, false);
    }
#undef MI_IDX_ONE
  } else {
#define MI_IDX_ONE false
    if (q_dtype == MI_IDX_Q_BF16) {
      if (scores_out) MI_IDX_LAUNCH_PRE(true, true);
      else MI_IDX_LAUNCH_PRE(false, true);
    } else {
      if (scores_out) MI_IDX_LAUNCH_PRE(true, false);
      else MI_IDX_LAUNCH_PRE(false, false);
    }
#undef MI_IDX_ONE
  }
#undef MI_IDX_LAUNCH_PRE
  if (num_merges > 0)
    hipLaunchKernelGGL(prefill_merge_kernel, dim3(num_merges), dim3(kTileCols), 0,
                       (hipStream_t)stream, cu_seqlens_q, seq_lens, context_lens, num_reqs,
                       total_q, num_heads, max_pages, (const int32_t *)plan,
                       (const uint64_t *)lists, topk_out, err);
  return mi_idx_check_launch("score_topk_prefill");
}
