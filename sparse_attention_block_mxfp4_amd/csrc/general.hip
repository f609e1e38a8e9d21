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
//     prefix (tokens 0 .. p % 128), on the scorers' block-scaled MFMA: a wave
//     takes up to 64 (row, head) columns (64 // H consecutive prefill rows,
//     or one decode request's rows) and runs one 8-tile pass per distinct
//     local page among them, each column keeping only its own page's tokens
//     up to its position;
//   select_general_kernel: per (row, head), one wave finds the
//     topk - force_begin - force_end best pages strictly between the two
//     windows (the local page among them when the trailing window is empty)
//     by an exact radix select over the ordered score bits, ties at the
//     threshold going to the lower ids, and writes them in ascending id order
//     between the forced windows.
#include <cmath>

#include "common.h"

namespace mi_idx {

constexpr int kLocalWaves = 4;
constexpr int kSelWaves = 4;

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

// Wave w of the grid takes rows t0 = w * rpw .. + rpw - 1 (rpw = 64 / H
// prefill rows, or one decode request's query_len rows); column
// cg * 16 + (lane & 15) of the wave is (row t0 + col / H, head col % H), as
// the B operand of four 16x16x128 MFMAs per token tile.  A pass over one
// page P loads each 16-token tile once (the A operand: token tile * 16 +
// (lane & 15), the 32 dims of lane group lane >> 4 and their E8M0 scale) and
// folds output row 4 (lane >> 4) + i -- token tile * 16 + 4 (lane >> 4) + i
// -- into the column's running maximum if the column's local page is P and
// the token is within its causal prefix.  A column with no readable local
// page (padding row, page past max_pages, invalid block-table entry) gets
// NaN, as a page max over a NaN token would.
template <bool kBf16>
__global__ __launch_bounds__(64 * kLocalWaves) void local_score_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ pages, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ ctx, int num_reqs, int query_len, int64_t total_rows, int H,
    int max_pages, float scale, float *__restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t16 = lane & 15, g = lane >> 4;
  // rows per wave: 64 // H consecutive prefill rows (one or two local pages),
  // or the query_len rows of one decode request (their own local pages; a
  // wave spanning several requests would walk their pages one after another)
  const int rpw = cu == nullptr ? query_len : 64 / H;
  const int64_t t0 = ((int64_t)blockIdx.x * kLocalWaves + wave) * rpw;
  if (t0 >= total_rows) return;   // whole wave; the kernel has no barrier
  // the request of the wave's first row (prefill rows), found once
  int r0 = 0;
  if (cu != nullptr) {
    int p0 = 0;
    row_position(t0, seq_lens, cu, ctx, num_reqs, query_len, r0, p0);
    r0 = __builtin_amdgcn_readfirstlane(r0);
  }
  // The four column groups' rows are resolved in phases, each phase's loads
  // for all four issued together: query operands; the request (rows are
  // consecutive: r0, or a later request past its first row, which is rare);
  // the position; the block-table entry.
  int64_t phys[4];
  int pmod[4];
  int64_t Tc[4];
  int hc[4];
  bool live[4];
  v8i bq[kBf16 ? 1 : 4];
  u32x4 bqh[kBf16 ? 4 : 1][4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const int col = cg * 16 + t16;
    const int rl = col / H;
    hc[cg] = col - rl * H;
    Tc[cg] = t0 + rl;
    live[cg] = rl < rpw && Tc[cg] < total_rows;
    phys[cg] = live[cg] ? -1 : -2;   // -2: no column here, -1: a row without a readable page
    pmod[cg] = 0;
    if constexpr (kBf16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) bqh[cg][k] = u32x4{0u, 0u, 0u, 0u};
    } else {
      bq[cg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (live[cg]) {
      const int64_t T = Tc[cg];
      if constexpr (kBf16) {
        load_q_bf16(q + (T * H + hc[cg]) * (2 * kDim), g, bqh[cg]);
      } else {
        const uint8_t *qp = q + (T * H + hc[cg]) * kDim;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(qp + 16 * g);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(qp + 64 + 16 * g);
        bq[cg] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    }
  }
  int rc[4], pc[4];
  if (cu == nullptr) {
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) rc[cg] = live[cg] ? (int)(Tc[cg] / query_len) : 0;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
      pc[cg] = live[cg] ? seq_lens[rc[cg]] - query_len +
                              (int)(Tc[cg] - (int64_t)rc[cg] * query_len)
                        : -1;
  } else {
    const int cu1 = r0 + 1 < num_reqs ? cu[r0 + 1] : 0x7FFFFFFF;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      int r = r0;
      if (live[cg] && Tc[cg] >= cu1) {
        r = r0 + 1;
        while (r + 1 < num_reqs && cu[r + 1] <= Tc[cg]) ++r;
      }
      rc[cg] = r;
    }
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
      pc[cg] = live[cg] ? ctx[rc[cg]] + (int)(Tc[cg] - cu[rc[cg]]) : -1;
  }
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const int p = pc[cg];
    if (live[cg] && p >= 0 && (p >> 7) < max_pages) {
      const int32_t v = block_table[(int64_t)rc[cg] * bt_stride + (p >> 7)];
      if (v >= 0 && (int64_t)v < num_blocks) phys[cg] = v;
    }
    pmod[cg] = p & (kPageTokens - 1);
  }
  float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  bool todo[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) todo[cg] = phys[cg] >= 0;
  for (;;) {
    // the next page: the first pending one of the lowest lane with any
    int64_t cand = -1;
#pragma unroll
    for (int cg = 3; cg >= 0; --cg)
      if (todo[cg]) cand = phys[cg];
    const uint64_t any = __ballot(cand >= 0);
    if (any == 0) break;
    const int src = __builtin_ctzll(any);
    const int64_t P = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                     (int)((uint64_t)cand >> 32), src) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)cand, src));
    bool use[4];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
      use[cg] = todo[cg] && phys[cg] == P;
      todo[cg] = todo[cg] && !use[cg];
    }
    const uint8_t *pg = pages + P * kPageBytes;
#pragma unroll
    for (int tl = 0; tl < 8; ++tl) {
      const uint8_t *tp = pg + (tl * 16 + t16) * kTokenBytes;
      const u32x4a4 a4 = *reinterpret_cast<const u32x4a4 *>(tp + 16 * g);
      const u32x4 a = {a4.x, a4.y, a4.z, a4.w};
      const uint32_t sc = tp[64 + g];
      const int tok0 = tl * 16 + 4 * g;
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        v4f c;
        if constexpr (kBf16) c = mfma_fp4_bf16(a, bqh[cg], sc);
        else c = mfma_fp4_fp8(a, bq[cg], sc);
        const int lim = use[cg] ? pmod[cg] : -1;
        c.x = tok0 <= lim ? c.x : -INFINITY;
        c.y = tok0 + 1 <= lim ? c.y : -INFINITY;
        c.z = tok0 + 2 <= lim ? c.z : -INFINITY;
        c.w = tok0 + 3 <= lim ? c.w : -INFINITY;
        m[cg] = fold4(m[cg], c);
      }
    }
  }
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    const float v = max_xor32(max_xor16(m[cg]));
    const int col = cg * 16 + t16;
    const int rl = col / H, h = col - rl * H;
    if (g == 0 && phys[cg] != -2)
      out[(t0 + rl) * H + h] = phys[cg] >= 0 ? scale * v : __uint_as_float(0x7FC00000u);
  }
}

// The score's order bits: the high word of the selection key (NaN lowest,
// -0 as +0), so that comparing them compares the scores.
__device__ __forceinline__ uint32_t score_order(float s) {
  return (uint32_t)(make_key(s, 0) >> 32);
}

// The LDS operations of one wave take effect in program order; this keeps
// the compiler from moving them across the phases of a radix pass.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Wave-wide scans in the lanes themselves (DPP), with no LDS round trip:
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from
// outside the row read 0), then a row's last lane broadcast into the next
// row (rows 1 and 3) and lane 31 into rows 2 and 3.  A disabled row keeps 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, true);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over lanes 0 .. lane.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  x += dpp0<kRowShr1>(x);
  x += dpp0<kRowShr2>(x);
  x += dpp0<kRowShr4>(x);
  x += dpp0<kRowShr8>(x);
  x += dpp0<kRowBcast15, 0xA>(x);
  x += dpp0<kRowBcast31, 0xC>(x);
  return x;
}

// Maximum over the wave (0 is the identity: the values are unsigned).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, dpp0<kRowShr1>(x));
  x = max(x, dpp0<kRowShr2>(x));
  x = max(x, dpp0<kRowShr4>(x));
  x = max(x, dpp0<kRowShr8>(x));
  x = max(x, dpp0<kRowBcast15, 0xA>(x));
  x = max(x, dpp0<kRowBcast31, 0xC>(x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Candidate keys of a row, visited in id order as (id = c0 + lane + 64 i),
// slots past the last candidate holding key 0: held in registers (up to
// 64 * NK candidates) ...
template <int NK>
struct RegKeys {
  uint32_t k[NK];
  int c0, c1, lane;
  template <class F>
  __device__ __forceinline__ void each(F &&f) const {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (c0 + 64 * i >= c1) break;
      const int j = c0 + lane + 64 * i;
      f(k[i], j, j < c1);
    }
  }
};

// ... or read again from the score row at every visit (longer rows).
struct StreamKeys {
  const float *srow;
  float lsc;
  int L, c0, c1, lane;
  template <class F>
  __device__ __forceinline__ void each(F &&f) const {
    // four slots' loads in flight at once, at addresses clamped into the
    // row's L >= 1 history scores
    for (int j0 = c0; j0 < c1; j0 += 256) {
      float raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[u] = srow[min(j0 + 64 * u + lane, L - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j0 + 64 * u >= c1) break;
        const int j = j0 + 64 * u + lane;
        const bool v = j < c1;
        f(v ? score_order(j < L ? raw[u] : lsc) : 0u, j, v);
      }
    }
  }
};

// The take best candidates of one row (take < the number of candidates),
// written ascending to dst.  An exact radix select on the order bits: bits
// above the highest bit where the candidates differ are common; from there
// 8-bit digits, each pass counting the keys that match the prefix found so
// far in a 256-bin LDS histogram (a key that does not match counts in a junk
// bin of its lane's, so the pass has no branch) and keeping the bin that
// holds the take-th largest, until that bin is taken whole or every bit is
// fixed.  Then a candidate is taken if its masked bits exceed the prefix, or
// equal it and it is among the first `rest` such candidates in id order.
// The padding slots (key 0, ids past every candidate) take part in the
// counts: they tie with the lowest possible key and come last in id order,
// and take < the candidates, so the take-th largest is a candidate's key, a
// bin holding padding is never taken whole, and no padding slot is chosen.
template <class Keys>
__device__ __forceinline__ void select_row(const Keys &keys, uint32_t take, uint32_t *h,
                                           int32_t *dst, int lane) {
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  keys.each([&](uint32_t k, int, bool v) {
    kmax = max(kmax, k);
    kmin = min(kmin, v ? k : 0xFFFFFFFFu);
  });
  kmax = wave_max(kmax);
  kmin = ~wave_max(~kmin);
  const uint32_t diff = kmax ^ kmin;
  // inbin: keys matching the final prefix; unknown (every candidate equal)
  // counts as ties
  uint32_t prefix = kmax, pmask = 0xFFFFFFFFu, rest = take, inbin = 0xFFFFFFFFu;
  if (diff != 0u) {
    const int hb = 31 - __builtin_clz(diff);
    pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    prefix = kmax & pmask;
    int sh = max(hb - 7, 0);
    for (;;) {
      *reinterpret_cast<u32x4 *>(h + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
      h[256 + lane] = 0u;
      wave_lds_sync();
      keys.each([&](uint32_t k, int, bool) {
        atomicAdd(&h[(k & pmask) == prefix ? (k >> sh) & 255u : 256u + lane], 1u);
      });
      wave_lds_sync();
      const u32x4 hb4 = *reinterpret_cast<const u32x4 *>(h + 4 * lane);
      const uint32_t mine = hb4.x + hb4.y + hb4.z + hb4.w;
      // keys in this lane's bins and every higher lane's
      const uint32_t incl = wave_prefix_sum(mine);
      const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl + mine;
      const uint32_t higher = above - mine;
      const bool here = higher < rest && rest <= above;   // exactly one lane
      uint32_t bin = 0u, nrest = 0u, nin = 0u;
      if (here) {
        const uint32_t hv[4] = {hb4.x, hb4.y, hb4.z, hb4.w};
        uint32_t c = higher;
        bin = 4u * lane;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if (c + hv[i] >= rest) {
            bin = 4u * lane + i;
            nin = hv[i];
            break;
          }
          c += hv[i];
        }
        nrest = rest - c;
      }
      const int src = __builtin_ctzll(__ballot(here));
      bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
      rest = (uint32_t)__builtin_amdgcn_readlane((int)nrest, src);
      inbin = (uint32_t)__builtin_amdgcn_readlane((int)nin, src);
      prefix = (prefix & ~(255u << sh)) | (bin << sh);
      pmask |= 255u << sh;
      if (rest == inbin || sh == 0) break;
      sh = max(sh - 8, 0);
      wave_lds_sync();
    }
  }
  uint32_t base = 0u;
  if (rest == inbin) {   // the threshold bin is taken whole: no tie to break
    keys.each([&](uint32_t k, int j, bool) {
      const bool sel = (k & pmask) >= prefix;
      const uint64_t ms = __ballot(sel);
      const uint32_t at = base + lanes_below(ms);
      if (sel && at < take) dst[at] = j;   // exactly take are chosen; the bound is a safety net
      base += (uint32_t)__builtin_popcountll(ms);
    });
  } else {
    uint32_t eqseen = 0u;
    keys.each([&](uint32_t k, int j, bool) {
      const uint32_t mk = k & pmask;
      const bool eq = mk == prefix;
      const uint64_t meq = __ballot(eq);
      const bool sel = mk > prefix || (eq && eqseen + lanes_below(meq) < rest);
      eqseen += (uint32_t)__builtin_popcountll(meq);
      const uint64_t ms = __ballot(sel);
      const uint32_t at = base + lanes_below(ms);
      if (sel && at < take) dst[at] = j;
      base += (uint32_t)__builtin_popcountll(ms);
    });
  }
}

// Per (row, head) = one wave: the forced windows and the take best
// candidates, ascending.  A row whose local page lies past scores_stride
// (not a scorer's output) is written as padding.
template <int NK>
__global__ __launch_bounds__(64 * kSelWaves) void select_general_kernel(
    const float *__restrict__ scores, int64_t stride, const float *__restrict__ local_scores,
    const int32_t *__restrict__ ranked, int64_t n, int topk, int init_blocks, int local_blocks,
    int max_k_tiles, int32_t *__restrict__ out) {
  __shared__ __align__(16) uint32_t s_hist[kSelWaves][256 + 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kSelWaves + wave;
  if (row >= n) return;   // whole wave; the kernel has no barrier
  const int L = ranked[row * kTopk + (kTopk - 1)];   // the row's local page, -1: padding
  int32_t *dst = out + row * topk;
  if (L < 0 || (int64_t)L > stride) {
    for (int i = lane; i < topk; i += 64) dst[i] = -1;
    return;
  }
  const int nvp = L + 1;
  if (nvp <= topk) {   // every valid page
    for (int i = lane; i < topk; i += 64) dst[i] = i < nvp ? i : -1;
    return;
  }
  const int fb = min(min(init_blocks, max_k_tiles), topk);
  const int fe = min(local_blocks, topk - fb);
  const int take = topk - fb - fe;
  const int c0 = fb, c1 = nvp - fe;   // candidates [c0, c1), take of them
  for (int i = lane; i < fb; i += 64) dst[i] = i;
  for (int i = lane; i < fe; i += 64) dst[fb + take + i] = nvp - fe + i;
  if (take == 0) return;
  const float *srow = scores + row * stride;
  const float lsc = c1 > L ? local_scores[row] : 0.f;   // the local page is a candidate
  if (c1 - c0 <= 64 * NK) {
    RegKeys<NK> keys;
    keys.c0 = c0;
    keys.c1 = c1;
    keys.lane = lane;
    // Every slot's load first, unconditional at an address clamped into the
    // row's L history scores (L >= 1 here), so all of them are in flight at
    // once; then the keys.  (Loads behind the slot tests went out one at a
    // time, each waited for before the next.)
    float raw[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (c0 + 64 * i >= c1) break;   // the slots past it are never visited
      raw[i] = srow[min(c0 + lane + 64 * i, L - 1)];
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (c0 + 64 * i >= c1) break;
      const int j = c0 + lane + 64 * i;
      keys.k[i] = j < c1 ? score_order(j < L ? raw[i] : lsc) : 0u;
    }
    select_row(keys, (uint32_t)take, s_hist[wave], dst + fb, lane);
  } else {
    const StreamKeys keys{srow, lsc, L, c0, c1, lane};
    select_row(keys, (uint32_t)take, s_hist[wave], dst + fb, lane);
  }
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
  // a decode request's query_len * num_heads <= 64 columns fit one wave
  const int rpw = prefill ? 64 / num_heads : query_len;
  const int64_t waves = (total_rows + rpw - 1) / rpw;
  const dim3 grid((unsigned)((waves + kLocalWaves - 1) / kLocalWaves)), block(64 * kLocalWaves);
  const uint8_t *qb = static_cast<const uint8_t *>(q);
  hipStream_t s = (hipStream_t)stream;
  if (q_dtype == MI_IDX_Q_BF16)
    hipLaunchKernelGGL(local_score_kernel<true>, grid, block, 0, s, qb, pages, num_blocks,
                       block_table, bt_stride, seq_lens, cu_seqlens_q, context_lens, num_reqs,
                       query_len, total_rows, num_heads, max_pages, scale, local_out);
  else
    hipLaunchKernelGGL(local_score_kernel<false>, grid, block, 0, s, qb, pages, num_blocks,
                       block_table, bt_stride, seq_lens, cu_seqlens_q, context_lens, num_reqs,
                       query_len, total_rows, num_heads, max_pages, scale, local_out);
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
  // Candidates per row <= scores_stride + 1: registers for up to 64 * NK of
  // them, longer rows re-read their scores at every pass.
  const dim3 grid((unsigned)((n + kSelWaves - 1) / kSelWaves)), block(64 * kSelWaves);
  hipStream_t s = (hipStream_t)stream;
  if (scores_stride + 1 <= 64 * 8)
    hipLaunchKernelGGL(select_general_kernel<8>, grid, block, 0, s, scores, scores_stride,
                       local_scores, ranked, n, topk, init_blocks, local_blocks, max_k_tiles, out);
  else if (scores_stride + 1 <= 64 * 16)
    hipLaunchKernelGGL(select_general_kernel<16>, grid, block, 0, s, scores, scores_stride,
                       local_scores, ranked, n, topk, init_blocks, local_blocks, max_k_tiles, out);
  else
    hipLaunchKernelGGL(select_general_kernel<32>, grid, block, 0, s, scores, scores_stride,
                       local_scores, ranked, n, topk, init_blocks, local_blocks, max_k_tiles, out);
  return mi_idx_check_launch("select_topk");
}
