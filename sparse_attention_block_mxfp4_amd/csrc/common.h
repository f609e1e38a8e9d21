// Shared device helpers of the MXFP4 lightning indexer kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mi_idx.h"

namespace mi_idx {

constexpr int kPageTokens = MI_IDX_PAGE_TOKENS;   // tokens per page
constexpr int kDim = MI_IDX_HEAD_DIM;             // index head dim
constexpr int kTokenBytes = MI_IDX_TOKEN_BYTES;   // 64 code bytes + 4 scales
constexpr int kPageBytes = MI_IDX_PAGE_BYTES;     // 8704
constexpr int kHist = MI_IDX_HISTORY;             // ranked history slots
constexpr int kTopk = MI_IDX_TOPK;                // + the local page

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
// 16 bytes that are only 4-byte aligned (a token's code bytes start at 68*t).
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 16x16x128 block-scaled MFMA: A = 16 tokens of E2M1 codes (one 32-dim
// scale block per lane), B = 16 query columns of E4M3, fp32 result.
//   A lane l: token (l & 15), dims [32*(l>>4), +32), 16 bytes, low nibble
//             first; its E8M0 byte scales those 32 dims.
//   B lane l: column (l & 15); bytes 0..15 = dims [16*(l>>4), +16) and bytes
//             16..31 = dims [64 + 16*(l>>4), +16) (the FP8 operand order);
//             scale byte 127 (x1).
//   C lane l: rows 4*(l>>4) + {0..3} (tokens), column (l & 15).
__device__ __forceinline__ v4f mfma_fp4_fp8(const u32x4 &a, const v8i &b,
                                            uint32_t a_scale) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v4f z = {0.f, 0.f, 0.f, 0.f};
  // format codes: 4 = FP4 E2M1 (A), 0 = FP8 E4M3 (B)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, z, 4, 0, 0,
                                                          (int)a_scale, 0, 127);
}

// As mfma_fp4_fp8, the A scale taken from byte kSel of the 32-bit word
// scales (the MFMA's scale byte select).
template <int kSel>
__device__ __forceinline__ v4f mfma_fp4_fp8_sel(const u32x4 &a, const v8i &b, uint32_t scales) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, z, 4, 0, kSel, (int)scales, 0,
                                                          127);
}

// ---- bfloat16 index-Q ------------------------------------------------------
// The block-scaled MFMA takes FP8/FP6/FP4 operands only, so a bf16 query runs
// on the bf16 MFMA: the page's FP4 codes are converted to bf16 (exactly: an
// E2M1 value times a power of two is a bf16 value) and a 16x16x128 tile
// becomes four 16x16x32 steps.  A lane keeps its usual 16 code bytes (the 32
// dims of one scale block); k-step s takes their dword s (8 dims), and the
// query operand of k-step s holds the same 8 dims -- a permutation of the
// summation order, which the dot product does not see.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// E8M0 byte -> the fp32 factor 2^(b-127) (b = 0: 2^-127, a subnormal;
// b = 255: NaN).
__device__ __forceinline__ float e8m0_scale(uint32_t b) {
  b &= 0xFFu;
  const uint32_t bits = b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : (b << 23));
  return __uint_as_float(bits);
}

// Eight E2M1 codes (one dword, low nibble first) -> eight bf16 values times
// the scale factor.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float sf) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 3);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// One 16x16x128 tile with a bf16 query: A as for mfma_fp4_fp8 (16 code bytes
// and the E8M0 byte of the lane's 32-dim block); b[s] = the query's 8 bf16
// values of dims 32*(l>>4) + 8s .. +8 for column (l & 15).  Same C layout.
__device__ __forceinline__ v4f mfma_fp4_bf16(const u32x4 &a, const u32x4 (&b)[4],
                                             uint32_t a_scale) {
  const float sf = e8m0_scale(a_scale);
  v4f c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16(a.x, sf),
                                              __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16(a.y, sf),
                                              __builtin_bit_cast(bf16x8, b[1]), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16(a.z, sf),
                                              __builtin_bit_cast(bf16x8, b[2]), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16(a.w, sf),
                                              __builtin_bit_cast(bf16x8, b[3]), c, 0, 0, 0);
  return c;
}

// Query operand of a bf16 column: qrow = the 128 bf16 values (256 bytes,
// 16-byte aligned) of the column's (row, head).
__device__ __forceinline__ void load_q_bf16(const uint8_t *qrow, int g, u32x4 (&b)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    b[s] = *reinterpret_cast<const u32x4 *>(qrow + 2 * (32 * g + 8 * s));
}

// Page maxima propagate NaN: a token whose q.k is NaN (an E8M0 scale byte
// 0xFF, a NaN query element) makes its page's score NaN, which the selection
// keys rank below every number.  IEEE 754-2019 maximum (gfx950:
// v_maximum3_f32, three operands like v_max3_f32), never the NaN-dropping
// fmax.
__device__ __forceinline__ float nmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float max4(const v4f &c) {
  return nmax(nmax(c.x, c.y), nmax(c.z, c.w));
}

// m = max(m, c.x, c.y, c.z, c.w) as two 3-input maxima.
__device__ __forceinline__ float fold4(float m, const v4f &c) {
  return nmax(nmax(nmax(nmax(m, c.x), c.y), c.z), c.w);
}

// Selection key: larger is better.  High word = the score's bits mapped to
// an unsigned order (NaN lowest, -0 folded into +0); low word = ~id so that
// equal scores prefer the lower id.  0 is "empty" (below every real key).
__device__ __forceinline__ uint64_t make_key(float s, int id) {
  uint32_t u = __float_as_uint(s);
  u = (u << 1) == 0u ? 0u : u;                                  // -0 -> +0
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  ord = (u & 0x7FFFFFFFu) > 0x7F800000u ? 0u : ord;             // NaN lowest (bits)
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ int key_id(uint64_t k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

// Sorted (descending) list of the best kHist keys, held in registers.
struct TopList {
  uint64_t k[kHist];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < kHist; ++i) k[i] = 0ull;
  }
  // Insert x with no branch (x = 0 leaves the list unchanged), so the caller's
  // basic block stays whole for the scheduler.  Every slot compares with x
  // at once and then takes its own key, x, or its upper neighbour's key: no
  // chain of dependent compare-exchanges through the list.
  __device__ __forceinline__ void insert_nb(uint64_t x) {
    bool c[kHist];
#pragma unroll
    for (int i = 0; i < kHist; ++i) c[i] = k[i] > x;
#pragma unroll
    for (int i = kHist - 1; i >= 1; --i) k[i] = c[i] ? k[i] : (c[i - 1] ? x : k[i - 1]);
    k[0] = c[0] ? k[0] : x;
  }
  // Insert x (no-op when x does not beat the current 15th key).
  __device__ __forceinline__ void insert(uint64_t x) {
    if (x <= k[kHist - 1]) return;
#pragma unroll
    for (int i = 0; i < kHist; ++i) {
      uint64_t hi = k[i] > x ? k[i] : x;
      uint64_t lo = k[i] > x ? x : k[i];
      k[i] = hi;
      x = lo;
    }
  }
};

// Max of v over lanes l and l^32 (resp. l^16), through gfx950's VALU lane
// swaps: for every lane the swap returns {own, partner} in some order.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Lanes 0..31 get max(a, a of lane+32), lanes 32..63 get max(b, b of lane-32).
__device__ __forceinline__ float max_split32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Even 16-lane rows get max(a, a of the next row), odd rows get max(b, b of
// the previous row).
__device__ __forceinline__ float max_split16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Local page of a row at position p, or -1 for a row that gets no selection:
// a padding row (p < 0) or a row whose causal history runs past the
// max_pages block-table columns the caller vouches for (refused: its history
// cannot be read).
__device__ __forceinline__ int local_page(int p, int max_pages) {
  return (p >= 0 && (p >> 7) <= max_pages) ? (p >> 7) : -1;
}

// Write one (row, head) output: ranked ids, -1 padding, then the local page.
__device__ __forceinline__ void write_row(int32_t *dst, const TopList &t,
                                          int L) {
  int32_t v[kTopk];
#pragma unroll
  for (int i = 0; i < kHist; ++i) v[i] = (L >= 0 && t.k[i] != 0ull) ? key_id(t.k[i]) : -1;
  v[kHist] = L >= 0 ? L : -1;
  int4 *d4 = reinterpret_cast<int4 *>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d4[i] = make_int4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

}  // namespace mi_idx

// Host-side status helpers (defined in api.hip).
int mi_idx_fail(int status, const char *fmt, ...);
int mi_idx_check_launch(const char *what);
void mi_idx_clear_error();
