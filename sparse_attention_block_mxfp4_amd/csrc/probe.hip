// HBM read and matrix-core ceilings of one MI355X, measured next to the
// specification figures (libmi_idx_probe.so, include/mi_idx_probe.h).
//
// read_stream: every byte of a buffer once, as 16-byte loads with
// consecutive lanes on consecutive addresses -- the best case of a read.
// read_pages: whole 8704-byte index-K pages in a caller-given order (a random
// permutation stands for a block table's scattered physical pages), each
// wave reading its pages' 544 16-byte chunks with every load of a page in
// flight at once and the next page's issued before the current one is
// consumed -- the access pattern the decode scorer's page walk reduces to.
// Both fold what they read into one word per thread and store it only when
// it equals a value the caller never passes, so the loads are kept and the
// writes are (almost) nothing.
//
// The matrix-core ceiling of the prefill scorer is measured the same way
// (mfma): every wave issues the exact MFMA instruction the scorer uses, either
// as eight independent accumulating chains (the instruction's own rate) or as
// the scorer's inner pattern -- a zeroed accumulator per tile whose four
// outputs are folded into a running maximum with max3 -- with the shader
// clock and the constant-rate wall clock read around the loop, so the clock
// the chip holds under matrix load is measured too.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mi_idx_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kPageBytes = 8704;
constexpr int kPageChunks = kPageBytes / 16;                // 544
constexpr int kChunksPerLane = (kPageChunks + 63) / 64;     // 9 (the last partial)

// Workgroup b reads 32 KB chunks b, b + grid, ...: load u of thread t takes
// 16 bytes at chunk + 16 (256 u + t), so each load instruction of the
// workgroup covers 4 KB of consecutive addresses.
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4 *__restrict__ buf,
                                                               int64_t n16, uint32_t never,
                                                               uint32_t *__restrict__ sink) {
  constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;   // 16-byte units per chunk
  uint32_t acc = 0;
  const int64_t full = n16 / kChunk;
  for (int64_t c = blockIdx.x; c < full; c += gridDim.x) {
    const u32x4 *p = buf + c * kChunk + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = full * kChunk + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const u32x4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == never) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void read_pages_kernel(const uint8_t *__restrict__ pages,
                                                              int64_t num_pages,
                                                              const int32_t *__restrict__ order,
                                                              int64_t n_order, int per_wave,
                                                              uint32_t never,
                                                              uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t first = wave * per_wave;
  if (first >= n_order) return;
  const int64_t last = first + per_wave < n_order ? first + per_wave : n_order;
  uint32_t acc = 0;
  // chunk c of the lane: lane + 64 c (the last one clamped to the page end)
  auto issue = [&](int64_t k, u32x4 (&r)[kChunksPerLane]) {
    int64_t id = order[k];
    id = id < 0 ? 0 : (id >= num_pages ? num_pages - 1 : id);   // stay inside the pool
    const u32x4 *pg = reinterpret_cast<const u32x4 *>(pages + id * kPageBytes);
#pragma unroll
    for (int c = 0; c < kChunksPerLane; ++c) {
      const int ch = lane + 64 * c;
      r[c] = pg[ch < kPageChunks ? ch : kPageChunks - 1];
    }
  };
  u32x4 a[kChunksPerLane], b[kChunksPerLane];
  issue(first, a);
  for (int64_t k = first; k < last; k += 2) {
    issue(k + 1 < last ? k + 1 : k, b);
#pragma unroll
    for (int c = 0; c < kChunksPerLane; ++c) acc ^= a[c].x ^ a[c].y ^ a[c].z ^ a[c].w;
    issue(k + 2 < last ? k + 2 : last - 1, a);
#pragma unroll
    for (int c = 0; c < kChunksPerLane; ++c) acc ^= b[c].x ^ b[c].y ^ b[c].z ^ b[c].w;
  }
  if (acc == never) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

constexpr int kChains = 8;   // MFMAs per loop iteration, independent of each other

// One MFMA of the probed instruction: kKind 0 is
// v_mfma_scale_f32_16x16x128_f8f6f4 with A FP4 E2M1 under E8M0 scale `sc`
// and B FP8 E4M3 (65 536 flops); kKind 1 is v_mfma_f32_16x16x32_bf16
// (16 384), on the same registers reinterpreted (`sc` unused).
template <int kKind>
__device__ __forceinline__ v4f probe_mfma(const u32x4 &a, const v8i &b, const v4f &acc, int sc) {
  if constexpr (kKind == 0) {
    const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc, 4, 0, 0, sc, 0, 127);
  } else {
    const u32x4 bw = {(uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, bw), acc, 0, 0, 0);
  }
}

__device__ __forceinline__ float fold_max(float m, const v4f &c) {
  return __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(m, c.x),
      __builtin_elementwise_maximum(__builtin_elementwise_maximum(c.y, c.z), c.w));
}

// Operands: A words a_word ^ j, B words b_word ^ (j << 8) for the j-th A and
// B register set (the caller picks small values, so the accumulating chains
// stay finite).  An accumulating chain cannot be hoisted out of the loop;
// in the fold mode the A scale (scaled MFMA) or one A word updated in place
// (bf16, one VALU op per tile as the scorer's conversion has) moves with the
// iteration, so no MFMA is loop-invariant.
//  kFold false: 8 accumulating chains, 8 A sets, one B set.
//  kFold true: the scorer's page loop -- two tiles (A sets) per iteration
//  against four column groups (B sets), each MFMA on a zeroed accumulator;
//  tile 1's MFMAs issue while tile 0's outputs are folded into the four
//  running maxima, and the next iteration's tile 0 while tile 1's are.
template <int kKind, bool kFold>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, uint32_t a_word, uint32_t b_word,
                                                        uint32_t never, uint32_t *__restrict__ sink,
                                                        uint64_t *__restrict__ clocks) {
  u32x4 a[kChains];
  v8i b[4];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    const uint32_t w = a_word ^ (uint32_t)j;
    a[j] = u32x4{w, w, w, w};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int w = (int)(b_word ^ ((uint32_t)j << 8));
    b[j] = v8i{w, w, w, w, w, w, w, w};
  }
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f c[kChains];
  float m[4];
#pragma unroll
  for (int j = 0; j < kChains; ++j) c[j] = zero;
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = -INFINITY;
  const uint64_t t0 = __builtin_readcyclecounter();
  const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    const int sc = 120 + (it & 7);
    if constexpr (kFold && kKind == 1) {
      a[0].x = a_word ^ (uint32_t)sc;
      a[1].x = a_word ^ 1u ^ (uint32_t)sc;
    }
    if constexpr (kFold) {
      // c[0..3]: tile 0 of this iteration, c[4..7]: tile 1 (of the last
      // iteration until overwritten)
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        c[cg] = probe_mfma<kKind>(a[0], b[cg], zero, sc);
        m[cg] = fold_max(m[cg], c[4 + cg]);
      }
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        c[4 + cg] = probe_mfma<kKind>(a[1], b[cg], zero, sc);
        m[cg] = fold_max(m[cg], c[cg]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kChains; ++j) c[j] = probe_mfma<kKind>(a[j], b[0], c[j], sc);
    }
  }
  const uint64_t t1 = __builtin_readcyclecounter();
  const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
  float f = 0.f;
  if constexpr (kFold) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f += fold_max(m[j], c[4 + j]);
  } else {
#pragma unroll
    for (int j = 0; j < kChains; ++j) f += c[j].x + c[j].y + c[j].z + c[j].w;
  }
  const uint32_t bits = __builtin_bit_cast(uint32_t, f);
  if (bits == never) sink[blockIdx.x * kThreads + threadIdx.x] = bits;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = w1 - w0;
  }
}

}  // namespace

extern "C" int mi_idx_probe_device(int *cus, int *clock_khz, int *wall_clock_khz) {
  if (!cus || !clock_khz || !wall_clock_khz) return 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess ||
      hipDeviceGetAttribute(wall_clock_khz, hipDeviceAttributeWallClockRate, dev) !=
          hipSuccess) {
    (void)hipGetLastError();
    return 4;
  }
  return 0;
}

extern "C" int mi_idx_probe_mfma(int kind, int fold, int iters, int blocks_per_cu,
                                 uint32_t a_word, uint32_t b_word, uint32_t *sink,
                                 int64_t sink_words, uint64_t *clocks, void *stream) {
  if (kind < 0 || kind > 1 || fold < 0 || fold > 1 || iters < 1 || blocks_per_cu < 1 ||
      blocks_per_cu > 8 || !sink || !clocks || ((uintptr_t)sink % 4) || ((uintptr_t)clocks % 8))
    return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 4;
  }
  const int64_t blocks = (int64_t)cus * blocks_per_cu;
  if (sink_words < blocks * kThreads) return 3;
  auto kern = kind == 0 ? (fold ? mfma_kernel<0, true> : mfma_kernel<0, false>)
                        : (fold ? mfma_kernel<1, true> : mfma_kernel<1, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, iters,
                     a_word, b_word, 0xFFFFFFFFu, sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int mi_idx_probe_read_stream(const void *buf, int64_t bytes, int blocks_per_cu,
                                        uint32_t *sink, int64_t sink_words, void *stream) {
  if (!buf || !sink || bytes < 16 || ((uintptr_t)buf % 16) || ((uintptr_t)sink % 4) ||
      blocks_per_cu < 1 || blocks_per_cu > 64)
    return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 4;
  }
  const int64_t blocks = (int64_t)cus * blocks_per_cu;
  if (sink_words < blocks * kThreads) return 3;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, static_cast<const u32x4 *>(buf), bytes / 16,
                     0xFFFFFFFFu, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int mi_idx_probe_read_pages(const uint8_t *pages, int64_t num_pages,
                                       const int32_t *order, int64_t n_order, int per_wave,
                                       uint32_t *sink, int64_t sink_words, void *stream) {
  if (!pages || !order || !sink || num_pages <= 0 || n_order <= 0 || per_wave < 1 ||
      ((uintptr_t)pages % 16))
    return 1;
  const int64_t waves = (n_order + per_wave - 1) / per_wave;
  const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7FFFFFFF || sink_words < blocks * kThreads) return 3;
  hipLaunchKernelGGL(read_pages_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, pages, num_pages, order, n_order, per_wave, 0xFFFFFFFFu,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
