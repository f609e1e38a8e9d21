// HBM read ceilings of one MI355X, measured next to the decode phase's
// 8 TB/s specification figure (libmi_idx_probe.so, include/mi_idx_probe.h).
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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mi_idx_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

}  // namespace

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
