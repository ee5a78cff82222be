// Streaming-read kernel: the bandwidth ceiling a one-launch read of a given
// size reaches on this device, measured beside the weight-streaming GEMMs
// so their roofline fraction can be read against both the published peak
// and what a plain read achieves.  Each work group reads one contiguous
// span with 16-byte non-temporal loads and folds what it read into one
// word, which is stored only when it equals `key` (so the loads cannot be
// dropped, and in practice nothing is written).

#include "common.h"
#include "internal.h"

#include <algorithm>

namespace sv {

// Measured on MI355X over reads of 117 MB to 1 GiB (fresh data each launch):
// contiguous spans per work group, 256 threads, batches of 16 loads per lane
// with the next batch in flight while one is folded, 2048 groups, came
// within 2% of the fastest of 20 shapes (256 to 1024 threads, 8 or 16 loads,
// 256 to 2048 groups, with and without the non-temporal hint) at every size.
constexpr int kProbeThreads = 256;
constexpr int kInFlight = 16;
constexpr unsigned kProbeGroups = 2048;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4* src, size_t n16,
                                                              uint32_t key, uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  constexpr size_t step = (size_t)kProbeThreads * kInFlight;
  uint32_t acc = 0;
  u32x4 cur[kInFlight], nxt[kInFlight];
  size_t i = beg + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kInFlight; ++u) {
    const size_t j = i + (size_t)u * kProbeThreads;
    cur[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
  }
  for (; i < end; i += step) {
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const size_t j = i + step + (size_t)u * kProbeThreads;
      nxt[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= cur[u].x ^ cur[u].y ^ cur[u].z ^ cur[u].w;
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) cur[u] = nxt[u];
  }
  if (acc == key) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t key, uint32_t* sink,
                              hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t want = (n16 + (size_t)kProbeThreads * kInFlight - 1) / ((size_t)kProbeThreads * kInFlight);
  const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>(want, kProbeGroups));
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kProbeThreads), 0, st,
                     reinterpret_cast<const u32x4*>(src), n16, key, sink);
  return hipGetLastError();
}

}  // namespace sv
