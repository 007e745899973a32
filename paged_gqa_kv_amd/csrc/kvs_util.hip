// Utility kernels: status-word clearing and the streaming bandwidth probe.
//
// Sources: "KV-Cache Offloading for LLM Inference -- Visual Reference"
// Sec. 2 (attention), Sec. 11 (EMA), Sec. 12 (priority, cut points);
// "GQA Per-Head Scoring Streams" (head grouping, stream aggregation, the
// 64-byte record); "KV cache offload" post, "Top row" (block tables);
// "Fitting a Million Tokens", Sec. 02 (FP8 E4M3 and KIVI 2-bit KV).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvs.h"
#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

__global__ void __launch_bounds__(64) clear_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// stream probe.  Read: each wave takes 8 KiB chunks (chunk w, w + waves, ...),
// eight 1 KiB non-temporal loads per chunk and two chunks in flight, so the
// whole grid sweeps the buffer front to back the way a decode wave reads a
// tile.  Copy: grid-stride 16-byte loads and stores.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) stream_read(const u4_t* __restrict__ src, size_t n16,
                                                  uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t waves = (size_t)gridDim.x * 4;
  const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t nchunks = n16 / 512;
  uint32_t acc = 0;
  for (size_t ch = w; ch < nchunks; ch += 2 * waves) {
    // the second chunk past the end re-reads the first and is not counted
    const bool second = ch + waves < nchunks;
    const u4_t* p = src + ch * 512 + lane;
    const u4_t* p2 = src + (second ? ch + waves : ch) * 512 + lane;
    u4_t v[8], v2[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + 64 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) v2[u] = __builtin_nontemporal_load(p2 + 64 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    if (second) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v2[u][0] ^ v2[u][1] ^ v2[u][2] ^ v2[u][3];
    }
  }
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (size_t i = nchunks * 512 + tid; i < n16; i += waves * 64) {
    const u4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = acc;
}

__global__ void __launch_bounds__(256) stream_copy(const u4_t* __restrict__ src, size_t n16,
                                                  u4_t* __restrict__ dst) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_clear(uint32_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(clear_words, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_probe(const void* src, void* dst, size_t bytes, int mode, int grid,
                        hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (mode == 0)
    hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u4_t*>(src), n16, static_cast<uint32_t*>(dst));
  else
    hipLaunchKernelGGL(stream_copy, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u4_t*>(src), n16, static_cast<u4_t*>(dst));
  return hipGetLastError();
}

}  // namespace kvs
