// The streaming-read reference kernel (declared in kvq_probe.h): how fast a
// kernel that only reads reaches HBM on this part, next to the decode kernels
// that read the packed cache once per token.
#include <hip/hip_runtime.h>

#include "kvq.h"
#include "kvq_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Each thread folds 16-byte words i, i + S, i + 2S, ... (S = all threads), kUnroll
// of them issued before the first is used.  The fold is written only if it equals
// a value no input makes likely, so the loads stay but the store almost never runs.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 w = src[i];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

extern "C" int kv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return KV_EINVAL;
  const size_t n16 = bytes / 16;
  // eight workgroups per compute unit of a 256-CU part, fewer for small buffers
  const size_t want = (n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  const unsigned blocks = (unsigned)(want < 2048 ? (want ? want : 1) : 2048);
  stream_read_kernel<<<blocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(src), n16,
                                                                               sink);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}
