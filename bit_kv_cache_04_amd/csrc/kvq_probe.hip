// Reference kernels (declared in kvq_probe.h): how fast a kernel that only
// reads reaches HBM on this part, next to the decode kernels that read the
// packed cache once per token; and how fast the matrix cores and the LDS run
// when nothing else competes, next to the latent decode that needs both.
#include <hip/hip_runtime.h>

#include "kvq.h"
#include "kvq_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread
constexpr int kStep = kThreads * kUnroll;

// Workgroup b reads its own contiguous run of 16-byte words [b * chunk,
// min(n16, (b + 1) * chunk)), kStep words (32 KiB) per step, every thread's
// kUnroll loads issued before the first is used (long contiguous runs per
// workgroup keep DRAM pages open: grid-strided reads measured 18% slower).  The
// fold is written only if it equals a value no input makes likely, so the loads
// stay but the store almost never runs.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                               size_t chunk, uint32_t* __restrict__ sink) {
  const size_t begin = (size_t)blockIdx.x * chunk;
  const size_t end = begin + chunk < n16 ? begin + chunk : n16;
  uint32_t acc = 0;
  size_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < end; i += kStep) {
    uint4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = src[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < end; i += kThreads) {
    const uint4 w = src[i];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));

// Two independent chains of 32x32x16 fp16 products per wave, 8 products per
// iteration; the operands depend on the thread so nothing folds away.
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* __restrict__ sink) {
  h8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0x1p-10f * (float)((threadIdx.x + i) & 15));
    b[i] = (_Float16)(0x1p-10f * (float)((blockIdx.x + i) & 7));
  }
  f16v_t c0{}, c1{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
  if (s == 1234.5f) *sink = s;  // almost never: the products stay, the store does not
}

// Each wave reads 1 KiB per instruction: lane l its 16 bytes at 16 l plus a
// per-iteration offset, so the 64 lanes cover 1 KiB of consecutive banks.
__global__ void __launch_bounds__(256) lds_probe_kernel(int iters, uint32_t* __restrict__ sink) {
  __shared__ uint4 buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    uint4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = buf[(((it * 8 + u) * 64 + wave * 1024) & 4095) + lane];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

extern "C" int kv_mfma_probe(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20) || !sink) return KV_EINVAL;
  mfma_probe_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}

extern "C" int kv_lds_probe(int32_t blocks, int32_t iters, uint32_t* sink, void* stream) {
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20) || !sink) return KV_EINVAL;
  lds_probe_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}

extern "C" int kv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return KV_EINVAL;
  const size_t n16 = bytes / 16;
  // up to eight workgroups per compute unit of a 256-CU part, each a whole
  // number of steps long
  const size_t steps = (n16 + kStep - 1) / kStep;
  const size_t blocks = steps < 2048 ? steps : 2048;
  const size_t chunk = (steps + blocks - 1) / blocks * kStep;
  stream_read_kernel<<<(unsigned)blocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), n16, chunk, sink);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}
