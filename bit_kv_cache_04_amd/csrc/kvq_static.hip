// kv_decode_attention_static: decode attention whose workspace is the
// library's own device array, for callers that cannot allocate device memory.
//
// The array `scratch` below is a file-scope __device__ object: every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is
// only a stand-in for the symbol); it asks the runtime for the device address
// once per device and uses that address for everything.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr size_t kStaticScratchBytes = kStaticWorkspaceBytes;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current), or nullptr when the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int kv_decode_attention_static(const kv_cache* c, const void* q, int32_t q_dtype, int32_t num_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                          float* out, const kv_decode_opts* opts, void* stream) {
  // the workspace this call needs (a size query: no launch, no allocation)
  size_t need = 0;
  int st = kv_decode_attention(c, q, q_dtype, num_q_heads, seq_lens, max_seq_len, softmax_scale, out, nullptr,
                               &need, opts, stream);
  if (st != KV_OK) return st;
  if (need > kStaticScratchBytes) return KV_EWORKSPACE;
  if (!q || !seq_lens || !out) return KV_EINVAL;
  void* ws = scratch_on_current_device();
  if (!ws) return KV_EDEVICE;
  size_t have = kStaticScratchBytes;
  return kv_decode_attention(c, q, q_dtype, num_q_heads, seq_lens, max_seq_len, softmax_scale, out, ws, &have, opts,
                             stream);
}
