// Arguments and launchers of the specialised decode kernels (HIP translation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// FP4 cache, head_dim 128, bf16 queries, G = Hq / H in {1, 2, 4, 8, 16}.
struct Fp4DecodeArgs {
  const uint8_t* k_codes;
  const uint16_t* k_scale;
  const uint8_t* v_codes;
  const uint16_t* v_scale;
  const uint16_t* q;  // bf16 [B][Hq][128]
  const int32_t* seq_lens;
  int max_len, H, cap, Hq;
  float scale_log2;
  float* part;  // [B][Hq][splits][130]: running max (log2 units), sum, output
  int splits, per_split;
};

bool fp4_fast_path_ok(const kv_layout& L, int num_q_heads, int q_dtype);
int launch_decode_fp4_fast(const Fp4DecodeArgs& a, int B, int G, hipStream_t st);

}  // namespace kvq
