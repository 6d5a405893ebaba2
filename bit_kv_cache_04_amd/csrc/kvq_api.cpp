// Exported entry points: argument validation on the host, then the launchers.
// Nothing here touches a GPU before every check has passed, so each error path
// can be exercised on a machine without one.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "kvq_internal.h"

using namespace kvq;

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" int kv_quant_append(const kv_cache* c, const void* k, const void* v, int32_t in_dtype,
                               int32_t start, int32_t n_new, void* ws, size_t* ws_bytes, void* stream) {
  (void)ws;
  int st = check_cache(c);
  if (st != KV_OK) return st;
  if (ws_bytes) *ws_bytes = 0;
  if (in_dtype != KV_DT_F32 && in_dtype != KV_DT_BF16) return KV_EUNSUPPORTED;
  if (start < 0 || n_new < 0) return KV_EINVAL;
  if ((int64_t)start + n_new > c->layout.capacity) return KV_ECAPACITY;
  if (n_new == 0) return KV_OK;
  const bool latent = c->layout.format == KV_FMT_LATENT_FP4;
  if (!k || (!latent && !v) || (latent && v)) return KV_EINVAL;
  if (!aligned(k, 16) || (v && !aligned(v, 16))) return KV_EINVAL;
  return launch_append(c, k, v, in_dtype, start, nullptr, n_new, stream);
}

extern "C" int kv_quant_append_ragged(const kv_cache* c, const void* k, const void* v, int32_t in_dtype,
                                      const int32_t* starts, int32_t n_new, void* ws, size_t* ws_bytes,
                                      void* stream) {
  (void)ws;
  int st = check_cache(c);
  if (st != KV_OK) return st;
  if (ws_bytes) *ws_bytes = 0;
  if (in_dtype != KV_DT_F32 && in_dtype != KV_DT_BF16) return KV_EUNSUPPORTED;
  if (!starts || n_new < 0) return KV_EINVAL;
  const kv_layout& L = c->layout;
  for (int b = 0; b < L.batch; ++b) {
    if (starts[b] < 0) return KV_EINVAL;
    if ((int64_t)starts[b] + n_new > L.capacity) return KV_ECAPACITY;
  }
  if (n_new == 0) return KV_OK;
  const bool latent = L.format == KV_FMT_LATENT_FP4;
  if (!k || (!latent && !v) || (latent && v)) return KV_EINVAL;
  if (!aligned(k, 16) || (v && !aligned(v, 16))) return KV_EINVAL;
  return launch_append(c, k, v, in_dtype, 0, starts, n_new, stream);
}

extern "C" int kv_decode_attention(const kv_cache* c, const void* q, int32_t q_dtype, int32_t num_q_heads,
                                   const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                                   float* out, void* ws, size_t* ws_bytes, const kv_decode_opts* opts,
                                   void* stream) {
  int st = check_cache(c);
  if (st != KV_OK) return st;
  const kv_layout& L = c->layout;
  if (num_q_heads < 1 || num_q_heads % L.num_kv_heads) return KV_EINVAL;
  if (num_q_heads / L.num_kv_heads > 1024) return KV_EUNSUPPORTED;
  if (max_seq_len < 1 || max_seq_len > L.capacity) return KV_EINVAL;
  if (q_dtype != KV_DT_F32 && q_dtype != KV_DT_BF16) return KV_EUNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return KV_EINVAL;
  const int req = opts ? opts->num_splits : 0;
  if (req < 0 || req > 1024) return KV_EINVAL;
  const int nq = opts && opts->num_queries > 0 ? opts->num_queries : 1;
  if ((opts && opts->num_queries < 0) || nq > max_seq_len) return KV_EINVAL;
  if (nq > 64) return KV_EUNSUPPORTED;
  const int flags = opts ? opts->flags : 0;
  if (flags & ~KV_DECODE_FP32) return KV_EINVAL;
  const bool fp32 = flags & KV_DECODE_FP32;
  // mixed precision: the splits cover the packed tokens from sink_tokens on, and
  // the bf16 window adds one split of partial rows
  const int packed_len = std::max(1, max_seq_len - (L.sink_tokens & ~31));  // matrix-core tiles start 32-aligned
  // the window's and the KIVI-2 staging tail's splits and the packed ones share
  // the merge's kMaxPartSplits
  const int extra = window_chunks(L) + tail_chunks(L);
  if (extra >= kMaxPartSplits) return KV_EUNSUPPORTED;
  const SplitPlan plan = plan_splits(&L, num_q_heads, nq, q_dtype, packed_len, req, fp32, kMaxPartSplits - extra);
  const int part_splits = plan.splits + extra;
  const DecodeWorkspace wsl = decode_workspace(&L, nq * num_q_heads, part_splits);
  if (!ws) {
    if (!ws_bytes) return KV_EINVAL;
    *ws_bytes = wsl.total;
    return KV_OK;
  }
  if (!ws_bytes || *ws_bytes < wsl.total) return KV_EWORKSPACE;
  if (!aligned(ws, 256)) return KV_EINVAL;
  if (!q || !seq_lens || !out) return KV_EINVAL;
  return launch_decode(c, q, q_dtype, num_q_heads, nq, seq_lens, max_seq_len, softmax_scale, out, ws, plan, wsl,
                       opts ? opts->ev_begin : nullptr, opts ? opts->ev_end : nullptr, stream, nullptr, 0, fp32);
}

extern "C" int kv_hsi_candidates(const float* scores, int32_t batch, int32_t score_stride, const int32_t* seq_lens,
                                 int32_t block, int32_t top_blocks, int32_t* pool, int32_t* pool_n, void* ws,
                                 size_t* ws_bytes, void* stream) {
  if (batch < 1 || batch > 65535 || score_stride < 1 || block < 1 || block > 64 || top_blocks < 1 ||
      (int64_t)top_blocks * block > INT32_MAX)
    return KV_EINVAL;
  const size_t need = hsi_candidates_workspace(batch, score_stride, block);
  if (!ws) {
    if (!ws_bytes) return KV_EINVAL;
    *ws_bytes = need;
    return KV_OK;
  }
  if (!ws_bytes || *ws_bytes < need) return KV_EWORKSPACE;
  if (!aligned(ws, 4) || !scores || !seq_lens || !pool || !pool_n) return KV_EINVAL;
  return launch_hsi_candidates(scores, batch, score_stride, seq_lens, block, top_blocks, pool, pool_n, ws, stream);
}

extern "C" int kv_hsi_select(const float* pool_scores, const int32_t* pool, const int32_t* pool_n, int32_t batch,
                             int32_t pool_cap, int32_t top_k, int32_t* sel, int32_t* sel_n, void* stream) {
  if (batch < 1 || batch > 65535 || pool_cap < 1 || top_k < 1) return KV_EINVAL;
  if (!pool_scores || !pool || !pool_n || !sel || !sel_n) return KV_EINVAL;
  return launch_hsi_select(pool_scores, pool, pool_n, batch, pool_cap, top_k, sel, sel_n, stream);
}

extern "C" int kv_decode_attention_sparse(const kv_cache* c, const void* q, int32_t q_dtype, int32_t num_q_heads,
                                          const int32_t* sel, const int32_t* sel_n, int32_t sel_cap,
                                          float softmax_scale, float* out, void* ws, size_t* ws_bytes,
                                          const kv_decode_opts* opts, void* stream) {
  int st = check_cache(c);
  if (st != KV_OK) return st;
  const kv_layout& L = c->layout;
  if (L.sink_tokens || L.recent_tokens) return KV_EUNSUPPORTED;
  if (num_q_heads < 1 || num_q_heads % L.num_kv_heads) return KV_EINVAL;
  if (num_q_heads / L.num_kv_heads > 1024) return KV_EUNSUPPORTED;
  if (sel_cap < 1) return KV_EINVAL;
  if (q_dtype != KV_DT_F32 && q_dtype != KV_DT_BF16) return KV_EUNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return KV_EINVAL;
  const int req = opts ? opts->num_splits : 0;
  if (req < 0 || req > 1024) return KV_EINVAL;
  if (opts && opts->num_queries > 1) return KV_EUNSUPPORTED;
  if (opts && opts->num_queries < 0) return KV_EINVAL;
  const int flags = opts ? opts->flags : 0;
  if (flags & ~KV_DECODE_FP32) return KV_EINVAL;
  const bool fp32 = flags & KV_DECODE_FP32;
  // the matrix-core kernels stage a split's positions: at most 512 per split, in
  // whole 128-token steps (FP4 / QJL) or 64-token steps (latent)
  const bool latent = !fp32 && latent_sparse_ok(L, num_q_heads, q_dtype);
  const bool mfma = !fp32 && !latent && (mfma_sparse_ok(L, num_q_heads, q_dtype) || turbo_sparse_ok(L, num_q_heads));
  SplitPlan plan = plan_splits(&L, num_q_heads, 1, q_dtype, sel_cap, req, !latent && !mfma);
  static_assert(kLatentSparseSlots == kMfmaSparseSlots, "one staging bound");
  if ((latent || mfma) && plan.tokens_per_split > kMfmaSparseSlots) {
    const int step = latent ? 64 : 128;
    const int splits = (sel_cap + kMfmaSparseSlots - 1) / kMfmaSparseSlots;
    const int per = ((sel_cap + splits - 1) / splits + step - 1) / step * step;
    plan = SplitPlan{(sel_cap + per - 1) / per, per};
    if (plan.splits > kMaxPartSplits) return KV_EUNSUPPORTED;  // more than 512 x 1024 selected slots
  }
  const DecodeWorkspace wsl = decode_workspace(&L, num_q_heads, plan.splits);
  if (!ws) {
    if (!ws_bytes) return KV_EINVAL;
    *ws_bytes = wsl.total;
    return KV_OK;
  }
  if (!ws_bytes || *ws_bytes < wsl.total) return KV_EWORKSPACE;
  if (!aligned(ws, 256)) return KV_EINVAL;
  if (!q || !sel || !sel_n || !out) return KV_EINVAL;
  return launch_decode(c, q, q_dtype, num_q_heads, 1, sel_n, sel_cap, softmax_scale, out, ws, plan, wsl,
                       opts ? opts->ev_begin : nullptr, opts ? opts->ev_end : nullptr, stream, sel, sel_cap, fp32);
}
