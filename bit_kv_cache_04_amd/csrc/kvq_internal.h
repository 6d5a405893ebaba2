// Internal declarations shared by the host translation units of libkvq.
#pragma once

#include <cstddef>
#include <cstdint>

#include "kvq.h"

namespace kvq {

constexpr int kFp4Group = 16;
constexpr int kKiviGroup = 32;
constexpr int kQjlM = 128;
constexpr int kLmBits = 2;

// Where the token rows of a cache live.  Paged storage: sequence b's position t
// is slot t % tokens of pool page table[b * per_seq + t / tokens].  A contiguous
// cache reads as one page of `capacity` tokens per sequence, page b (table NULL).
struct PageMap {
  const int32_t* table;  // device [B][per_seq], or nullptr
  int tokens;            // tokens per page (contiguous: capacity)
  int per_seq;           // table entries per sequence
  int num_pages;         // pages in the pool (contiguous: batch)
  int shift;             // paged: log2(tokens) (pages are a power of two)
};
// bf16(1/sqrt(d)): the magnitude of every entry of the structured rotation
float hadamard_magnitude(int d);

// TurboQuant's rotation as the kernels take it: the dense matrix (kind
// KV_ROT_DENSE) or a Hadamard transform, behind a bit-reversal of the channels
// for KV_ROT_HADAMARD_BITREV, scaled by mag.
struct RotArg {
  const float* rot;
  int kind;
  float mag;
};
inline RotArg rot_arg(const kv_cache* c) {
  const int kind = c->layout.rotation;
  return RotArg{c->rot, kind, kind == KV_ROT_DENSE ? 0.f : hadamard_magnitude(c->layout.head_dim)};
}

inline PageMap page_map(const kv_cache* c) {
  const kv_layout& L = c->layout;
  if (L.page_tokens > 0) {
    int shift = 0;
    while ((1 << shift) < L.page_tokens) ++shift;
    return PageMap{c->block_table, L.page_tokens, L.capacity / L.page_tokens, L.num_pages, shift};
  }
  return PageMap{nullptr, L.capacity, 1, L.batch, 0};
}

// KV_OK if the layout is one this library supports, else the status to return.
int check_layout(const kv_layout* L);
// KV_OK if every buffer and constant the format needs is non-NULL.
int check_cache(const kv_cache* c);

// Width of the query a caller passes (d, or d + rope for the latent format).
int query_width(const kv_layout* L);
// Width of the prepared fp32 query the attention kernel reads: the query itself,
// [R q, S R q] for TURBO, S q for QJL1.
int prepared_query_width(const kv_layout* L);
// Width of the attention output / value vector.
int value_width(const kv_layout* L);

// Context splits per (sequence, KV head) and the tokens each split covers.
struct SplitPlan {
  int splits;
  int tokens_per_split;
};
// The matrix-core decode kernel covers this cache / query combination (nq query
// tokens per sequence).
bool mfma_fast_path_ok(const kv_layout& L, int num_q_heads, int nq, int q_dtype);
// The TurboQuant matrix-core kernel covers this cache / query combination.
bool turbo_fast_path_ok(const kv_layout& L, int num_q_heads, int nq);
// The shared-latent matrix-core kernel covers this cache / query combination.
bool latent_fast_path_ok(const kv_layout& L, int num_q_heads, int nq, int q_dtype);
// The KIVI-2 matrix-core kernel covers this cache.
bool kivi_fast_path_ok(const kv_layout& L);
// Columns of the matrix-core kernel that takes n (query, head) pairs, n <= 32:
// n rounded up to 1, 2, 4, 8, 16 or 32 (two blocks of 16, FP4 keys only).
int mfma_columns(int n);
// Partial rows a decode call may write per (sequence, query): the merge keeps
// each split's (max, sum) in LDS arrays of this length.
constexpr int kMaxPartSplits = 1024;
// general: the plan of the general kernel (sparse decode), whatever the layout;
// max_splits: the most splits the plan may use (at most kMaxPartSplits)
SplitPlan plan_splits(const kv_layout* L, int num_q_heads, int nq, int q_dtype, int max_seq_len, int requested,
                      bool general = false, int max_splits = kMaxPartSplits);

// Workspace of a decode call: prepared queries, then per-split partial results
// (running max, running sum, unnormalised output) — offsets in bytes.
struct DecodeWorkspace {
  size_t qprep_off, qpiece_off, part_off, cnt_off, total;
};
// Pieces of the query operand of a bit-key product, FP6 for TurboQuant and FP8
// for QJL: per product, 4 pieces x (4 blocks x 32 code bytes (FP6: 24 used) +
// 4 scale bytes + 12 unused).
constexpr int kPieceProductBytes = 4 * 144;
constexpr int kTurboPieceBytes = 3 * kPieceProductBytes;  // code words 0..3, 4..7, sketch
// TURBO: the two constant terms (fp32) in the unused bytes of the first
// (product, piece) record: lv0 * scale * sum(R q), -kappa * scale * sum(S R q)
constexpr int kTurboPieceConstOff = 132;
constexpr int kQjlPieceBytes = kPieceProductBytes;        // sketch
DecodeWorkspace decode_workspace(const kv_layout* L, int num_q_heads, int splits);
// Size of the library's own decode workspace (kv_decode_attention_static).
constexpr size_t kStaticWorkspaceBytes = size_t(128) << 20;
// Mixed precision: splits of partial rows the bf16 window takes (one per 64 of
// its sink_tokens + recent_tokens positions), 0 without a window.
inline int window_chunks(const kv_layout& L) { return (L.sink_tokens + L.recent_tokens + 63) / 64; }
// KIVI-2: the keys of a sequence's incomplete last group wait uncoded in
// staging; a dense decode reads those tokens in one more split of partial rows.
inline int tail_chunks(const kv_layout& L) { return L.format == KV_FMT_KIVI2 ? 1 : 0; }

// Device launchers (defined in the HIP translation units).  Arguments are
// validated by the caller.
// Appends at `start` for every sequence, or at starts[b] (host array) when
// starts is given.
int launch_append(const kv_cache* c, const void* k, const void* v, int in_dtype, int start,
                  const int32_t* starts, int n_new, void* stream);
// sel: sparse decode over the positions sel[b][0 .. seq_lens[b]) (row stride
// sel_stride) on the general kernel; nullptr for the dense decode.
int launch_decode(const kv_cache* c, const void* q, int q_dtype, int num_q_heads, int nq,
                  const int32_t* seq_lens, int max_seq_len, float scale, float* out, void* ws,
                  const SplitPlan& plan, const DecodeWorkspace& wsl, void* ev_begin, void* ev_end,
                  void* stream, const int32_t* sel = nullptr, int sel_stride = 0, bool fp32 = false);
// Sparse decode of a contiguous latent cache runs on the latent matrix-core
// kernel, whose splits stage at most this many selected positions each.
constexpr int kLatentSparseSlots = 512;
inline bool latent_sparse_ok(const kv_layout& L, int num_q_heads, int q_dtype) {
  return latent_fast_path_ok(L, num_q_heads, 1, q_dtype) && L.page_tokens == 0;
}
// So does that of a contiguous FP4 or QJL cache on the FP4 / QJL matrix-core kernel.
constexpr int kMfmaSparseSlots = 512;
inline bool mfma_sparse_ok(const kv_layout& L, int num_q_heads, int q_dtype) {
  return mfma_fast_path_ok(L, num_q_heads, 1, q_dtype) && L.page_tokens == 0 && !L.sink_tokens && !L.recent_tokens;
}
// ... and that of a contiguous TurboQuant cache on its matrix-core kernel.
inline bool turbo_sparse_ok(const kv_layout& L, int num_q_heads) {
  return turbo_fast_path_ok(L, num_q_heads, 1) && L.page_tokens == 0;
}
// HSI selection (kvq_hsi.hip).
size_t hsi_candidates_workspace(int batch, int stride, int blk);
int launch_hsi_candidates(const float* scores, int batch, int stride, const int32_t* seq_lens, int blk,
                          int top_blocks, int32_t* pool, int32_t* pool_n, void* ws, void* stream);
int launch_hsi_select(const float* pool_scores, const int32_t* pool, const int32_t* pool_n, int batch, int pool_cap,
                      int top_k, int32_t* sel, int32_t* sel_n, void* stream);

}  // namespace kvq
