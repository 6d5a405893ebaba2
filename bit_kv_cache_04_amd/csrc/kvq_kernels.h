// Arguments and launchers of the specialised decode kernels (HIP translation units).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {

// Matrix-core decode: head_dim 128, FP4 values, G = Hq / H in {1, 2, 4, 8, 16};
// keys FP4 (bf16 queries) or 1-bit QJL with m = 128 (projected fp32 queries).
struct MfmaDecodeArgs {
  const uint8_t* k_codes;   // FP4 keys: [B][H][cap][64]
  const uint16_t* k_scale;  //           [B][H][cap][8] bf16
  const uint8_t* k_sketch;  // QJL keys: [B][H][cap][16]
  const uint16_t* k_norm;   //           [B][H][cap] fp16
  const uint8_t* v_codes;   // [B][H][cap][64]
  const uint16_t* v_scale;  // [B][H][cap][8] bf16
  const uint16_t* rope;     // latent: [B][cap][64] bf16 (k_codes [B][cap][256], k_scale [B][cap][32])
  // KIVI-2 (k_codes, v_codes [B][H][cap][d / 4]): key scale / zero f32 [B][H][cap / 32][d],
  // value scale / zero f32 [B][H][cap][d / 32], key staging [B][H][4 + 32 d] (count, then keys)
  const float *k_scale_f, *k_zero_f, *v_scale_f, *v_zero_f, *k_stage;
  PageMap pm;               // token rows: [B][H][cap] above, or a paged pool
  // latent sparse decode: slot i of sequence b reads position sel[b * sel_stride + i]
  // (seq_lens counts slots, at most kLatentSparseSlots per split); nullptr: dense
  const int32_t* sel;
  int sel_stride;
  const void* q;            // FP4: bf16 [B][Hq][128]; QJL: fp32 S q [B][Hq][128]
  const uint8_t* qpieces;   // QJL: [B][Hq][kQjlPieceBytes], FP8 pieces of S q
  const int32_t* seq_lens;
  int max_len, H, cap, Hq;
  float scale_log2;  // softmax scale * log2(e)
  float kappa;       // QJL: sqrt(pi/2) / m
  float* part;       // [B][nq][Hq][splits][130]: running max (log2 units), sum, output
  int splits, per_split;
  // nq query tokens per sequence of gr query heads per KV head, numbered
  // c = j * gr + g (query j, head g; q [B][nq][Hq][.]); one launch takes the
  // ncol of them from c0 as its columns.  The latent kernel takes one query per
  // launch: query c0 of nq (its heads are the columns).
  int nq, gr, c0, ncol;
  // packed tokens [t_lo, L - recent) of a sequence of length L (split s from
  // t_lo + s * per_split); partial rows hold part_splits splits
  int t_lo, recent, part_splits;
};

int launch_decode_mfma(const MfmaDecodeArgs& a, int format, int B, int G, hipStream_t st);

// KIVI-2 on the matrix cores (d = 64 or 128, contiguous, dense; columns c0 ..
// c0 + ncol of the (query, head) pairs, ncol <= 16, q the prepared fp32
// queries): the coded tokens of each split, up to the sequence's incomplete
// group, and with `tail` (a last grid column) that group's staged tokens as
// partial split `splits`.
int launch_decode_kivi(const MfmaDecodeArgs& a, int d, bool tail, int B, hipStream_t st);

// TurboQuant cache (d = 128, m = 128, 2-bit symmetric codebook): per query
// row the FP6 pieces of the scaled key-product operands and the two constant
// terms (kTurboPieceBytes, written by the query preparation).
struct TurboDecodeArgs {
  const uint8_t* k_codes;   // [B][H][cap][32]
  const uint8_t* k_sketch;  // [B][H][cap][16]
  const uint16_t* k_norm;   // [B][H][cap] fp16
  const uint16_t* k_rnorm;  // [B][H][cap] fp16
  const uint8_t* v_codes;   // [B][H][cap][32]
  const uint16_t* v_norm;   // [B][H][cap] fp16
  PageMap pm;               // token rows: [B][H][cap] above, or a paged pool
  const float* levels;      // 4 codebook levels, ascending, symmetric
  const uint8_t* qpieces;   // [B][nq][Hq][kTurboPieceBytes]
  const int32_t* seq_lens;
  int max_len, H, cap, Hq;
  float* part;  // [B][nq][Hq][part_splits][130]
  int splits, per_split;
  // nq query tokens per sequence of gr query heads per KV head, numbered
  // c = j * gr + g (query j, head g); one launch takes the ncol <= 16 of them
  // from c0 as its columns
  int nq, gr, c0, ncol;
  // mixed precision: packed tokens [t_lo, L - recent); split s from
  // (t_lo & ~31) + s * per_split (tiles start 32-aligned, tokens below t_lo masked)
  int t_lo, recent, part_splits;
  // sparse decode: slot i of sequence b reads position sel[b * sel_stride + i]
  // (seq_lens counts slots, at most kMfmaSparseSlots per split); nullptr: dense
  const int32_t* sel;
  int sel_stride;
};

int launch_decode_turbo(const TurboDecodeArgs& a, int B, hipStream_t st);

// Shared-latent cache (512 FP4 + 64 bf16 RoPE), bf16 queries, Hq in {32, 64, 128}.
bool latent_fast_path_ok(const kv_layout& L, int num_q_heads, int nq, int q_dtype);
int launch_decode_latent(const MfmaDecodeArgs& a, int B, hipStream_t st);

}  // namespace kvq
