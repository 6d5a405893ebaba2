/*
 * kvq.h - low-bit KV-cache append and decode attention (C ABI).
 *
 * The problem, as the pages state it (page "TurboQuant vs OSCAR vs EpiCache:
 * the battle over KV-cache compression", section on the KV-cache memory
 * bottleneck): a decoder stores one key and one value vector per token, per
 * layer, per KV head; every newly generated token then reads the whole cache
 * from HBM, so decoding is bound by memory bandwidth, and the bytes stored per
 * token are layers x KV heads x head dim x 2 tensors x bytes per element.
 * This library stores K/V in packed low-bit formats and runs decode attention
 * directly on the packed bytes:
 *
 *   kv_quant_append      write new tokens' K/V into a packed cache (one layer);
 *                        kv_quant_append_ragged: at a position per sequence
 *   kv_decode_attention  each sequence's query token (or last few tokens)
 *                        attends over its cache
 *   kv_bytes_per_token   stored bytes per token for a layout and layer count
 *   kv_hsi_candidates,   hierarchical sparse indexing: a candidate pool of
 *   kv_hsi_select        positions, then the final selection from it
 *   kv_decode_attention_sparse  decode over selected positions only
 * plus host helpers for buffer sizes and the methods' constants.  Caches are
 * contiguous or paged (a pool of pages and a block table per sequence).
 *
 * Formats (each cited where it is defined):
 *   KV_FMT_KIVI2      2-bit asymmetric; keys per channel over 32-token groups,
 *                     values per token over 32-channel groups, fp32 scale and
 *                     zero (page "TurboQuant vs OSCAR vs EpiCache", section
 *                     "quantization frontiers", KIVI paragraph).
 *   KV_FMT_FP4        E2M1 nibbles with one bf16 scale per 16 channels, for K
 *                     and V (page "How DeepSeek-V4.1-Flash cut KV-cache storage
 *                     by 4x via CSA2", section on numerical precision).
 *   KV_FMT_TURBO      keys: seeded Haar rotation, 2-bit Gaussian Lloyd-Max
 *                     codes of the rotated unit vector, 1-bit QJL sign sketch
 *                     of the residual, fp16 norm and fp16 residual norm; values:
 *                     rotation + 2-bit Lloyd-Max + fp16 norm (page "TurboQuant
 *                     vs OSCAR vs EpiCache", section "quantization frontiers",
 *                     stages one and two).
 *   KV_FMT_QJL1_FP4V  keys: 1-bit QJL sign sketch + fp16 norm; values: FP4.
 *   KV_FMT_LATENT_FP4 one 512-wide latent per token shared by all query heads,
 *                     stored FP4, plus a 64-wide RoPE key kept bf16 (page "How
 *                     DeepSeek-V4.1-Flash cut KV-cache storage by 4x via
 *                     CSA2", CSA2 section: a 512-d latent shared across heads
 *                     with a 64-d RoPE part).
 *   KV_FMT_BF16       uncompressed reference for kv_bytes_per_token only.
 *
 * Packed layout: arrays are C-contiguous and token-major; sequence b, KV head
 * h, token t index ((b*H + h)*capacity + t).  Bit order is least significant
 * first: FP4 channel 2j in the low nibble of byte j; 2-bit channel 4j+i in
 * bits [2i+1:2i] of byte j; sketch row 8j+i in bit i of byte j.  bf16/fp16
 * values are stored as their 16-bit patterns.
 *
 * Ownership and errors: every pointer passed is owned by the caller; device
 * pointers must stay valid until the stream work completes.  The library never
 * allocates device memory and keeps no global state.  Every error is a
 * negative status returned before any work is enqueued, except KV_EDEVICE,
 * which reports a failed launch; faults inside a kernel surface at the caller's
 * next synchronisation.  Calls are asynchronous on `stream` (a hipStream_t; NULL
 * is the default stream).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kv_format {
  KV_FMT_BF16 = 0,
  KV_FMT_KIVI2 = 1,
  KV_FMT_FP4 = 2,
  KV_FMT_TURBO = 3,
  KV_FMT_QJL1_FP4V = 4,
  KV_FMT_LATENT_FP4 = 5
};

enum kv_dtype { KV_DT_F32 = 0, KV_DT_BF16 = 1 };

enum kv_status {
  KV_OK = 0,
  KV_EINVAL = -1,        /* malformed argument: NULL pointer, bad size, misaligned KIVI append */
  KV_ECAPACITY = -2,     /* tokens beyond the cache capacity */
  KV_EUNSUPPORTED = -3,  /* a valid request this library does not implement */
  KV_EWORKSPACE = -4,    /* workspace missing or smaller than required */
  KV_EDEVICE = -5        /* a kernel launch failed */
};

/* Shape of one layer's cache.  Supported: KIVI2 head_dim 64|128, group 32,
 * capacity a multiple of 32; FP4 head_dim 64|128, group 16; TURBO head_dim 128,
 * qjl_m 128, lm_bits 2; QJL1_FP4V head_dim 128, qjl_m 128, group 16;
 * LATENT_FP4 num_kv_heads 1, head_dim 512, rope_dim 64, group 16.  Fields a
 * format does not use must be 0, except `group`, which is always the format's
 * quantisation group (0 for TURBO).
 *
 * Mixed precision (every format but LATENT_FP4, both <= capacity): the first
 * sink_tokens tokens of every sequence and its last recent_tokens tokens are
 * also kept in bf16 and decode reads them from there, the rest through the
 * packed codes (page "TurboQuant vs OSCAR vs EpiCache", section "quantization
 * frontiers: TurboQuant and OSCAR": sink and recent tokens stay BF16 while the
 * history is compressed).  A window token's logit is <q, bf16 key> and its
 * value the bf16 value, in the original basis (TURBO: the history's output is
 * mapped back through R^T, the window's is not).  KIVI2 keys of a sequence's
 * incomplete group that fall outside the window keep their exact staged fp32
 * values.  The recent window is a ring of the last recent_tokens tokens
 * appended to a sequence (slot t mod recent_tokens), so decode must see each
 * sequence at the length it was appended to.  0 and 0 turn it off.
 *
 * Paged storage (page_tokens > 0, any format): the per-token buffers hold a
 * pool of num_pages pages instead of B x capacity slots; page p holds
 * page_tokens consecutive positions of one sequence for all H heads, token
 * slot s of head h at row ((p*H + h)*page_tokens + s) (KIVI2 key scale / zero:
 * row ((p*H + h)*(page_tokens/32) + s/32)).  kv_cache.block_table maps each
 * sequence's logical page j (positions [j*page_tokens, (j+1)*page_tokens)) to
 * a pool page, so sequences grow a page at a time and whole pages return to
 * the pool (page "TurboQuant vs OSCAR vs EpiCache", OSCAR's deployment list:
 * kernels that work with paged attention; page "How TriAttention cut LLM
 * memory use 10x", paged memory fragmentation: paged allocators reclaim whole
 * blocks).  page_tokens is a power of two, at least 32, that divides
 * capacity; num_pages >= 1.  Windows and K_STAGE stay per sequence.  page_tokens 0 (and num_pages
 * 0) is the contiguous layout. */
typedef struct kv_layout {
  int32_t format;       /* enum kv_format */
  int32_t batch;        /* sequences B */
  int32_t num_kv_heads; /* H */
  int32_t head_dim;     /* d (latent width for LATENT_FP4) */
  int32_t rope_dim;     /* LATENT_FP4: bf16 RoPE key width; else 0 */
  int32_t capacity;     /* token slots per sequence */
  int32_t group;        /* FP4 scale group (16) or KIVI group (32) */
  int32_t qjl_m;        /* QJL sketch rows (TURBO, QJL1_FP4V) */
  int32_t lm_bits;      /* Lloyd-Max bits (TURBO) */
  int32_t sink_tokens;   /* leading tokens kept bf16 (mixed precision), else 0 */
  int32_t recent_tokens; /* trailing tokens kept bf16 (mixed precision), else 0 */
  int32_t page_tokens;   /* paged storage: tokens per page, else 0 */
  int32_t num_pages;     /* paged storage: pages in the pool, else 0 */
  int32_t rotation;      /* TURBO: enum kv_rotation; every other format 0 */
} kv_layout;

/* How TURBO applies its rotation R (layout.rotation).  KV_ROT_DENSE reads R from
 * kv_cache.rot as a d x d matrix.  The two structured kinds are the rotation
 * kv_make_hadamard_rotation writes (bit_reverse 1 or 0): R = H P / sqrt(d), a
 * Hadamard transform behind a bit-reversal permutation of the channels (page
 * "TurboQuant vs OSCAR vs EpiCache", section "quantization frontiers", the
 * OSCAR paragraph).  With them the append, the query preparation and the merge
 * apply R (and R^T) as a butterfly in O(d log d) instead of a d x d product,
 * every entry being +-bf16(1/sqrt(d)); the results are those of the dense
 * product with that matrix (bit for bit in the append wherever its fp64 sums
 * are exact, as they are for bf16 inputs), and kv_cache.rot is not read (it may
 * be NULL).  Any other value, or a nonzero one for another format, is
 * KV_EINVAL. */
enum kv_rotation { KV_ROT_DENSE = 0, KV_ROT_HADAMARD_BITREV = 1, KV_ROT_HADAMARD = 2 };

/* Buffers of a cache, by role.  Element types and shapes (Tc = capacity; with
 * paged storage every [B][H][Tc] reads [num_pages][H][page_tokens], [B][Tc]
 * reads [num_pages][page_tokens] and KIVI2's [B][H][Tc/32] reads
 * [num_pages][H][page_tokens/32]):
 *   K_CODES  u8   KIVI2 [B][H][Tc][d/4]; FP4 [B][H][Tc][d/2]; TURBO [B][H][Tc][d/4];
 *                 LATENT [B][Tc][d/2]
 *   K_SCALE  KIVI2 f32 [B][H][Tc/32][d]; FP4 bf16 [B][H][Tc][d/16]; LATENT bf16 [B][Tc][d/16]
 *   K_ZERO   f32  KIVI2 [B][H][Tc/32][d]
 *   K_SKETCH u8   TURBO, QJL1 [B][H][Tc][m/8]
 *   K_NORM   f16  TURBO, QJL1 [B][H][Tc]
 *   K_RNORM  f16  TURBO [B][H][Tc]  (residual norm)
 *   V_CODES  u8   KIVI2 [B][H][Tc][d/4]; FP4, QJL1 [B][H][Tc][d/2]; TURBO [B][H][Tc][d/4]
 *   V_SCALE  KIVI2 f32 [B][H][Tc][d/32]; FP4, QJL1 bf16 [B][H][Tc][d/16]
 *   V_ZERO   f32  KIVI2 [B][H][Tc][d/32]
 *   V_NORM   f16  TURBO [B][H][Tc]
 *   ROPE     bf16 LATENT [B][Tc][rope_dim]
 *   SINK_K, SINK_V      bf16 [B][H][sink_tokens][d]    (mixed precision)
 *   RECENT_K, RECENT_V  bf16 [B][H][recent_tokens][d]  (mixed precision; token
 *                       t in slot t mod recent_tokens)
 *   K_STAGE  KIVI2 [B][H][4 + 32 d] 32-bit words: word 0 the number of tokens
 *                 appended to the sequence (int32), words 1..3 unused, then as
 *                 f32 [32][d] the keys of its last, incomplete 32-token group
 *                 (token t in row t mod 32), which have no key code yet
 * Decode reads whole 32-token tiles and may read a few tiles past a
 * sequence's end, giving those slots zero weight: every slot within capacity
 * (every page of a pool) must hold finite data, as zeroed buffers and appends
 * of finite inputs do.                                                         */
enum kv_buffer {
  KV_BUF_K_CODES = 0, KV_BUF_K_SCALE, KV_BUF_K_ZERO, KV_BUF_K_SKETCH, KV_BUF_K_NORM,
  KV_BUF_K_RNORM, KV_BUF_V_CODES, KV_BUF_V_SCALE, KV_BUF_V_ZERO, KV_BUF_V_NORM,
  KV_BUF_ROPE, KV_BUF_SINK_K, KV_BUF_SINK_V, KV_BUF_RECENT_K, KV_BUF_RECENT_V, KV_BUF_K_STAGE, KV_BUF_COUNT
};

/* A cache: its layout, device buffers (NULL where the format has none) and
 * the method's constants, as device arrays of fp32 (made by the helpers below):
 *   rot        TURBO with layout.rotation KV_ROT_DENSE: d x d rotation R,
 *              row-major, y = R x, bf16-valued, 16-byte aligned (not read,
 *              and may be NULL, with a structured rotation)
 *   proj       TURBO, QJL1: m x d QJL matrix S, row-major, bf16-valued,
 *              16-byte aligned
 *   lm_levels  TURBO: 2^lm_bits Lloyd-Max levels, ascending and symmetric
 *              (levels[i] = -levels[last - i], as kv_lloyd_max_gaussian makes
 *              them: the matrix-core decode relies on it and, given levels
 *              with lv0 + lv3 != lv1 + lv2, returns NaN outputs; the general
 *              kernel, opts->flags KV_DECODE_FP32, reads any levels)
 *   lm_thresh  TURBO: 2^lm_bits - 1 thresholds, ascending
 * A missing or misaligned constant is KV_EINVAL.                           */
typedef struct kv_cache {
  kv_layout layout;
  void* buf[KV_BUF_COUNT];
  const float* rot;
  const float* proj;
  const float* lm_levels;
  const float* lm_thresh;
  /* paged storage: device int32 [B][capacity / page_tokens], row-major, the
   * pool page of each sequence's logical page (caller-owned; read by the
   * kernels when they run).  Entries a call touches must lie in [0, num_pages)
   * and no two sequences may append into one page at once.  An entry outside
   * the pool is never followed: appends to it are dropped and decode reads it
   * as zero bytes (that sequence's output is then unspecified).  NULL for the
   * contiguous layout; NULL with page_tokens > 0 is KV_EINVAL. */
  const int32_t* block_table;
} kv_cache;

/* Options for kv_decode_attention; pass NULL for defaults.
 *   num_splits   context splits per (sequence, KV head), 0..1024; 0 picks one
 *                from the shape; the workspace size depends on it.  With bf16
 *                windows the window takes (sink_tokens + recent_tokens) / 64
 *                (rounded up) more splits and the packed splits are capped at
 *                1024 minus those; a window of more than 65,472 tokens is
 *                KV_EUNSUPPORTED
 *   ev_begin/end optional hipEvent_t recorded on `stream` immediately before
 *                and after the split-context attention kernel (for timing)
 *   num_queries  query tokens per sequence, 1..64 (0 means 1): several drafted
 *                positions checked in one pass (page "How DeepSeek-V4.1-Flash
 *                cut KV-cache storage by 4x via CSA2", section "numerical
 *                precision & hardware efficiency": a draft model proposes
 *                several positions at once).  The queries are the last
 *                num_queries tokens of each sequence, already appended; query j
 *                sees the first seq_lens[b] - (num_queries - 1 - j) tokens.
 *                The workspace size depends on it.
 *   flags        0, or KV_DECODE_FP32: dequantise and compute on the fp32
 *                vector kernel for every format (slower).
 * Range of the default path: FP4 keys and values and the LATENT latent feed the
 * matrix cores as fp16, where E2M1 x bf16 scale is exact when every group scale
 * s = bf16(absmax / 6) is 0 or lies in [2^-16, 65504 / 6] (absmax from about
 * 5.5e-4 to 65504), and a bf16 query is exact in fp16 when each |q| is 0 or
 * lies in [2^-17, 65504].  Outside those ranges values round like fp16 (a
 * group absmax or query above 65504 becomes infinite); a cache or query that
 * may leave them is decoded exactly with KV_DECODE_FP32.  fp32 queries always
 * take the fp32 kernel for FP4 and LATENT caches.  KIVI-2 caches with 64 or
 * 128 channels (contiguous, no windows) read their coded key groups on the
 * matrix cores: a key term q_c * s_c enters as an fp16 pair hi + lo (error
 * below 2^-20 relative or 2^-24 absolute), the zero term sum_c q_c z_c in fp32,
 * and a value as code * s + z rounded once to fp16; |q_c * s_c| and every
 * dequantised value must stay below 65504 there.  The keys of a sequence's
 * incomplete last group (still in staging) are read by the fp32 kernel. */
enum kv_decode_flags { KV_DECODE_FP32 = 1 };
typedef struct kv_decode_opts {
  int32_t num_splits;
  void* ev_begin;
  void* ev_end;
  int32_t num_queries;
  int32_t flags;
} kv_decode_opts;

/* Bytes of one buffer of a cache with this layout; 0 if the format has no
 * such buffer or the layout is invalid.  Host only. */
size_t kv_buffer_bytes(const kv_layout* L, int32_t which);

/* Bytes stored per token over `num_layers` layers: packed codes plus the
 * metadata kept for that token (KIVI key scale/zero, kept per 32 tokens, counted
 * as 1/32 per token) for all KV heads (page "TurboQuant vs OSCAR vs EpiCache",
 * KV-cache memory bottleneck section: layers x KV heads x head dim x 2 x bytes
 * per element for BF16).  Host only; returns 0 for an invalid layout or
 * num_layers < 1.  BF16 needs only format, num_kv_heads and head_dim.  The
 * bf16 sink and recent windows of mixed precision are a fixed cost per
 * sequence, not per token, and are not counted. */
size_t kv_bytes_per_token(const kv_layout* L, int32_t num_layers);

/* Append n_new tokens at positions [start, start+n_new) of every sequence.
 *   k, v      device, [B][H][n_new][d] in `in_dtype` (KV_DT_F32 or KV_DT_BF16);
 *             LATENT_FP4: k is [B][n_new][d + rope_dim] (latent then RoPE key)
 *             and v must be NULL
 *   ws        unused by every current format: pass NULL; *ws_bytes (if given)
 *             is set to 0
 * KIVI2 quantises keys per channel over whole 32-token groups: the keys of a
 * sequence's last incomplete group wait in K_STAGE (as fp32 of the input) and
 * are coded when a later append completes the group, from the staged keys and
 * the new ones; values are coded per token at once.  So KIVI2 appends to a
 * sequence must follow each other (each starting where the previous ended)
 * whenever a group is left incomplete; decode reads a sequence's staged keys
 * for its tokens from 32 * floor(A / 32) on, A the tokens appended to it (a
 * decode over a shorter prefix reads coded groups) (page "TurboQuant vs OSCAR vs
 * EpiCache", section "quantization frontiers", KIVI paragraph: keys quantised
 * per channel, values per token).  start + n_new > capacity: KV_ECAPACITY.  n_new == 0
 * enqueues nothing.  The method's encoding steps are those of the format
 * definitions above (TurboQuant: norm, rotate, divide, Lloyd-Max code,
 * residual, residual norm, sketch of the residual, in that order).  With mixed
 * precision every token is still packed; tokens below sink_tokens and the last
 * recent_tokens of the append are also stored as bf16 (round to nearest even). */
int kv_quant_append(const kv_cache* c, const void* k, const void* v, int32_t in_dtype,
                    int32_t start, int32_t n_new, void* ws, size_t* ws_bytes, void* stream);

/* As kv_quant_append, but sequence b appends its n_new tokens at positions
 * [starts[b], starts[b] + n_new): sequences at different lengths, as a batch of
 * token-by-token decodes leaves them.
 *   starts    host int32 [B], read during the call (the positions travel to the
 *             kernels by value: nothing is allocated, and a captured graph
 *             replays the positions it was captured with)
 * starts NULL or a negative start: KV_EINVAL; starts[b] + n_new > capacity:
 * KV_ECAPACITY.  Other errors and behaviour as kv_quant_append. */
int kv_quant_append_ragged(const kv_cache* c, const void* k, const void* v, int32_t in_dtype,
                           const int32_t* starts, int32_t n_new, void* ws, size_t* ws_bytes, void* stream);

/* One query token per sequence attends over the first seq_lens[b] cached
 * tokens of its sequence (no mask; a query head hq reads KV head hq / (Hq/H)):
 *   out[b][hq] = sum_t softmax_t(scale * logit(q[b][hq], t)) * value(t)
 * (with opts->num_queries = nq > 1: q[b][j][hq] over the first
 * seq_lens[b] - (nq - 1 - j) tokens into out[b][j][hq]; q and out carry the
 * extra [nq] dimension after [B], and each seq_lens[b] must be at least nq: a
 * query that sees no token gets zeros)
 * (page "TurboQuant vs OSCAR vs EpiCache", section on the KV-cache memory
 * bottleneck: each new token reads the whole cache).  Logits per format: the
 * dot product with the dequantised key (KIVI2, FP4; LATENT: latent part plus
 * RoPE part); TURBO: n*(<Rq, u~> + sqrt(pi/2)/m * gamma * <S R q, sigma>);
 * QJL1: sqrt(pi/2)/m * n * <S q, sigma>; sigma = +-1 from the sketch bits.
 *   q         device, [B][Hq][d] (LATENT: [B][Hq][d + rope_dim]) in q_dtype
 *   seq_lens  device int32 [B], each in [1, max_seq_len]; values beyond
 *             max_seq_len are clamped to it
 *   out       device fp32 [B][Hq][d] (LATENT: [B][Hq][d]); for TURBO the value
 *             path is mapped back with R^T
 *   ws        device workspace of *ws_bytes bytes, 256-byte aligned, filled with
 *             zeros before its first use (every call leaves it zeroed again);
 *             ws == NULL is a size query that writes *ws_bytes and returns KV_OK.
 *             Calls that overlap on one workspace race.
 * Errors: num_q_heads not a multiple of H, max_seq_len outside
 * [1, capacity], NULL pointers: KV_EINVAL; workspace smaller than required:
 * KV_EWORKSPACE. */
int kv_decode_attention(const kv_cache* c, const void* q, int32_t q_dtype, int32_t num_q_heads,
                        const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                        float* out, void* ws, size_t* ws_bytes, const kv_decode_opts* opts,
                        void* stream);

/* kv_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is the library's own
 * device array of 128 MiB, one per GPU, held until the process ends; it is
 * looked up (never allocated) on the first call on each device, and this call
 * allocates and frees nothing.  Every call on a GPU uses that GPU's array, so
 * calls that overlap on one GPU (on different streams, or from several host
 * threads) race; calls in stream order do not.  Nothing in it has to start at
 * zero: each call writes every partial result it reads.
 * Arguments, behaviour and errors as kv_decode_attention, on the current
 * device, plus: a call whose workspace (the size kv_decode_attention reports
 * for it) exceeds 128 MiB is KV_EWORKSPACE, and a failed lookup of the array is
 * KV_EDEVICE. */
int kv_decode_attention_static(const kv_cache* c, const void* q, int32_t q_dtype, int32_t num_q_heads,
                               const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                               float* out, const kv_decode_opts* opts, void* stream);

/* ---- the method's constants (host memory, host only) ---- */

/* Lloyd-Max quantiser for N(0, 1/dim) with 2^bits levels: the fixed point of
 * "thresholds are midpoints of neighbouring levels" and "each level is the
 * mean of the source over its cell", iterated in fp64 and rounded to fp32
 * (page "TurboQuant vs OSCAR vs EpiCache", section "quantization frontiers",
 * stage one: a precomputed optimal scalar quantiser per coordinate).
 * levels: 2^bits floats, thresholds: 2^bits - 1 floats, ascending.
 * bits in [1, 4], dim >= 1; else KV_EINVAL. */
int kv_lloyd_max_gaussian(int32_t bits, int32_t dim, float* levels, float* thresholds);

/* Haar rotation from a d x d matrix of iid N(0,1) draws (row-major fp64): the
 * orthogonal factor Q of gauss = Q R with diag(R) > 0, rounded to bf16 values,
 * written as fp32 row-major (same section, stage one: a random rotation).
 * d in [1, 1024]; a rank-deficient input gives KV_EINVAL. */
int kv_make_rotation(const double* gauss, int32_t d, float* rot);

/* Structured rotation in place of the random one: R = H P / sqrt(d), H the
 * Sylvester Hadamard matrix (H[i][k] = (-1)^popcount(i & k)) and P the
 * bit-reversal permutation of the d input channels (applied first; identity
 * when bit_reverse is 0), so that a few loud channels are spread evenly over
 * every coordinate (page "TurboQuant vs OSCAR vs EpiCache", section
 * "quantization frontiers", the OSCAR paragraph: a Hadamard transform with a
 * bit-reversal permutation).  Written as fp32 row-major, y = R x; every entry is
 * +-bf16(1/sqrt(d)), so R R^T is the identity times a scalar within 2^-8 of 1.
 * It takes the place of kv_make_rotation's output in kv_cache.rot.  d a power
 * of two in [1, 1024], else KV_EINVAL. */
int kv_make_hadamard_rotation(int32_t d, int32_t bit_reverse, float* rot);

/* QJL matrix from m x d iid N(0,1) draws (row-major fp64): each draw rounded
 * to bf16, written as fp32 (same section, stage two). */
int kv_make_projection(const double* gauss, int32_t m, int32_t d, float* proj);

/* Hierarchical sparse indexing, full mode (page "How DeepSeek-V4.1-Flash cut
 * KV-cache storage by 4x via CSA2", HSI section: the first layer scores every
 * position, keeps the blocks of 8 with the largest maximum score, 2048 of them,
 * as the candidate pool).  Per sequence b with L = min(seq_lens[b],
 * score_stride): the score of block j is the largest of scores[b][t] over
 * t in [j*block, min(L, (j+1)*block)); the top_blocks blocks with the largest
 * scores (all when there are fewer; equal scores: the lower block first) give
 * pool[b][0 .. pool_n[b]), their positions below L in ascending order.
 *   scores     device f32 [B][score_stride], finite (-0 equals +0); the
 *              indexer's scores, an input
 *   seq_lens   device int32 [B]
 *   pool       device int32 [B][top_blocks * block] out (entries past pool_n[b]
 *              are left as they were); pool_n device int32 [B] out
 *   ws         device workspace, 4-byte aligned; ws NULL: *ws_bytes is set to
 *              its size (B * ceil(score_stride / block) * 4) and nothing runs
 * block in [1, 64], top_blocks >= 1, B <= 65535, else KV_EINVAL. */
int kv_hsi_candidates(const float* scores, int32_t batch, int32_t score_stride, const int32_t* seq_lens,
                      int32_t block, int32_t top_blocks, int32_t* pool, int32_t* pool_n, void* ws,
                      size_t* ws_bytes, void* stream);

/* Hierarchical sparse indexing, reindex mode (same section: later layers score
 * only the pool and keep the final top 512).  Per sequence b: of the entries
 * pool[b][0 .. min(pool_n[b], pool_cap)), the top_k with the largest
 * pool_scores[b][i] (all when there are fewer; equal scores: the earlier entry
 * first) as positions in pool order, sel[b][0 .. sel_n[b]).
 *   pool_scores  device f32 [B][pool_cap], finite: the layer's score of pool
 *                entry i (an input)
 *   pool, pool_n device, as kv_hsi_candidates writes them (pool_cap = its row
 *                length)
 *   sel          device int32 [B][top_k] out; sel_n device int32 [B] out */
int kv_hsi_select(const float* pool_scores, const int32_t* pool, const int32_t* pool_n, int32_t batch,
                  int32_t pool_cap, int32_t top_k, int32_t* sel, int32_t* sel_n, void* stream);

/* Decode over selected positions (same section: attention reads only the
 * top-k positions).  As kv_decode_attention with one query per sequence, but
 * query (b, hq) attends over the positions sel[b][0 .. min(sel_n[b], sel_cap))
 * only: a softmax over their logits.  Positions outside [0, capacity) (and
 * rows on pages outside a paged pool) are skipped; a sequence with none left
 * gets zeros.  KIVI2 keys past a sequence's coded groups come from K_STAGE as
 * in dense decode.  Caches with bf16 windows and opts->num_queries > 1 are
 * KV_EUNSUPPORTED, and so is sel_cap > 524,288 on a contiguous FP4, QJL1,
 * TURBO or LATENT cache (their kernels stage at most 512 positions per split,
 * 1024 splits).  The workspace size (a call with ws NULL) depends on
 * sel_cap and opts->num_splits. */
int kv_decode_attention_sparse(const kv_cache* c, const void* q, int32_t q_dtype, int32_t num_q_heads,
                               const int32_t* sel, const int32_t* sel_n, int32_t sel_cap, float softmax_scale,
                               float* out, void* ws, size_t* ws_bytes, const kv_decode_opts* opts, void* stream);

/* Static description of a status code. */
const char* kv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
