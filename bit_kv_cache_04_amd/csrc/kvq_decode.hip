// Decode attention over the packed cache: query preparation, split-context
// attention with an online softmax, and the log-sum-exp merge of the splits.
//
// Every new token reads the whole cache (page "TurboQuant vs OSCAR vs EpiCache",
// KV-cache memory bottleneck section), so the attention kernel streams packed
// tiles once and never writes scores to memory (page "How TriAttention cut LLM
// memory use 10x without losing accuracy": fused attention keeps the score
// matrix on chip).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_kernels.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  // cache
  const uint8_t* k_codes;
  const void* k_scale;
  const float* k_zero;
  const float* k_stage;  // KIVI2 [B][H][4 + 32 d]: tokens appended (int), then the incomplete group's keys
  const uint8_t* k_sketch;
  const uint16_t* k_norm;
  const uint16_t* k_rnorm;
  const uint8_t* v_codes;
  const void* v_scale;
  const float* v_zero;
  const uint16_t* v_norm;
  const uint16_t* rope;
  const float* levels;
  int H, cap, d, rope_dim;
  PageMap pm;  // token rows (paged storage or contiguous)
  // sparse decode: slot i of sequence b reads position sel[b * sel_stride + i]
  // (seq_lens then counts slots); nullptr: slot i is position i
  const int32_t* sel;
  int sel_stride;
  // query / output
  const float* qv;  // prepared queries [B][nq][Hq][QW]
  int Hq, G, head_blocks, hb_size;
  int nq, Gr;       // query tokens per sequence, query heads per KV head (G = nq * Gr)
  const int32_t* seq_lens;
  int max_len;
  float scale_log2;  // softmax scale * log2(e)
  float kappa;       // sqrt(pi/2) / m
  float* part;       // [B][nq][Hq][part_splits][DV + 2]: m (log2 units), l, o[DV]
  int splits, per_split;
  int t_lo, recent, part_splits;  // packed tokens [t_lo, L - recent), split s from t_lo + s * per_split
  // KIVI2 dense decode: the splits stop at the first staged token; with
  // tail_split >= 0 the workgroups of grid column `splits` (one per KV head,
  // head block and sequence) take the staged tokens and write partial split
  // tail_split
  int tail_split;
};

// ---------------------------------------------------------------- per-format element access

// Virtual key element c of token t of sequence-head bh, at cache row `row`; the
// logit is <prepared q, key>.  kstage: the first token whose key is read from
// staging (KIVI2 only).
template <int FMT>
__device__ __forceinline__ float key_elem(const DecodeArgs& a, size_t bh, size_t row, int t, int c, int kstage) {
  if constexpr (FMT == KV_FMT_FP4 || FMT == KV_FMT_LATENT_FP4) {
    if (FMT == KV_FMT_LATENT_FP4 && c >= a.d) return bf16_to_f32(a.rope[row * a.rope_dim + (c - a.d)]);
    const uint32_t nib = (a.k_codes[row * (a.d / 2) + c / 2] >> (4 * (c & 1))) & 15u;
    const float s = bf16_to_f32(static_cast<const uint16_t*>(a.k_scale)[row * (a.d / 16) + c / 16]);
    return e2m1_value(nib) * s;
  } else if constexpr (FMT == KV_FMT_KIVI2) {
    if (t >= kstage) return a.k_stage[bh * (4 + 32 * a.d) + 4 + (t & 31) * a.d + c];  // not yet coded
    const uint32_t code = (a.k_codes[row * (a.d / 4) + c / 4] >> (2 * (c & 3))) & 3u;
    const size_t m = row / 32 * a.d + c;  // pages and the layout hold whole groups
    return fmaf((float)code, static_cast<const float*>(a.k_scale)[m], a.k_zero[m]);
  } else if constexpr (FMT == KV_FMT_TURBO) {
    const float n = f16_to_f32(a.k_norm[row]);
    if (c < 128) {
      const uint32_t code = (a.k_codes[row * 32 + c / 4] >> (2 * (c & 3))) & 3u;
      return n * a.levels[code];
    }
    const int i = c - 128;
    const uint32_t bit = (a.k_sketch[row * 16 + i / 8] >> (i & 7)) & 1u;
    const float g = f16_to_f32(a.k_rnorm[row]);
    return (bit ? 1.f : -1.f) * (a.kappa * g * n);
  } else {  // QJL1
    const float n = f16_to_f32(a.k_norm[row]);
    const uint32_t bit = (a.k_sketch[row * 16 + c / 8] >> (c & 7)) & 1u;
    return (bit ? 1.f : -1.f) * (a.kappa * n);
  }
}

// Value element c of the token at cache row `row` (TURBO: in the rotated space,
// times n_v).
template <int FMT>
__device__ __forceinline__ float value_elem(const DecodeArgs& a, size_t row, int c) {
  if constexpr (FMT == KV_FMT_FP4 || FMT == KV_FMT_QJL1_FP4V) {
    const uint32_t nib = (a.v_codes[row * (a.d / 2) + c / 2] >> (4 * (c & 1))) & 15u;
    const float s = bf16_to_f32(static_cast<const uint16_t*>(a.v_scale)[row * (a.d / 16) + c / 16]);
    return e2m1_value(nib) * s;
  } else if constexpr (FMT == KV_FMT_KIVI2) {
    const uint32_t code = (a.v_codes[row * (a.d / 4) + c / 4] >> (2 * (c & 3))) & 3u;
    const size_t m = row * (a.d / 32) + c / 32;
    return fmaf((float)code, static_cast<const float*>(a.v_scale)[m], a.v_zero[m]);
  } else if constexpr (FMT == KV_FMT_TURBO) {
    const uint32_t code = (a.v_codes[row * 32 + c / 4] >> (2 * (c & 3))) & 3u;
    return f16_to_f32(a.v_norm[row]) * a.levels[code];
  } else {
    return 0.f;  // latent values alias the key tile
  }
}

// ---------------------------------------------------------------- split-context attention

// One workgroup per (split, KV head x head block, sequence).  Each token tile is
// dequantised into LDS once and used by every query head of the block; the
// running max / sum per head implement the online softmax.
template <int FMT, int DK, int DV, int TT, int HB>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  constexpr bool kAlias = (FMT == KV_FMT_LATENT_FP4);
  constexpr int NT = 256;
  constexpr int OPT = (HB * DV + NT - 1) / NT;
  __shared__ float qs[HB][DK];
  __shared__ float ks[TT][DK + 1];
  __shared__ float vs[kAlias ? 1 : TT][kAlias ? 1 : DV + 1];
  __shared__ float ss[HB][TT];
  __shared__ float ms[HB], ls[HB], al[HB];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int h = blockIdx.y / a.head_blocks, hb = blockIdx.y % a.head_blocks;
  const int b = blockIdx.z;
  const int vh0 = hb * a.hb_size;  // first row (query j, head g: row j * Gr + g) of this block
  const int nh = min(a.hb_size, a.G - vh0);
  const size_t bh = (size_t)b * a.H + h;
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  // KIVI2: keys from the first token of the appended sequence's incomplete group on are staged
  const int kstage = FMT == KV_FMT_KIVI2 ? reinterpret_cast<const int*>(a.k_stage)[bh * (4 + 32 * a.d)] & ~31 : a.cap;
  const bool tail = FMT == KV_FMT_KIVI2 && a.tail_split >= 0 && split == a.splits;
  const int t_begin = tail ? max(a.t_lo, kstage) : a.t_lo + split * a.per_split;
  int t_end = tail ? max(a.t_lo, L - a.recent) : min(max(a.t_lo, L - a.recent), t_begin + a.per_split);
  if (FMT == KV_FMT_KIVI2 && !a.sel && !tail) t_end = min(t_end, kstage);  // the staged tokens: the tail split
  const int out_split = tail ? a.tail_split : split;
  // query / output row of block row hh; query j sees the first L - (nq - 1 - j) tokens
  auto qrow = [&](int hh) {
    const int vh = vh0 + hh;
    return ((size_t)b * a.nq + vh / a.Gr) * a.Hq + (size_t)h * a.Gr + vh % a.Gr;
  };
  __shared__ int lim[HB];
  __shared__ size_t trow[TT];  // cache rows of the tile's tokens (kNoRow: no row; masked)
  __shared__ int tpos[TT];     // their positions

  for (int e = tid; e < HB * DK; e += NT) {
    const int hh = e / DK, c = e % DK;
    qs[hh][c] = hh < nh ? a.qv[qrow(hh) * DK + c] : 0.f;
  }
  if (tid < HB) {
    ms[tid] = -INFINITY;
    ls[tid] = 0.f;
    lim[tid] = L - (a.nq - 1 - (vh0 + tid) / a.Gr);
  }
  float o[OPT];
#pragma unroll
  for (int j = 0; j < OPT; ++j) o[j] = 0.f;
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    const int nt = min(TT, t_end - t0);
    if (tid < TT) {
      const int pos = tid >= nt ? -1 : a.sel ? a.sel[(size_t)b * a.sel_stride + t0 + tid] : t0 + tid;
      tpos[tid] = pos;
      trow[tid] = pos >= 0 && pos < a.cap ? token_row(a.pm, a.H, b, h, pos) : kNoRow;
    }
    __syncthreads();
    for (int e = tid; e < TT * DK; e += NT) {
      const int t = e / DK, c = e % DK;
      const size_t row = trow[t];
      ks[t][c] = t < nt && row != kNoRow ? key_elem<FMT>(a, bh, row, tpos[t], c, kstage) : 0.f;
    }
    if constexpr (!kAlias) {
      for (int e = tid; e < TT * DV; e += NT) {
        const int t = e / DV, c = e % DV;
        vs[t][c] = t < nt && trow[t] != kNoRow ? value_elem<FMT>(a, trow[t], c) : 0.f;
      }
    }
    __syncthreads();
    for (int p = tid; p < HB * TT; p += NT) {
      const int hh = p / TT, t = p % TT;
      float s = 0.f;
      for (int c = 0; c < DK; ++c) s = fmaf(qs[hh][c], ks[t][c], s);
      ss[hh][t] = (t < nt && hh < nh && t0 + t < lim[hh] && trow[t] != kNoRow) ? s * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    if (tid < nh) {
      float mx = -INFINITY;
      for (int t = 0; t < nt; ++t) mx = fmaxf(mx, ss[tid][t]);
      const float mnew = fmaxf(ms[tid], mx);
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // a row that has seen no token yet
      const float alpha = exp2f(ms[tid] - mref);
      float sum = 0.f;
      for (int t = 0; t < TT; ++t) {
        const float p = t < nt ? exp2f(ss[tid][t] - mref) : 0.f;
        ss[tid][t] = p;
        sum += p;
      }
      ls[tid] = ls[tid] * alpha + sum;
      ms[tid] = mnew;
      al[tid] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int e = tid + j * NT;
      if (e < HB * DV) {
        const int hh = e / DV, c = e % DV;
        if (hh < nh) {
          float acc = o[j] * al[hh];
          for (int t = 0; t < nt; ++t) acc = fmaf(ss[hh][t], kAlias ? ks[t][c] : vs[t][c], acc);
          o[j] = acc;
        }
      }
    }
    __syncthreads();
  }
  // partial results of this split
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int e = tid + j * NT;
    if (e < HB * DV) {
      const int hh = e / DV, c = e % DV;
      if (hh < nh) {
        float* p = a.part + (qrow(hh) * a.part_splits + out_split) * (DV + 2);
        p[2 + c] = o[j];
        if (c == 0) {
          p[0] = ms[hh];
          p[1] = ls[hh];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 windows

// Mixed precision: attention of the (query, head) rows of one (sequence, KV
// head) over the tokens its cache keeps in bf16, the sink t < S and the recent
// t >= L - W (the packed kernels cover [S, L - W)).  The logit is <q, bf16 key>.
// Window positions p enumerate those tokens in order; workgroup (chunk, row
// block) takes positions [64 chunk, 64 chunk + 64) for 16 rows and writes them
// as split `split + chunk` of the partial rows, so that the window's short
// serial chains run side by side.
constexpr int kWinChunk = 64;

struct WindowArgs {
  const void* q;  // raw queries [B][nq][Hq][D] (fp32 or bf16)
  const uint16_t *sink_k, *sink_v, *rec_k, *rec_v;
  const int32_t* seq_lens;
  int max_len, cap, H, Hq, gr, nq, S, W;
  float scale_log2;
  float* part;
  int part_splits, split, row_blocks;
};

template <typename QT, int D>
__global__ void __launch_bounds__(256) decode_window_kernel(WindowArgs a) {
  constexpr int NT = 256, HB = 16, TT = 32, OPT = HB * D / NT, C8 = D / 8;
  __shared__ float qs[HB][D];
  __shared__ float ks[TT][D + 1];
  __shared__ float vs[TT][D + 1];
  __shared__ float ss[HB][TT];
  __shared__ float ms[HB], ls[HB], al[HB];
  __shared__ int lim[HB];
  const int tid = threadIdx.x;
  const int rb = blockIdx.x % a.row_blocks, chunk = blockIdx.x / a.row_blocks;
  const int h = blockIdx.y, b = blockIdx.z;
  const int vh0 = rb * HB;
  const int nh = min(HB, a.nq * a.gr - vh0);
  const size_t bh = (size_t)b * a.H + h;
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  const int ns = min(a.S, L);        // sink tokens [0, ns)
  const int rs = max(a.S, L - a.W);  // recent tokens [rs, L)
  const int nw = ns + max(0, L - rs);
  const int p_begin = chunk * kWinChunk, p_end = min(nw, p_begin + kWinChunk);
  auto token = [&](int p) { return p < ns ? p : rs + (p - ns); };
  auto qrow = [&](int hh) {
    const int vh = vh0 + hh;
    return ((size_t)b * a.nq + vh / a.gr) * a.Hq + (size_t)h * a.gr + vh % a.gr;
  };
  for (int e = tid; e < HB * D; e += NT) {
    const int hh = e / D, c = e % D;
    qs[hh][c] = hh < nh ? load_as_f32(static_cast<const QT*>(a.q) + qrow(hh) * D, c) : 0.f;
  }
  if (tid < HB) {
    ms[tid] = -INFINITY;
    ls[tid] = 0.f;
    lim[tid] = L - (a.nq - 1 - (vh0 + tid) / a.gr);
  }
  float o[OPT];
#pragma unroll
  for (int j = 0; j < OPT; ++j) o[j] = 0.f;
  __syncthreads();
  for (int p0 = p_begin; p0 < p_end; p0 += TT) {
    const int nt = min(TT, p_end - p0);
    // 8 bf16 of one token's K and V per thread and step (16-byte loads)
    for (int e = tid; e < TT * C8; e += NT) {
      const int t = e / C8, c8 = (e % C8) * 8;
      uint4 kr{0u, 0u, 0u, 0u}, vr{0u, 0u, 0u, 0u};
      if (t < nt) {
        const int tok = token(p0 + t);
        const size_t off = tok < a.S ? (bh * a.S + tok) * D + c8 : (bh * a.W + tok % a.W) * D + c8;
        kr = *reinterpret_cast<const uint4*>((tok < a.S ? a.sink_k : a.rec_k) + off);
        vr = *reinterpret_cast<const uint4*>((tok < a.S ? a.sink_v : a.rec_v) + off);
      }
      const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w}, vw[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ks[t][c8 + 2 * i] = __uint_as_float(kw[i] << 16);
        ks[t][c8 + 2 * i + 1] = __uint_as_float(kw[i] & 0xFFFF0000u);
        vs[t][c8 + 2 * i] = __uint_as_float(vw[i] << 16);
        vs[t][c8 + 2 * i + 1] = __uint_as_float(vw[i] & 0xFFFF0000u);
      }
    }
    __syncthreads();
    for (int p = tid; p < nh * TT; p += NT) {
      const int hh = p / TT, t = p % TT;
      float sx = 0.f;
      for (int c = 0; c < D; ++c) sx = fmaf(qs[hh][c], ks[t][c], sx);
      ss[hh][t] = (t < nt && token(p0 + t) < lim[hh]) ? sx * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    if (tid < nh) {
      float mx = -INFINITY;
      for (int t = 0; t < nt; ++t) mx = fmaxf(mx, ss[tid][t]);
      const float mnew = fmaxf(ms[tid], mx);
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // a row that has seen no token yet
      const float alpha = exp2f(ms[tid] - mref);
      float sum = 0.f;
      for (int t = 0; t < TT; ++t) {
        const float pw = t < nt ? exp2f(ss[tid][t] - mref) : 0.f;
        ss[tid][t] = pw;
        sum += pw;
      }
      ls[tid] = ls[tid] * alpha + sum;
      ms[tid] = mnew;
      al[tid] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int e = tid + j * NT, hh = e / D, c = e % D;
      if (hh < nh) {
        float acc = o[j] * al[hh];
        for (int t = 0; t < nt; ++t) acc = fmaf(ss[hh][t], vs[t][c], acc);
        o[j] = acc;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int e = tid + j * NT, hh = e / D, c = e % D;
    if (hh < nh) {
      float* p = a.part + (qrow(hh) * a.part_splits + a.split + chunk) * (D + 2);
      p[2 + c] = o[j];
      if (c == 0) {
        p[0] = ms[hh];
        p[1] = ls[hh];
      }
    }
  }
}

// ---------------------------------------------------------------- query preparation

// Nearest E4M3 (OCP FP8, 3 mantissa bits) of y, |y| < 128: the code and its
// value; magnitudes below the smallest normal, 2^-6, become zero (the caller
// keeps them in its residual).
__device__ __forceinline__ uint32_t e4m3_code(float y, float& val) {
  const uint32_t sgn = __float_as_uint(y) & 0x80000000u;
  const float ay = fabsf(y);
  if (!(ay >= 0x1p-6f)) {
    val = 0.f;
    return 0u;
  }
  uint32_t u = __float_as_uint(ay);
  u = (u + 0x7FFFFu + ((u >> 20) & 1u)) & ~0xFFFFFu;  // ties to even on 3 mantissa bits
  val = __uint_as_float(u | sgn);
  const uint32_t ef = (u >> 23) - 127u + 7u;            // 1 .. 14
  return (sgn >> 24) | (ef << 3) | ((u >> 20) & 7u);
}

// FP6 E2M3 code of y, |y| < 4.25, rounded to nearest even: steps of 1/8 below 2
// (subnormals 0 .. 7/8 and [1, 2)), 1/4 in [2, 4), 1/2 from 4.  `val` is the
// value the code stands for.
__device__ __forceinline__ uint32_t e2m3_code(float y, float& val) {
  const uint32_t sgn = __float_as_uint(y) >> 31;
  const float ay = fabsf(y);
  const float step = ay < 2.f ? 0.125f : (ay < 4.f ? 0.25f : 0.5f);
  const float inv = ay < 2.f ? 8.f : (ay < 4.f ? 4.f : 2.f);  // 1 / step, a power of two
  const float qv = __builtin_rintf(ay * inv) * step;           // exact quotient, ties to even
  val = sgn ? -qv : qv;
  uint32_t mag;
  if (qv < 1.f) {
    mag = (uint32_t)(qv * 8.f);  // exponent field 0
  } else {
    const int e = qv < 2.f ? 1 : (qv < 4.f ? 2 : 3);  // exponent field, bias 1
    const float unit = e == 1 ? 1.f : (e == 2 ? 0.5f : 0.25f);  // 2^-(e - 1)
    mag = ((uint32_t)e << 3) | (uint32_t)((qv * unit - 1.f) * 8.f);
  }
  return (sgn << 5) | mag;
}

// Query pieces of the bit-key products (TurboQuant, QJL).  The key products
// take the key bits as FP4 operands (one bit per nibble) against FP8 (QJL) or
// FP6 (TurboQuant) operands with a power-of-two scale per block of 32
// (v_mfma_scale_f32_16x16x128_f8f6f4).  Block j (element e = 8 d + n, the bit
// 4 n + d of one key word) of
//   TURBO product 0 / 1 (code words 4 m + j, m = 0 / 1): the coefficient of
//     bit d % 2 (a2 for the low bit b0, a1 for the high bit b1) times
//     (R q)[16 (4 m + j) + 2 n + d / 2];
//   TURBO product 2, QJL product 0 (sketch dword j): ask (S R q or S q)[32 j + 4 n + d].
// Each block is split into 4 pieces: piece p holds the nearest code of the
// residual left by pieces < p, at a scale 2^e that puts the residual's largest
// magnitude in [64, 128) for E4M3 (3 mantissa bits to 448: the pieces' sum is
// within 2^-20 of the block's largest value) or in [2, 4) for E2M3 (3 mantissa
// bits to 7.5, steps of 1/8 below 2: each piece leaves at most 2^-4 of the
// residual's largest magnitude, the sum is within 2^-16).  Layout per (product,
// piece): 4 blocks of 32 bytes (E4M3: byte e = element e; E2M3: 24 bytes, element
// e at bits [6 e, 6 e + 6)), then the 4 blocks' E8M0 scale bytes (e + 127), 144
// bytes in all.  32 threads per block, as many blocks at a time as the workgroup
// has threads for.
// Threads [0, nthr) of the caller's group (tid = index in the group, both
// multiples of 32 apart from tid's low bits) do the work.
// Lane exchanges within a 16-lane row by DPP (quad permutations, row rotations).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
// max of x over the 32 lanes of its half-wave: quad exchanges, two row
// rotations, then the row pair
__device__ __forceinline__ float max_half_wave(float x) {
  x = fmaxf(x, __uint_as_float(dpp_u<0xB1>(__float_as_uint(x))));   // lane ^ 1
  x = fmaxf(x, __uint_as_float(dpp_u<0x4E>(__float_as_uint(x))));   // lane ^ 2
  x = fmaxf(x, __uint_as_float(dpp_u<0x124>(__float_as_uint(x))));  // row_ror:4
  x = fmaxf(x, __uint_as_float(dpp_u<0x128>(__float_as_uint(x))));  // row_ror:8
  return max_xor16(x);
}

__device__ void prepared_query_pieces(int nprod, const float* qrot, const float* qsk, float a1, float a2, float ask,
                                      bool fp6, uint8_t* out, int tid, int nthr) {
  const int e = tid & 31, d = e >> 3, n = e & 7;
  // TURBO (FP6): the key operand's element 8 d + n is its bit times 1, 2, 4, 4
  // for d = 0, 1, 2, 3, so this side carries 1, 1/2, 1/4, 1/4
  const float dfac = fp6 ? (d == 0 ? 1.f : d == 1 ? 0.5f : 0.25f) : 1.f;
  for (int blk = tid >> 5; blk < 4 * nprod; blk += nthr >> 5) {
    const int prod = blk >> 2, j = blk & 3;
    const bool code = prod < nprod - 1;
    float r = dfac * (code ? ((d & 1) ? a1 : a2) * qrot[16 * (4 * prod + j) + 2 * n + (d >> 1)]
                           : ask * qsk[32 * j + 4 * n + d]);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float M = max_half_wave(fabsf(r));
      int ex = 0;
      if (M > 0.f) {
        int k;
        frexpf(M, &k);  // M = f 2^k, f in [0.5, 1)
        ex = k - (fp6 ? 2 : 7);
      }
      if (ex < -127) {  // a residual below the scales' range is left out
        ex = -127;
        r = 0.f;
      }
      float val;
      uint8_t* dst = out + (prod * 4 + p) * 144;
      if (fp6) {
        // elements 4 g .. 4 g + 3 fill the 3 bytes from 3 g: gather them in 2 steps
        uint32_t v = e2m3_code(ldexpf(r, -ex), val) << (6 * (e & 3));
        v |= dpp_u<0xB1>(v);  // lane ^ 1
        v |= dpp_u<0x4E>(v);  // lane ^ 2
        if ((e & 3) == 0) {
          uint8_t* b3 = dst + j * 32 + 3 * (e >> 2);
          b3[0] = (uint8_t)v;
          b3[1] = (uint8_t)(v >> 8);
          b3[2] = (uint8_t)(v >> 16);
        }
      } else {
        dst[j * 32 + e] = (uint8_t)e4m3_code(ldexpf(r, -ex), val);
      }
      r -= ldexpf(val, ex);
      if (e == 0) dst[128 + j] = (uint8_t)(ex + 127);
    }
  }
}

// Prepared fp32 query of the formats other than TURBO (prep_turbo_kernel):
// S q (QJL1), with the FP8 pieces of its key product when `pieces` is given,
// or q itself.  128 threads; the product takes one output per thread, whose
// row of S is loaded into registers beside the query.
template <typename QT>
__global__ void __launch_bounds__(128) prep_query_kernel(const QT* __restrict__ q, int qw_in, int qw_out, int fmt,
                                                         const float* __restrict__ proj, float* __restrict__ out,
                                                         uint8_t* __restrict__ pieces) {
  __shared__ float qin[640];
  __shared__ float qsr[128];
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const bool qjl = fmt == KV_FMT_QJL1_FP4V;
  float4 m[32];
  if (qjl) {
    const float4* src = reinterpret_cast<const float4*>(proj + (size_t)tid * 128);
#pragma unroll
    for (int j4 = 0; j4 < 32; ++j4) m[j4] = src[j4];
  }
  for (int c = tid; c < qw_in; c += nthr) qin[c] = load_as_f32(q + row * qw_in, c);
  __syncthreads();
  float* dst = out + row * qw_out;
  if (qjl) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int j4 = 0; j4 < 32; j4 += 2) {
      const float4 v = m[j4], u = m[j4 + 1];
      acc0 = fmaf(v.x, qin[4 * j4], acc0);
      acc0 = fmaf(v.y, qin[4 * j4 + 1], acc0);
      acc0 = fmaf(v.z, qin[4 * j4 + 2], acc0);
      acc0 = fmaf(v.w, qin[4 * j4 + 3], acc0);
      acc1 = fmaf(u.x, qin[4 * j4 + 4], acc1);
      acc1 = fmaf(u.y, qin[4 * j4 + 5], acc1);
      acc1 = fmaf(u.z, qin[4 * j4 + 6], acc1);
      acc1 = fmaf(u.w, qin[4 * j4 + 7], acc1);
    }
    const float acc = acc0 + acc1;
    dst[tid] = acc;
    qsr[tid] = acc;
    if (pieces) {
      __syncthreads();
      prepared_query_pieces(1, nullptr, qsr, 0.f, 0.f, 1.f, false, pieces + row * kQjlPieceBytes, tid, nthr);
    }
  } else {
    for (int c = tid; c < qw_out; c += nthr) dst[c] = qin[c];
  }
}

// TurboQuant query preparation, one query row per workgroup of 384 threads:
// threads i < 128 form (R q)[i] and then (S R q)[i] from row i of R and S
// (float4 loads), [R q | S R q] is written (fp32, for the general kernel), and
// when `pieces` is given all 12 blocks of FP6 pieces (prepared_query_pieces)
// are made at once, with the constant terms.  An asymmetric codebook (lv0 +
// lv3 != lv1 + lv2), which the bit-plane key products cannot represent, makes
// the constant terms NaN: every output of the matrix-core kernel is then NaN
// rather than silently wrong.
constexpr int kTurboPrepThreads = 384;

template <typename QT>
__global__ void __launch_bounds__(kTurboPrepThreads) prep_turbo_kernel(
    const QT* __restrict__ q, RotArg ra, const float* __restrict__ proj,
    const float* __restrict__ levels, float scale_log2, float kappa, float* __restrict__ out,
    uint8_t* __restrict__ pieces) {
  __shared__ float qin[128];
  __shared__ float qrot[128];
  __shared__ float qsr[128];
  __shared__ float red[2][2];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const bool prod = tid < 128;
  const bool dense = ra.kind == KV_ROT_DENSE;
  // a structured rotation: channel rot_perm(k) at position k, then the butterfly
  if (prod) (dense ? qin : qrot)[tid] = load_as_f32(q + row * 128, dense ? tid : rot_perm(tid, ra.kind));
  const float lv0 = levels[0], lv1 = levels[1], lv2 = levels[2], lv3 = levels[3];
  __syncthreads();
  auto matvec = [&](const float* __restrict__ m, const float* x) {
    const float4* mr = reinterpret_cast<const float4*>(m + (size_t)tid * 128);
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
    for (int j4 = 0; j4 < 32; j4 += 2) {
      const float4 v = mr[j4], u = mr[j4 + 1];
      acc0 = fmaf(v.x, x[4 * j4], acc0);
      acc0 = fmaf(v.y, x[4 * j4 + 1], acc0);
      acc0 = fmaf(v.z, x[4 * j4 + 2], acc0);
      acc0 = fmaf(v.w, x[4 * j4 + 3], acc0);
      acc1 = fmaf(u.x, x[4 * j4 + 4], acc1);
      acc1 = fmaf(u.y, x[4 * j4 + 5], acc1);
      acc1 = fmaf(u.z, x[4 * j4 + 6], acc1);
      acc1 = fmaf(u.w, x[4 * j4 + 7], acc1);
    }
    return acc0 + acc1;
  };
  float rq = 0.f, srq = 0.f;
  if (dense) {
    if (prod) {
      rq = matvec(ra.rot, qin);
      qrot[tid] = rq;
    }
  } else {
    for (int h = 1; h < 128; h <<= 1) {
      hadamard_stage(qrot, 1, 128, h, tid, kTurboPrepThreads);
      __syncthreads();
    }
    if (prod) {
      rq = ra.mag * qrot[tid];
      qrot[tid] = rq;
    }
  }
  __syncthreads();
  if (prod) {
    srq = matvec(proj, qrot);
    qsr[tid] = srq;
    out[row * 256 + tid] = rq;
    out[row * 256 + 128 + tid] = srq;
  }
  if (!pieces) return;  // uniform across the workgroup
  __syncthreads();
  uint8_t* pr = pieces + row * kTurboPieceBytes;
  prepared_query_pieces(3, qrot, qsr, (lv2 - lv0) * scale_log2, (lv1 - lv0) * scale_log2, 2.f * kappa * scale_log2,
                        true, pr, tid, kTurboPrepThreads);
  if (prod) {  // the sums of R q and S R q: two waves
    float sr = rq, ss = srq;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sr += __shfl_xor(sr, off);
      ss += __shfl_xor(ss, off);
    }
    if ((tid & 63) == 0) {
      red[tid >> 6][0] = sr;
      red[tid >> 6][1] = ss;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const bool symmetric = lv0 + lv3 == lv1 + lv2;
    float* cst = reinterpret_cast<float*>(pr + kTurboPieceConstOff);
    cst[0] = symmetric ? lv0 * scale_log2 * (red[0][0] + red[1][0]) : __builtin_nanf("");
    cst[1] = -kappa * scale_log2 * (red[0][1] + red[1][1]);
  }
}

// ---------------------------------------------------------------- merge

// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s, for one
// (sequence, query head) row per blockIdx.x and the columns
// [64 * NJ * blockIdx.y, 64 * NJ * (blockIdx.y + 1)).  The splits' (m, l) pairs
// are read once into LDS and turned into weights there; wave w then sums the
// splits w, w + W, ... (W waves) for every column of the block, lane l owning
// columns NJ * l .. NJ * l + NJ - 1, so that the loads of different splits are
// independent and spread over the block; the W wave sums are added in wave
// order.  TURBO (the whole row in one block) maps the rotated output back with
// R^T, every thread taking a slice of the rows of R; its splits from rot_splits
// on (the bf16 window's) are already in the original basis and are added after
// that product.  A row with no tokens at all writes zeros.
constexpr int kMaxSplits = kMaxPartSplits;

template <int NJ>
constexpr int merge_max_waves() {
  return NJ >= 4 ? 4 : 16;
}

template <int NJ>
__global__ void __launch_bounds__(64 * merge_max_waves<NJ>()) merge_kernel(const float* __restrict__ part,
                                                                           int splits, int rot_splits, int dv,
                                                                           int fmt, RotArg ra,
                                                                           float* __restrict__ out) {
  constexpr int CW = 64 * NJ, MW = merge_max_waves<NJ>();
  constexpr bool kTurboCols = NJ == 2;  // TURBO rows (dv = 128) take this column blocking
  __shared__ float sm_w[kMaxSplits];  // m_s, then the weights
  __shared__ float sm_l[kMaxSplits];
  __shared__ float red_m[MW], red_l[MW];
  __shared__ float sums[MW][CW];
  __shared__ float sums_o[kTurboCols ? MW : 1][kTurboCols ? CW : 1];  // TURBO: splits past rot_splits
  __shared__ float ov[CW], ovo[kTurboCols ? CW : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x, W = nthr >> 6;
  const size_t row = blockIdx.x;
  const size_t stride = (size_t)dv + 2;
  const float* p = part + row * (size_t)splits * stride;
  const bool turbo = fmt == KV_FMT_TURBO;
  const int s_rot = turbo ? rot_splits : splits;
  const int c0 = CW * blockIdx.y;
  const float* pc = p + 2 + c0 + NJ * lane;  // 8-byte aligned: rows and the header are even
  // this wave's first PF splits' outputs (s = wave + W k below s_rot), loaded
  // beside the (m, l) pairs instead of after the weights
  constexpr int PF = 32 / NJ;
  float pre[PF][NJ];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int s = wave + k * W;
#pragma unroll
    for (int j = 0; j < NJ; j += (NJ == 1 ? 1 : 2)) {
      if constexpr (NJ == 1) {
        pre[k][0] = s < s_rot ? pc[s * stride] : 0.f;
      } else {
        const float2 v = s < s_rot ? *reinterpret_cast<const float2*>(pc + s * stride + j) : float2{0.f, 0.f};
        pre[k][j] = v.x;
        pre[k][j + 1] = v.y;
      }
    }
  }
  float M = -INFINITY;
  for (int s = tid; s < splits; s += nthr) {
    const float2 ml = *reinterpret_cast<const float2*>(p + s * stride);
    sm_w[s] = ml.x;
    sm_l[s] = ml.y;
    M = fmaxf(M, ml.x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = red_m[0];
  for (int i = 1; i < W; ++i) M = fmaxf(M, red_m[i]);
  float l = 0.f;
  for (int s = tid; s < splits; s += nthr) {  // each thread revisits only its own entries
    const float ms = sm_w[s];
    const float ws = ms == -INFINITY ? 0.f : exp2f(ms - M);
    sm_w[s] = ws;
    l += ws * sm_l[s];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  if (lane == 0) red_l[wave] = l;
  __syncthreads();
  l = red_l[0];
  for (int i = 1; i < W; ++i) l += red_l[i];
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  constexpr int kMergeUnroll = 16 / NJ;
  // weighted sum of the splits s0, s0 + W, ... below s1 for this lane's
  // columns, in that order (the first PF from the prefetched values if pre)
  auto weighted = [&](int s0, int s1, float (&acc)[NJ], bool use_pre) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = 0.f;
    int s = s0;
    if (use_pre) {
#pragma unroll
      for (int k = 0; k < PF; ++k, s += W) {
        if (s < s1) {
          const float ws = sm_w[s];
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[j] = fmaf(ws, pre[k][j], acc[j]);
        }
      }
    }
#pragma unroll kMergeUnroll
    for (; s < s1; s += W) {
      const float ws = sm_w[s];
      if constexpr (NJ == 1) {
        acc[0] = fmaf(ws, pc[s * stride], acc[0]);
      } else {
#pragma unroll
        for (int j = 0; j < NJ; j += 2) {
          const float2 v = *reinterpret_cast<const float2*>(pc + s * stride + j);
          acc[j] = fmaf(ws, v.x, acc[j]);
          acc[j + 1] = fmaf(ws, v.y, acc[j + 1]);
        }
      }
    }
  };
  {
    float acc[NJ];
    weighted(wave, s_rot, acc, true);
#pragma unroll
    for (int j = 0; j < NJ; ++j) sums[wave][NJ * lane + j] = acc[j];
    if constexpr (kTurboCols) {
      if (turbo) {
        weighted(s_rot + wave, splits, acc, false);
#pragma unroll
        for (int j = 0; j < NJ; ++j) sums_o[wave][NJ * lane + j] = acc[j];
      }
    }
  }
  __syncthreads();
  float* dst = out + row * dv;
  for (int c = tid; c < CW; c += nthr) {
    float t = sums[0][c];
    for (int i = 1; i < W; ++i) t += sums[i][c];
    if (!turbo) {
      dst[c0 + c] = t * inv_l;
    } else if constexpr (kTurboCols) {
      ov[c] = t * inv_l;
      float t2 = sums_o[0][c];
      for (int i = 1; i < W; ++i) t2 += sums_o[i][c];
      ovo[c] = t2 * inv_l;
    }
  }
  if constexpr (kTurboCols) {
    if (!turbo) return;  // CW == dv below
    __syncthreads();
    if (ra.kind != KV_ROT_DENSE) {
      // R^T o = mag (H o) read at the reversed positions
      for (int h = 1; h < CW; h <<= 1) {
        hadamard_stage(ov, 1, CW, h, tid, nthr);
        __syncthreads();
      }
      for (int c = tid; c < CW; c += nthr) dst[c] = ra.mag * ov[rot_perm(c, ra.kind)] + ovo[c];
      return;
    }
    const float* __restrict__ rot = ra.rot;
    // P slices of the rows of R: thread (q, c) sums j in [q * CW / P, (q + 1) * CW / P)
    const int P = nthr >= CW ? min(nthr / CW, MW) : 1;
    const int span = CW / P;
    for (int e = tid; e < P * CW; e += nthr) {
      const int q = e / CW, c = e % CW;
      float a = 0.f;
#pragma unroll 8
      for (int j = q * span; j < (q + 1) * span; ++j) a = fmaf(rot[j * CW + c], ov[j], a);
      sums[q][c] = a;
    }
    __syncthreads();
    for (int c = tid; c < CW; c += nthr) {
      float a = sums[0][c];
      for (int q = 1; q < P; ++q) a += sums[q][c];
      dst[c] = a + ovo[c];
    }
  }
}

// Column blocks: TURBO and many rows take the whole row per block (up to 8
// columns per lane); few rows take 64-column blocks so that more workgroups
// share the loads; otherwise 128 columns.  Waves: about four splits each.
void launch_merge(const float* part, int rows, int splits, int rot_splits, int dv, int fmt, RotArg rot,
                  float* out, hipStream_t st) {
  int nj;
  if (fmt == KV_FMT_TURBO || rows >= 2048) nj = dv / 64;
  else if (rows < 256 || dv % 128 != 0) nj = 1;
  else nj = 2;
  const int col_blocks = dv / (64 * nj);
  const dim3 grid(rows, col_blocks);
  auto waves = [&](int max_w) { return std::min(max_w, std::max(1, (splits + 3) / 4)); };
  switch (nj) {
    case 1: merge_kernel<1><<<grid, 64 * waves(merge_max_waves<1>()), 0, st>>>(part, splits, rot_splits, dv, fmt, rot, out); break;
    case 2: merge_kernel<2><<<grid, 64 * waves(merge_max_waves<2>()), 0, st>>>(part, splits, rot_splits, dv, fmt, rot, out); break;
    default: merge_kernel<8><<<grid, 64 * waves(merge_max_waves<8>()), 0, st>>>(part, splits, rot_splits, dv, fmt, rot, out); break;
  }
}

template <int FMT, int DK, int DV, int HB>
void launch_split(const DecodeArgs& a, int B, hipStream_t st) {
  dim3 grid(a.splits + (a.tail_split >= 0 ? 1 : 0), a.H * a.head_blocks, B);
  decode_split_kernel<FMT, DK, DV, 32, HB><<<grid, 256, 0, st>>>(a);
}

// The bf16 window split of a mixed-precision cache (partial split `split`).
void launch_window(const kv_cache* c, const void* q, int q_dtype, int num_q_heads, int nq, const int32_t* seq_lens,
                   int max_seq_len, float scale, float* part, int part_splits, int split, hipStream_t st) {
  const kv_layout& L = c->layout;
  WindowArgs w{};
  w.q = q;
  w.sink_k = static_cast<const uint16_t*>(c->buf[KV_BUF_SINK_K]);
  w.sink_v = static_cast<const uint16_t*>(c->buf[KV_BUF_SINK_V]);
  w.rec_k = static_cast<const uint16_t*>(c->buf[KV_BUF_RECENT_K]);
  w.rec_v = static_cast<const uint16_t*>(c->buf[KV_BUF_RECENT_V]);
  w.seq_lens = seq_lens;
  w.max_len = max_seq_len;
  w.cap = L.capacity;
  w.H = L.num_kv_heads;
  w.Hq = num_q_heads;
  w.gr = num_q_heads / L.num_kv_heads;
  w.nq = nq;
  w.S = L.sink_tokens;
  w.W = L.recent_tokens;
  w.scale_log2 = scale * kLog2e;
  w.part = part;
  w.part_splits = part_splits;
  w.split = split;
  w.row_blocks = (nq * w.gr + 15) / 16;
  const dim3 grid(w.row_blocks * window_chunks(L), L.num_kv_heads, L.batch);
  const bool f32 = q_dtype == KV_DT_F32;
  if (L.head_dim == 64) {
    if (f32) decode_window_kernel<float, 64><<<grid, 256, 0, st>>>(w);
    else decode_window_kernel<uint16_t, 64><<<grid, 256, 0, st>>>(w);
  } else {
    if (f32) decode_window_kernel<float, 128><<<grid, 256, 0, st>>>(w);
    else decode_window_kernel<uint16_t, 128><<<grid, 256, 0, st>>>(w);
  }
}

}  // namespace

// Arguments of the general kernel (and of the KIVI2 staging tail).
static DecodeArgs general_args(const kv_cache* c, int num_q_heads, int nq, const int32_t* seq_lens, int max_seq_len,
                               float scale, const float* qv, float* part, const SplitPlan& plan, int part_splits,
                               const int32_t* sel, int sel_stride) {
  const kv_layout& L = c->layout;
  DecodeArgs a{};
  a.k_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_K_CODES]);
  a.k_scale = c->buf[KV_BUF_K_SCALE];
  a.k_zero = static_cast<const float*>(c->buf[KV_BUF_K_ZERO]);
  a.k_stage = static_cast<const float*>(c->buf[KV_BUF_K_STAGE]);
  a.k_sketch = static_cast<const uint8_t*>(c->buf[KV_BUF_K_SKETCH]);
  a.k_norm = static_cast<const uint16_t*>(c->buf[KV_BUF_K_NORM]);
  a.k_rnorm = static_cast<const uint16_t*>(c->buf[KV_BUF_K_RNORM]);
  a.v_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_V_CODES]);
  a.v_scale = c->buf[KV_BUF_V_SCALE];
  a.v_zero = static_cast<const float*>(c->buf[KV_BUF_V_ZERO]);
  a.v_norm = static_cast<const uint16_t*>(c->buf[KV_BUF_V_NORM]);
  a.rope = static_cast<const uint16_t*>(c->buf[KV_BUF_ROPE]);
  a.levels = c->lm_levels;
  a.H = L.num_kv_heads;
  a.cap = L.capacity;
  a.d = L.head_dim;
  a.rope_dim = L.rope_dim;
  a.pm = page_map(c);
  a.sel = sel;
  a.sel_stride = sel_stride;
  a.qv = qv;
  a.Hq = num_q_heads;
  a.nq = nq;
  a.Gr = num_q_heads / L.num_kv_heads;
  a.G = nq * a.Gr;  // rows per (sequence, KV head): query j, head g is row j * Gr + g
  a.hb_size = std::min(a.G, 16);
  a.head_blocks = (a.G + a.hb_size - 1) / a.hb_size;
  a.seq_lens = seq_lens;
  a.max_len = max_seq_len;
  a.scale_log2 = scale * kLog2e;
  a.kappa = (float)(1.2533141373155002512 / (double)(L.qjl_m > 0 ? L.qjl_m : 1));
  a.part = part;
  a.splits = plan.splits;
  a.per_split = plan.tokens_per_split;
  a.t_lo = L.sink_tokens;
  a.recent = L.recent_tokens;
  a.part_splits = part_splits;
  a.tail_split = -1;
  return a;
}

// KIVI2 dense decode: the staged tokens of every (sequence, KV head) as partial
// split `split` (one workgroup per (KV head, head block, sequence)).
static void launch_kivi_tail(DecodeArgs a, int split, int B, hipStream_t st) {
  a.tail_split = split;
  a.splits = 0;  // the launch's workgroups are all tail workgroups
  const dim3 grid(1, a.H * a.head_blocks, B);
  if (a.d == 64) decode_split_kernel<KV_FMT_KIVI2, 64, 64, 32, 16><<<grid, 256, 0, st>>>(a);
  else decode_split_kernel<KV_FMT_KIVI2, 128, 128, 32, 16><<<grid, 256, 0, st>>>(a);
}

int launch_decode(const kv_cache* c, const void* q, int q_dtype, int num_q_heads, int nq, const int32_t* seq_lens,
                  int max_seq_len, float scale, float* out, void* ws, const SplitPlan& plan,
                  const DecodeWorkspace& wsl, void* ev_begin, void* ev_end, void* stream, const int32_t* sel,
                  int sel_stride, bool fp32) {
  const kv_layout& L = c->layout;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  float* qv = reinterpret_cast<float*>(wsb + wsl.qprep_off);
  float* part = reinterpret_cast<float*>(wsb + wsl.part_off);
  const int B = L.batch;
  const int rows = B * nq * num_q_heads;  // (sequence, query token, query head)
  // mixed precision: the packed kernels take [sink, L - recent) and the bf16
  // window kernel one more split
  const bool windowed = L.sink_tokens || L.recent_tokens;
  // KIVI2 dense decode: the staged tokens take the split after the window's
  const int tail_split = sel || !tail_chunks(L) ? -1 : plan.splits + window_chunks(L);
  const int part_splits = plan.splits + window_chunks(L) + (tail_split >= 0 ? 1 : 0);
  const int qw_in = query_width(&L), qw_out = prepared_query_width(&L);
  // fp32: every format on the general kernel (exact for any magnitude)
  if (!fp32 && (sel ? latent_sparse_ok(L, num_q_heads, q_dtype) : latent_fast_path_ok(L, num_q_heads, nq, q_dtype))) {
    MfmaDecodeArgs f{};
    f.k_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_K_CODES]);
    f.k_scale = static_cast<const uint16_t*>(c->buf[KV_BUF_K_SCALE]);
    f.rope = static_cast<const uint16_t*>(c->buf[KV_BUF_ROPE]);
    f.pm = page_map(c);
    f.sel = sel;
    f.sel_stride = sel_stride;
    f.q = q;
    f.seq_lens = seq_lens;
    f.max_len = max_seq_len;
    f.H = L.num_kv_heads;
    f.cap = L.capacity;
    f.Hq = num_q_heads;
    f.scale_log2 = scale * kLog2e;
    f.part = part;
    f.splits = plan.splits;
    f.per_split = plan.tokens_per_split;
    f.nq = nq;
    if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return KV_EDEVICE;
    for (f.c0 = 0; f.c0 < nq; ++f.c0) {  // one pass over the cache per query token
      int rc = launch_decode_latent(f, B, st);
      if (rc != KV_OK) return rc;
    }
    if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), st) != hipSuccess) return KV_EDEVICE;
    launch_merge(part, rows, part_splits, plan.splits, L.head_dim, L.format, rot_arg(c), out, st);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
  }
  const bool mfma =
      !fp32 && (sel ? mfma_sparse_ok(L, num_q_heads, q_dtype) : mfma_fast_path_ok(L, num_q_heads, nq, q_dtype));
  const bool turbo = !fp32 && (sel ? turbo_sparse_ok(L, num_q_heads) : turbo_fast_path_ok(L, num_q_heads, nq));
  // FP4 keys read the caller's bf16 queries as they are; every other format
  // first prepares its fp32 query (projection / rotation)
  uint8_t* qpieces = turbo || (mfma && L.format == KV_FMT_QJL1_FP4V)
                         ? reinterpret_cast<uint8_t*>(wsb + wsl.qpiece_off)
                         : nullptr;
  const float kappa = (float)(1.2533141373155002512 / (double)(L.qjl_m > 0 ? L.qjl_m : 1));
  // KIVI-2 on the matrix cores: on grids under 256 workgroups the staged tokens
  // take a last column of the same launch (their launch latency then
  // dominates; at scale that column's code measured slower for the main
  // workgroups), else the general kernel; there fp32 queries are read as they
  // are (every other path reads the prepared copy).
  const bool kivi = !fp32 && !sel && kivi_fast_path_ok(L);
  const bool kivi_fold = kivi && (long)plan.splits * L.num_kv_heads * B < 256;
  const bool q_direct = kivi_fold && q_dtype == KV_DT_F32;
  if (L.format == KV_FMT_TURBO) {
    if (q_dtype == KV_DT_F32)
      prep_turbo_kernel<float><<<rows, kTurboPrepThreads, 0, st>>>(static_cast<const float*>(q), rot_arg(c), c->proj,
                                                                   c->lm_levels, scale * kLog2e, kappa, qv, qpieces);
    else
      prep_turbo_kernel<uint16_t><<<rows, kTurboPrepThreads, 0, st>>>(
          static_cast<const uint16_t*>(q), rot_arg(c), c->proj, c->lm_levels, scale * kLog2e, kappa, qv, qpieces);
  } else if (!(mfma && L.format == KV_FMT_FP4) && !q_direct) {
    if (q_dtype == KV_DT_F32)
      prep_query_kernel<float><<<rows, 128, 0, st>>>(static_cast<const float*>(q), qw_in, qw_out, L.format, c->proj,
                                                     qv, qpieces);
    else
      prep_query_kernel<uint16_t><<<rows, 128, 0, st>>>(static_cast<const uint16_t*>(q), qw_in, qw_out, L.format,
                                                        c->proj, qv, qpieces);
  }
  if (turbo) {
    TurboDecodeArgs f{};
    f.k_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_K_CODES]);
    f.k_sketch = static_cast<const uint8_t*>(c->buf[KV_BUF_K_SKETCH]);
    f.k_norm = static_cast<const uint16_t*>(c->buf[KV_BUF_K_NORM]);
    f.k_rnorm = static_cast<const uint16_t*>(c->buf[KV_BUF_K_RNORM]);
    f.v_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_V_CODES]);
    f.v_norm = static_cast<const uint16_t*>(c->buf[KV_BUF_V_NORM]);
    f.levels = c->lm_levels;
    f.pm = page_map(c);
    f.sel = sel;
    f.sel_stride = sel_stride;
    f.qpieces = qpieces;
    f.seq_lens = seq_lens;
    f.max_len = max_seq_len;
    f.H = L.num_kv_heads;
    f.cap = L.capacity;
    f.Hq = num_q_heads;
    f.part = part;
    f.splits = plan.splits;
    f.per_split = plan.tokens_per_split;
    f.nq = nq;
    f.gr = num_q_heads / L.num_kv_heads;
    f.t_lo = L.sink_tokens;
    f.recent = L.recent_tokens;
    f.part_splits = part_splits;
    if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return KV_EDEVICE;
    // one launch per 16 (query, head) pairs of a KV head, each over the whole
    // cache: a sequence's queries share the tiles
    for (f.c0 = 0; f.c0 < nq * f.gr; f.c0 += 16) {
      f.ncol = std::min(16, nq * f.gr - f.c0);
      int rc = launch_decode_turbo(f, B, st);
      if (rc != KV_OK) return rc;
    }
    if (windowed) launch_window(c, q, q_dtype, num_q_heads, nq, seq_lens, max_seq_len, scale, part, part_splits,
                                plan.splits, st);
    if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), st) != hipSuccess) return KV_EDEVICE;
    launch_merge(part, rows, part_splits, plan.splits, L.head_dim, L.format, rot_arg(c), out, st);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
  }
  if (mfma) {
    MfmaDecodeArgs f{};
    f.k_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_K_CODES]);
    f.k_scale = static_cast<const uint16_t*>(c->buf[KV_BUF_K_SCALE]);
    f.k_sketch = static_cast<const uint8_t*>(c->buf[KV_BUF_K_SKETCH]);
    f.k_norm = static_cast<const uint16_t*>(c->buf[KV_BUF_K_NORM]);
    f.v_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_V_CODES]);
    f.v_scale = static_cast<const uint16_t*>(c->buf[KV_BUF_V_SCALE]);
    f.pm = page_map(c);
    f.sel = sel;
    f.sel_stride = sel_stride;
    f.q = L.format == KV_FMT_FP4 ? q : static_cast<const void*>(qv);
    f.qpieces = qpieces;
    f.seq_lens = seq_lens;
    f.max_len = max_seq_len;
    f.H = L.num_kv_heads;
    f.cap = L.capacity;
    f.Hq = num_q_heads;
    f.scale_log2 = scale * kLog2e;
    f.kappa = (float)(1.2533141373155002512 / (double)(L.qjl_m > 0 ? L.qjl_m : 1));
    f.part = part;
    f.splits = plan.splits;
    f.per_split = plan.tokens_per_split;
    f.nq = nq;
    f.gr = num_q_heads / L.num_kv_heads;
    f.t_lo = L.sink_tokens;
    f.recent = L.recent_tokens;
    f.part_splits = part_splits;
    if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return KV_EDEVICE;
    // one launch per 32 (FP4: two blocks of 16 columns sharing the dequantised
    // tiles) or 16 (query, head) pairs of a KV head, each over the whole cache
    const int per_launch = L.format == KV_FMT_FP4 ? 32 : 16;
    for (f.c0 = 0; f.c0 < nq * f.gr; f.c0 += per_launch) {
      f.ncol = std::min(per_launch, nq * f.gr - f.c0);
      int rc = launch_decode_mfma(f, L.format, B, mfma_columns(f.ncol), st);
      if (rc != KV_OK) return rc;
    }
    if (windowed) launch_window(c, q, q_dtype, num_q_heads, nq, seq_lens, max_seq_len, scale, part, part_splits,
                                plan.splits, st);
    if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), st) != hipSuccess) return KV_EDEVICE;
    launch_merge(part, rows, part_splits, plan.splits, L.head_dim, L.format, rot_arg(c), out, st);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
  }

  DecodeArgs a = general_args(c, num_q_heads, nq, seq_lens, max_seq_len, scale, qv, part, plan, part_splits,
                               sel, sel_stride);
  if (kivi) {
    MfmaDecodeArgs f{};
    f.k_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_K_CODES]);
    f.v_codes = static_cast<const uint8_t*>(c->buf[KV_BUF_V_CODES]);
    f.k_scale_f = static_cast<const float*>(c->buf[KV_BUF_K_SCALE]);
    f.k_zero_f = static_cast<const float*>(c->buf[KV_BUF_K_ZERO]);
    f.v_scale_f = static_cast<const float*>(c->buf[KV_BUF_V_SCALE]);
    f.v_zero_f = static_cast<const float*>(c->buf[KV_BUF_V_ZERO]);
    f.k_stage = static_cast<const float*>(c->buf[KV_BUF_K_STAGE]);
    f.pm = page_map(c);
    f.q = q_direct ? q : qv;
    f.seq_lens = seq_lens;
    f.max_len = max_seq_len;
    f.H = L.num_kv_heads;
    f.cap = L.capacity;
    f.Hq = num_q_heads;
    f.scale_log2 = scale * kLog2e;
    f.part = part;
    f.splits = plan.splits;
    f.per_split = plan.tokens_per_split;
    f.nq = nq;
    f.gr = num_q_heads / L.num_kv_heads;
    f.part_splits = part_splits;
    if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return KV_EDEVICE;
    // one launch per 16 (query, head) pairs of a KV head, each over the whole cache
    for (f.c0 = 0; f.c0 < nq * f.gr; f.c0 += 16) {
      f.ncol = std::min(16, nq * f.gr - f.c0);
      int rc = launch_decode_kivi(f, L.head_dim, kivi_fold, B, st);
      if (rc != KV_OK) return rc;
    }
    if (!kivi_fold) launch_kivi_tail(a, tail_split, B, st);
    if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), st) != hipSuccess) return KV_EDEVICE;
    launch_merge(part, rows, part_splits, plan.splits, L.head_dim, L.format, rot_arg(c), out, st);
    return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
  }

  // KIVI2: the staged tokens' workgroups follow the splits' in the same launch
  a.tail_split = tail_split;
  if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), st) != hipSuccess) return KV_EDEVICE;
  switch (L.format) {
    case KV_FMT_KIVI2:
      if (L.head_dim == 64) launch_split<KV_FMT_KIVI2, 64, 64, 16>(a, B, st);
      else launch_split<KV_FMT_KIVI2, 128, 128, 16>(a, B, st);
      break;
    case KV_FMT_FP4:
      if (L.head_dim == 64) launch_split<KV_FMT_FP4, 64, 64, 16>(a, B, st);
      else launch_split<KV_FMT_FP4, 128, 128, 16>(a, B, st);
      break;
    case KV_FMT_TURBO: launch_split<KV_FMT_TURBO, 256, 128, 16>(a, B, st); break;
    case KV_FMT_QJL1_FP4V: launch_split<KV_FMT_QJL1_FP4V, 128, 128, 16>(a, B, st); break;
    case KV_FMT_LATENT_FP4: launch_split<KV_FMT_LATENT_FP4, 576, 512, 16>(a, B, st); break;
    default: return KV_EUNSUPPORTED;
  }
  if (windowed) launch_window(c, q, q_dtype, num_q_heads, nq, seq_lens, max_seq_len, scale, part, part_splits,
                              plan.splits, st);
  if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), st) != hipSuccess) return KV_EDEVICE;
  launch_merge(part, rows, part_splits, plan.splits, L.head_dim, L.format, rot_arg(c), out, st);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}

}  // namespace kvq
