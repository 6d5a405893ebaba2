// Decode attention on the matrix cores over a shared latent cache: every query
// head attends to one 512-channel latent per token (FP4 E2M1, one bf16 scale per
// 16 channels) plus a 64-channel bf16 RoPE key; the value is the latent itself
// (page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2", CSA2
// section: one 512-channel latent shared by the heads, with a 64-channel RoPE
// part).
//
// With 128 query heads on one latent the per-token work is a dense contraction
// (2 x 128 x (576 + 512) flop per 448 packed bytes), far past the HBM ridge, so
// the whole tile math runs on v_mfma_f32_32x32x16_{f16,bf16}.
//
// One workgroup = one (sequence, context split), 4 waves, one per SIMD.  Wave w
// owns heads [32 w, 32 w + 32) (Hq = 32 or 64: the waves past the heads repeat
// the last head group's work and write nothing): its query operand (144 registers) and its 32 x 512 fp32
// output accumulators (256 registers) stay in registers for the whole split.
// Every wave reads the whole dequantised tile from LDS, so the fewer, wider waves
// keep the LDS instructions per tile (next to the matrix cores, the binding
// resource) at half those of sixteen-head waves.
//
// The packed tiles come into registers by plain buffer loads, two tiles ahead
// (each thread its 1/256 of the tile), and are dequantised from there into one
// of three token-major fp16 tiles in LDS.  A wave issues in order, and its
// vector and LDS work runs beside a matrix product only when issued after it,
// so each tile's work is split in two phases of fenced groups, each group one
// product followed by the vector work that hides behind it:
//   1. S^T = K Q^T on tile i (36 products), with the dequantisation of tile
//      i + 1 and then the loads of tile i + 2;
//   2. O += P V for tile i - 1 (32 products, V read transposed with
//      ds_read_b64_tr_b16), with the online softmax of tile i (each lane pair
//      holds one head; the reference max moves only when a tile max passes it
//      by 2^8, and the accumulators are rescaled before the products of the
//      next tile).
// One workgroup barrier per tile.
// FP4 element values times their bf16 scale are exact in fp16 (within its range);
// the bf16 query's latent part is exact in fp16 within the fp16 normal range.
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_kernels.h"

namespace kvq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4_t* lds_s4_ptr;

constexpr int kNT = 256;  // threads per workgroup: 4 waves
constexpr int kTile = 32;
constexpr int kLat = 512, kRope = 64;
constexpr int kBufs = 3;  // dequantised tiles in LDS
// Kt: 32 token rows of 576 halves (fp16 latent, then bf16 RoPE), row stride
// 73 x 16 bytes, so that row r starts at bank word 36 r mod 64 (distinct
// 16-byte bank groups for the 16 rows of a half).  Token t = 16 c + 8 h +
// 4 h2 + e (e < 4) lives in row kt_phys(t) = 16 c + 4 e + 2 h + h2: the four
// tokens e = 0..3 that a transposing PV read takes sit in rows whose starts
// are 16 bank words apart, so the read's 32-byte pieces fill all 64 banks;
// the key reads and the dequantised writes touch sixteen rows of one half at
// a time, which any arrangement of the half keeps apart.
constexpr int kKtStride = kLat + kRope + 8;
constexpr int kKtHalves = kTile * kKtStride;
constexpr int kRsrcFlags = 0x00020000;

__host__ __device__ constexpr int kt_phys(int t) { return (t & 16) | ((t & 3) << 2) | ((t >> 2) & 3); }

// rows between tokens t and t + 4 (h2), t and t + 16 (c)
constexpr int kRowH2 = 1, kRowC = 16;
__host__ __device__ constexpr bool kt_phys_steps_hold() {
  for (int t = 0; t < 32; ++t) {
    if (!(t & 4) && kt_phys(t + 4) != kt_phys(t) + kRowH2) return false;
    if (t < 16 && kt_phys(t + 16) != kt_phys(t) + kRowC) return false;
  }
  return true;
}
static_assert(kt_phys_steps_hold(), "token row steps");

// Row rho of the QK A operand holds token qk_token(rho) (bits 2 and 3 of rho
// swapped): then the result rows a lane holds (i % 4 + 8 (i / 4) + 4 (lane / 32),
// i = 0..15) are the tokens 16 (i / 8) + 8 (lane / 32) + i % 8, exactly the
// k-slots that lane supplies as the A operand of the two 16-token PV products.
__host__ __device__ constexpr int qk_token(int rho) { return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

template <int SEL>
__device__ __forceinline__ h2_t fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ h2_t splat_bf16(uint32_t s) {
  const float f = __uint_as_float(s << 16);
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(f, f));
}

__device__ __forceinline__ uint32_t bf16x2_to_h2(uint32_t lo_hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(lo_hi << 16),
                                                                __uint_as_float(lo_hi & 0xFFFF0000u)));
}

// Transposing LDS read: within each 16-lane group, lane i gets element i % 4 of
// the 8-byte chunks addressed by lanes 4 e + i / 4, e = 0..3.
__device__ __forceinline__ s4_t read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(p));
}

// o *= f for one accumulator held in an AGPR, without the compiler staging the
// whole accumulator array through arch VGPRs.
__device__ __forceinline__ void scale_acc(float& x, float f) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(t)
               : "v"(f));
}

struct Res {
  __amdgpu_buffer_rsrc_t codes, scale, rope;
};

// This thread's share of one packed tile: code chunks of 16 bytes (32 channels
// of one token), their two bf16 scales (4 bytes), and one 16-byte chunk of the
// RoPE rows (chunk r is token r % 32, channels 8 (r / 32) + [0, 8)).  Code chunk
// j of thread tid is token chunk_token(tid, j), channels 32 (tid / 16) + [0, 32):
// sixteen consecutive lanes take sixteen tokens, whose fp16 rows start in
// distinct LDS banks, so that their dequantised writes do not conflict.
// RoPE chunk r = tid.
struct Packed {
  v4i_t c[2];
  int s[2];
  v4i_t r;
};

__device__ __forceinline__ int chunk_token(int tid, int j) { return 16 * j + (tid & 15); }

// Load P of this thread's share of a tile whose token k (of 32) sits at token
// offset tok(k) of the resources (tok < 0, or past the end of a resource:
// zeros): P = 2 j is code chunk j, P = 2 j + 1 its scales, P = 4 the RoPE chunk.
template <int P, class TokOf>
__device__ __forceinline__ void load_part(Packed& p, int tid, const Res& res, TokOf tok) {
  if constexpr (P == 4) {
    const int tr = tok(tid & 31);
    const uint32_t orp = tr < 0 ? 0xFFFFFFFFu : (uint32_t)tr * 128u + (tid >> 5) * 16;
    p.r = __builtin_amdgcn_raw_buffer_load_b128(res.rope, orp, 0, 0);
  } else {
    constexpr int j = P / 2;
    const int t = tok(chunk_token(tid, j)), cc = tid >> 4;
    if constexpr (P % 2 == 0) {
      const uint32_t oc = t < 0 ? 0xFFFFFFFFu : (uint32_t)t * 256u + cc * 16;
      p.c[j] = __builtin_amdgcn_raw_buffer_load_b128(res.codes, oc, 0, 0);
    } else {
      const uint32_t os = t < 0 ? 0xFFFFFFFFu : (uint32_t)t * 64u + cc * 4;
      p.s[j] = __builtin_amdgcn_raw_buffer_load_b32(res.scale, os, 0, 0);
    }
  }
}

// Dequantisation of this thread's share of a tile into the token-major fp16
// tile kt, in nine units: unit u < 8 is octet u % 4 (8 channels) of code chunk
// u / 4, unit 8 the RoPE chunk.  A unit runs in three stages (convert, scale,
// store), each in a later group than the one before it, so that no stage waits
// on a result of its own group; stage 0 of a chunk's first unit also makes the
// chunk's two scales into fp16 pairs.
struct DequantState {
  h2_t sc[2][2];   // the chunks' scales as fp16 pairs
  h2_t v[9][4];    // unit values: converted, then scaled
};

template <int U, int STAGE>
__device__ __forceinline__ void dequant_stage(const Packed& p, uint16_t* kt, int tid, DequantState& d) {
  if constexpr (U == 8) {
    if constexpr (STAGE == 2)
      *reinterpret_cast<v4i_t*>(kt + kt_phys(tid & 31) * kKtStride + kLat + 8 * (tid >> 5)) = p.r;
  } else {
    constexpr int j = U / 4, q = U % 4;  // octet q: channels 32 cc + 8 q + [0, 8), scale group 2 cc + q / 2
    if constexpr (STAGE == 0) {
      if constexpr (q == 0) {
        const uint32_t sw = (uint32_t)p.s[j];
        d.sc[j][0] = splat_bf16(sw & 0xFFFFu);
        d.sc[j][1] = splat_bf16(sw >> 16);
      }
      const uint32_t w = (uint32_t)p.c[j][q];
      d.v[U][0] = fp4x2<0>(w);
      d.v[U][1] = fp4x2<1>(w);
      d.v[U][2] = fp4x2<2>(w);
      d.v[U][3] = fp4x2<3>(w);
    } else if constexpr (STAGE == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) d.v[U][e] = d.v[U][e] * d.sc[j][q >> 1];
    } else {
      const int t = chunk_token(tid, j), cc = tid >> 4;
      *reinterpret_cast<uint4*>(kt + kt_phys(t) * kKtStride + 32 * cc + 8 * q) =
          uint4{__builtin_bit_cast(uint32_t, d.v[U][0]), __builtin_bit_cast(uint32_t, d.v[U][1]),
                __builtin_bit_cast(uint32_t, d.v[U][2]), __builtin_bit_cast(uint32_t, d.v[U][3])};
    }
  }
}

// f(integral_constant<int, K>) for K in the sequence, in order.
template <typename F, int... K>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, K...>, F&& f) {
  (f(std::integral_constant<int, K>{}), ...);
}

// The whole dequantisation of this thread's share, unscheduled (first tile).
__device__ __forceinline__ void dequant_tile(const Packed& p, uint16_t* kt, int tid) {
  DequantState d;
  for_each_index(std::make_integer_sequence<int, 9>{}, [&](auto U) {
    constexpr int u = decltype(U)::value;
    dequant_stage<u, 0>(p, kt, tid, d);
    dequant_stage<u, 1>(p, kt, tid, d);
    dequant_stage<u, 2>(p, kt, tid, d);
  });
}

// Per-wave state that lives across tiles.
struct LatentWave {
  h8_t ql[32];   // query, latent part (fp16): B operand of 32 k-steps
  b8_t qr[4];    // query, RoPE part (bf16): 4 k-steps
  f16v_t o[16];  // output accumulators, N block n = channels 32 n + [0, 32)
  float m_run;   // running reference max (log2 units) of this lane's head
  float l_run;   // running sum over this lane's tokens (the lane pair is added at the end)
};

// Phase 1 of a tile: S^T = K Q^T for this wave's 32 heads on tile kt (one
// accumulation chain in VGPRs, so that the output accumulators keep every
// AGPR; operand reads D products ahead), with this thread's
// dequantisation of the next tile into kt_next (unit u behind products 3 u + 1
// to 3 u + 3)
// and, each once its registers are free, the five loads of the tile after it
// (refill(pk, P) issues load P).
template <int D, class Refill>
__device__ __forceinline__ f16v_t qk_phase(const LatentWave& w, const uint16_t* kt, int ka, Packed& pk,
                                           uint16_t* kt_next, int tid, Refill refill) {
  h8_t kf[36];
  DequantState dq;
  f16v_t s = f16v_t{};
  auto read = [&](int k) { kf[k] = *reinterpret_cast<const h8_t*>(kt + ka + 16 * k); };
#pragma unroll
  for (int k = 0; k < D; ++k) read(k);
  __builtin_amdgcn_sched_barrier(0);
  for_each_index(std::make_integer_sequence<int, 36>{}, [&](auto K) {
    constexpr int k = decltype(K)::value;
    if constexpr (k + D < 36) read(k + D);
    if constexpr (k == 0)
      asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(s) : "v"(kf[0]), "v"(w.ql[0]));
    else if constexpr (k < 32)
      asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(s) : "v"(kf[k]), "v"(w.ql[k]));
    else
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(kf[k]), "v"(w.qr[k - 32]));
    // unit u: convert behind product 3 u + 1, scale behind 3 u + 2, store behind 3 u + 3
    if constexpr (k >= 1 && (k - 1) / 3 < 9) dequant_stage<(k - 1) / 3, (k - 1) % 3>(pk, kt_next, tid, dq);
    // each load once the units before it have consumed its registers
    if constexpr (k == 12) refill(pk, std::integral_constant<int, 0>{});
    if constexpr (k == 14) refill(pk, std::integral_constant<int, 1>{});
    if constexpr (k == 24) refill(pk, std::integral_constant<int, 2>{});
    if constexpr (k == 27) refill(pk, std::integral_constant<int, 3>{});
    if constexpr (k == 29) refill(pk, std::integral_constant<int, 4>{});
    __builtin_amdgcn_sched_barrier(0);
  });
  // the logits are read by vector instructions next: the last product's result
  // needs its wait states (the assembler statements are opaque to the compiler)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
  return s;
}

// max of three floats (the logits come from matrix products written in
// assembler statements, so the compiler cannot prove them canonical and would
// add a canonicalising max per operand to fmaxf)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Softmax of one tile's logits s (this lane: head col, tokens 16 (i / 8) +
// 8 half + i % 8; masked tokens hold -inf), spread over the 32 groups of a
// product phase: group g runs softmax_part<g>.  Makes the tile's probabilities
// (fp16, the A operand of the two PV products of the tile), adds their sum to
// l_run and leaves in alpha the factor the accumulators must be scaled by
// before the tile's products (1 unless the reference max moved).  A wave
// issues in order, so each group's vector work depends only on results of
// earlier groups: the max is a tree over groups 2..8, and logit pair m is
// scaled in group 12 + m, exponentiated in 13 + m and packed and summed in
// 14 + m.
struct SoftmaxState {
  float mx[7];      // partial maxima of the raw logits
  float sw[2];      // the two halves' maxima after the lane-pair swap
  float tmax, m_new, arg, m_use, alpha, psum;
  bool bump;
  float x[8][2], p[8][2];
};

template <int G>
__device__ __forceinline__ void softmax_part(LatentWave& w, SoftmaxState& st, const f16v_t& s, float c,
                                             h8_t (&pn)[2]) {
  // the max of the 16 raw logits (c > 0 keeps the order), then of the lane pair
  if constexpr (G == 2) { st.mx[0] = max3(s[0], s[1], s[2]); st.mx[1] = max3(s[3], s[4], s[5]); }
  if constexpr (G == 3) { st.mx[2] = max3(s[6], s[7], s[8]); st.mx[3] = max3(s[9], s[10], s[11]); }
  if constexpr (G == 4) { st.mx[4] = max3(s[12], s[13], s[14]); st.mx[5] = max3(st.mx[0], st.mx[1], s[15]); }
  if constexpr (G == 5) st.mx[6] = max3(st.mx[2], st.mx[3], st.mx[4]);
  if constexpr (G == 6) st.mx[0] = fmaxf(st.mx[5], st.mx[6]);
  if constexpr (G == 7) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.mx[0]), __float_as_uint(st.mx[0]), false, false);
    st.sw[0] = __uint_as_float(r[0]);
    st.sw[1] = __uint_as_float(r[1]);
  }
  if constexpr (G == 8) st.tmax = fmaxf(st.sw[0], st.sw[1]) * c;
  if constexpr (G == 9) {
    st.bump = st.tmax > w.m_run + 8.f;
    st.m_new = st.bump ? st.tmax : w.m_run;
  }
  if constexpr (G == 10) {
    st.arg = w.m_run - st.m_new;
    st.m_use = st.m_new == -INFINITY ? 0.f : st.m_new;  // a head with no token yet: every p is 0
    w.m_run = st.m_new;
  }
  if constexpr (G == 11) st.alpha = __builtin_amdgcn_exp2f(st.arg);
  if constexpr (G >= 12 && G < 20) {
    constexpr int m = G - 12;
    st.x[m][0] = __builtin_fmaf(s[2 * m], c, -st.m_use);
    st.x[m][1] = __builtin_fmaf(s[2 * m + 1], c, -st.m_use);
  }
  if constexpr (G >= 13 && G < 21) {
    constexpr int m = G - 13;
    st.p[m][0] = __builtin_amdgcn_exp2f(st.x[m][0]);
    st.p[m][1] = __builtin_amdgcn_exp2f(st.x[m][1]);
  }
  if constexpr (G == 13) st.alpha = st.bump ? st.alpha : 1.f;
  if constexpr (G >= 14 && G < 22) {
    constexpr int m = G - 14, i = 2 * m;
    const float ps = st.p[m][0] + st.p[m][1];
    st.psum = m == 0 ? ps : st.psum + ps;
    const h2_t pp = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(st.p[m][0], st.p[m][1]));
    pn[i >> 3][i & 7] = pp[0];
    pn[i >> 3][(i & 7) + 1] = pp[1];
  }
  if constexpr (G == 22) w.l_run = w.l_run * st.alpha + st.psum;
}

// Phase 2 of a tile: O += P V for the previous tile (if PV; its probabilities
// pf, its fp16 copy kt): product (n, c) takes channels 32 n + [0, 32) over
// tokens 16 c + [0, 16), its B operand two transposing reads of four tokens
// each, issued E products ahead; with the softmax of this tile's logits s (if
// SM).  Returns the factor the accumulators must be scaled by before this
// tile's products.
template <bool PV, bool SM, int E>
__device__ __forceinline__ float pv_phase(LatentWave& w, const h8_t (&pf)[2], const uint16_t* kt, int vb,
                                          const f16v_t& s, float c, h8_t (&pn)[2]) {
  constexpr int kH2 = kRowH2 * kKtStride;  // h2 = 1: token + 4
  constexpr int kC = kRowC * kKtStride;    // c = 1: token + 16
  s4_t vf[32][2];
  SoftmaxState st;
  auto vread = [&](int j) {
    const int n = j >> 1, cc = j & 1;
    vf[j][0] = read_tr16(kt + vb + cc * kC + 32 * n);
    vf[j][1] = read_tr16(kt + vb + cc * kC + kH2 + 32 * n);
  };
  if constexpr (PV) {
#pragma unroll
    for (int j = 0; j < E; ++j) vread(j);
  }
  __builtin_amdgcn_sched_barrier(0);
  for_each_index(std::make_integer_sequence<int, 32>{}, [&](auto J) {
    constexpr int j = decltype(J)::value;
    if constexpr (PV) {
      if constexpr (j + E < 32) vread(j + E);
      const h8_t v = __builtin_bit_cast(h8_t, __builtin_shufflevector(vf[j][0], vf[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
      w.o[j >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pf[j & 1], v, w.o[j >> 1], 0, 0, 0);
    }
    if constexpr (SM) softmax_part<j>(w, st, s, c, pn);
    __builtin_amdgcn_sched_barrier(0);
  });
  return SM ? st.alpha : 1.f;
}

// The logits of tile tokens not below t_end or (sparse) without their bit in
// `valid` become -inf (this lane: tokens 16 (i / 8) + 8 half + i % 8).
__device__ __forceinline__ void mask_tile(f16v_t& s, int half, int tt, int t_end, uint32_t valid) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = 16 * (i >> 3) + 8 * half + (i & 7);
    if (!(tt + j < t_end && ((valid >> j) & 1u))) s[i] = -INFINITY;
  }
}

// O *= alpha per head (output rows are heads i % 4 + 8 (i / 4) + 4 half; head
// r's alpha is in lane r), when any head's reference max moved.  The reads
// start at least 48 wait states after the last product that wrote them (more
// than a 32x32x16 product's latency).
__device__ __forceinline__ void rescale(LatentWave& w, float alpha, int half) {
  if (__ballot(alpha != 1.f)) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float ar = __shfl(alpha, (i & 3) + 8 * (i >> 2) + 4 * half);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        float x = w.o[n][i];
        scale_acc(x, ar);
        w.o[n][i] = x;
      }
    }
    asm volatile("s_nop 7");  // VALU writes of the accumulators, then MFMA reads of them
  }
}

// PAGED: token rows in pool pages named by the block table, resources per tile.
// SPARSE (contiguous caches): the split's slots read the positions a.sel names,
// staged in LDS; slots without a valid position are masked.
template <bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_latent_kernel(MfmaDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Kt[kBufs][kKtHalves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves past the heads (Hq = 32 or 64) compute on the last head group's query
  // (so that every wave runs the same code) and write nothing
  const bool heads = 32 * wave < a.Hq;
  const int hgroup = heads ? wave : a.Hq / 32 - 1;
  const int split = blockIdx.x, b = blockIdx.y;
  // several queries per sequence: this launch takes query j = a.c0 of a.nq,
  // which sees the first L - (nq - 1 - j) tokens
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap) - (a.nq - 1 - a.c0);
  const size_t qrow0 = ((size_t)b * a.nq + a.c0) * a.Hq;  // its first query / output row
  const int t_begin = split * a.per_split;
  const int t_end = min(L, t_begin + a.per_split);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;
  const int col = lane & 31, half = lane >> 5;  // head of this lane's column, its lane half
  static_assert(!(PAGED && SPARSE), "sparse decode reads contiguous caches");
  __shared__ int spos[SPARSE ? kLatentSparseSlots : 1];
  __shared__ uint32_t svalid[SPARSE ? kLatentSparseSlots / kTile : 1];  // bit j: slot j of the tile is valid
  if constexpr (SPARSE) {
    const int32_t* sb = a.sel + (size_t)b * a.sel_stride;
    for (int i = tid; i < a.per_split; i += kNT) {
      const int slot = t_begin + i;
      int p = slot < t_end ? sb[slot] : -1;
      spos[i] = p >= 0 && p < a.cap ? p : -1;
    }
    __syncthreads();
    for (int ti = tid; ti < a.per_split / kTile; ti += kNT) {
      uint32_t m = 0;
      for (int j = 0; j < kTile; ++j) m |= (spos[ti * kTile + j] >= 0 ? 1u : 0u) << j;
      svalid[ti] = m;
    }
    __syncthreads();
  }

  // resources over nrows token rows from row0 (nrows 0: every read is zeros)
  auto res_at = [&](size_t row0, int nrows) {
    return Res{rsrc(a.k_codes + row0 * 256, (size_t)nrows * 256), rsrc(a.k_scale + row0 * 32, (size_t)nrows * 64),
               rsrc(a.rope + row0 * 64, (size_t)nrows * 128)};
  };
  const Res res = res_at((size_t)b * a.cap, a.cap);
  // where tile index ti (tokens t_begin + 32 ti + [0, 32)) is read from: its
  // resources and first token offset (sparse: its first slot); a missing tile
  // or token reads past the end of its resources: zeros
  struct TileSrc {
    Res res;
    int t0;
  };
  auto tile_src = [&](int ti) -> TileSrc {
    const int t = t_begin + ti * kTile;
    if constexpr (SPARSE) {
      return TileSrc{res, t < t_end ? t - t_begin : -1};
    } else if constexpr (!PAGED) {
      return TileSrc{res, t < t_end ? t : a.cap};
    } else {
      const int pg = t < t_end ? page_of_uniform(a.pm, b, t) : -1;
      return TileSrc{res_at((size_t)(pg < 0 ? 0 : pg) * a.pm.tokens, pg < 0 ? 0 : a.pm.tokens),
                     pg < 0 ? 0 : t & (a.pm.tokens - 1)};
    }
  };
  // load P of the tile src names
  auto load_from = [&](Packed& p, const TileSrc& src, auto P) {
    constexpr int part = decltype(P)::value;
    if constexpr (SPARSE)
      load_part<part>(p, tid, src.res, [&](int k) { return src.t0 < 0 ? -1 : spos[src.t0 + k]; });
    else
      load_part<part>(p, tid, src.res, [&](int k) { return src.t0 + k; });
  };
  auto load_at = [&](Packed& p, int ti) {
    const TileSrc src = tile_src(ti);
    for_each_index(std::make_integer_sequence<int, 5>{}, [&](auto P) { load_from(p, src, P); });
  };
  auto refill_from = [&](const TileSrc& src) { return [&, src](Packed& p, auto P) { load_from(p, src, P); }; };
  Packed pk;  // this thread's share of the next tile to dequantise
  load_at(pk, 0);

  LatentWave w;
  // ---------------- the query operand: 32 fp16 latent steps, 4 bf16 RoPE steps
  // (B operand of the 32x32x16 products: head col, channels 16 k + 8 half + [0, 8))
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow0 + 32 * hgroup + col) * (kLat + kRope);
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * s + 8 * half);
      w.ql[s] = __builtin_bit_cast(h8_t, uint4{bf16x2_to_h2(raw.x), bf16x2_to_h2(raw.y), bf16x2_to_h2(raw.z),
                                               bf16x2_to_h2(raw.w)});
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      w.qr[s] = __builtin_bit_cast(b8_t, *reinterpret_cast<const uint4*>(qp + kLat + 16 * s + 8 * half));
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) w.o[n] = f16v_t{};
  w.m_run = -INFINITY;
  w.l_run = 0.f;

  // lane constants of the fragment reads (kept opaque so that the compiler does
  // not hoist one address register per read out of the loop)
  // this lane's QK A operand: token qk_token(col), channels 16 k + 8 half + [0, 8)
  int ka = kt_phys(qk_token(col)) * kKtStride + 8 * half;
  // this lane's transposing PV reads: lane (group G = lane / 16, j = lane % 16)
  // addresses channels 32 n + 16 (G % 2) + 4 (j % 4) + [0, 4) of token
  // 16 c + 8 half + 4 h2 + j / 4, so that it receives channel 32 n + col of
  // tokens 16 c + 8 half + 4 h2 + [0, 4): its PV B operand k-slots
  const int jj = lane & 15, gg = lane >> 4;
  int vb = kt_phys(8 * half + (jj >> 2)) * kKtStride + 16 * (gg & 1) + 4 * (jj & 3);
  asm volatile("" : "+v"(ka), "+v"(vb));

  // Tile i: its dequantised copy Kt[i % 3], written during tile i - 1.  Before
  // the products of tile i every wave has finished tile i - 1, whose phase 2
  // read Kt[(i - 2) % 3], the buffer tile i + 1 takes.
  const float c = a.scale_log2;
  h8_t pf[2];           // probabilities of the previous tile
  float alpha = 1.f;    // the accumulators' pending factor
  if (ntiles > 0) {
    dequant_tile(pk, Kt[0], tid);
    load_at(pk, 1);
    __syncthreads();
    f16v_t s = qk_phase<3>(w, Kt[0], ka, pk, Kt[1], tid, refill_from(tile_src(2)));
    if (kTile > t_end - t_begin || (SPARSE && svalid[0] != 0xFFFFFFFFu))
      mask_tile(s, half, t_begin, t_end, SPARSE ? svalid[0] : 0xFFFFFFFFu);
    alpha = pv_phase<false, true, 3>(w, pf, Kt[0], vb, s, c, pf);
  }
  int cur = 1;  // buffer of tile i
  for (int i = 1; i < ntiles; ++i) {
    __syncthreads();
    const int prv = cur == 0 ? kBufs - 1 : cur - 1, nxt = cur == kBufs - 1 ? 0 : cur + 1;
    const int tt = t_begin + i * kTile;
    const TileSrc src = tile_src(i + 2);
    f16v_t s = qk_phase<3>(w, Kt[cur], ka, pk, Kt[nxt], tid, refill_from(src));
    rescale(w, alpha, half);
    if (tt + kTile > t_end || (SPARSE && svalid[i] != 0xFFFFFFFFu))
      mask_tile(s, half, tt, t_end, SPARSE ? svalid[i] : 0xFFFFFFFFu);
    h8_t pn[2];
    alpha = pv_phase<true, true, 3>(w, pf, Kt[prv], vb, s, c, pn);
    pf[0] = pn[0];
    pf[1] = pn[1];
    cur = nxt;
  }
  if (ntiles > 0) {  // the last tile's products
    rescale(w, alpha, half);
    const int prv = cur == 0 ? kBufs - 1 : cur - 1;
    h8_t unused[2];
    pv_phase<true, false, 3>(w, pf, Kt[prv], vb, f16v_t{}, c, unused);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the refills past the last tile have returned

  // ---------------- partial result of this split
  if (!heads) return;
  const float l_run = w.l_run + __shfl_xor(w.l_run, 32);
  const size_t row0 = qrow0 + 32 * wave;
  if (half == 0) {
    float* p = a.part + ((row0 + col) * a.splits + split) * (kLat + 2);
    p[0] = w.m_run;
    p[1] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int head = (r & 3) + 8 * (r >> 2) + 4 * half;
    float* p = a.part + ((row0 + head) * a.splits + split) * (kLat + 2) + 2 + col;
#pragma unroll
    for (int n = 0; n < 16; ++n) p[32 * n] = w.o[n][r];
  }
}

template <bool PAGED, bool SPARSE>
int launch_latent(const MfmaDecodeArgs& a, int B, hipStream_t st) {
  if (a.Hq != 32 && a.Hq != 64 && a.Hq != 128) return KV_EUNSUPPORTED;
  decode_latent_kernel<PAGED, SPARSE><<<dim3(a.splits, B), kNT, 0, st>>>(a);
  return KV_OK;
}

}  // namespace

int launch_decode_latent(const MfmaDecodeArgs& a, int B, hipStream_t st) {
  if (a.sel) return a.pm.table ? KV_EUNSUPPORTED : launch_latent<false, true>(a, B, st);
  return a.pm.table ? launch_latent<true, false>(a, B, st) : launch_latent<false, false>(a, B, st);
}

}  // namespace kvq
