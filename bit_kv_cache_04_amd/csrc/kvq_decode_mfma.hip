// Decode attention on the matrix cores (gfx950) for caches whose values are FP4
// E2M1 with one bf16 scale per 16 channels: FP4 keys, or 1-bit QJL keys.
//
// One workgroup = 4 waves over one (sequence, KV head, context split); each
// wave streams its own 32-token tiles of packed codes from HBM into a private
// two-stage LDS ring with direct-to-LDS buffer loads (the next tile is in
// flight while the current one is computed, without holding registers), and
// keeps an online-softmax state for all query heads of the group.  Per tile
// and wave:
//   S^T = K_tile . Q^T   v_mfma_f32_16x16x32_f16 (rows = tokens, cols = heads)
//   online softmax       per head = per lane column; row max over the 4 lane quarters
//   O  += P . V_tile     8 v_mfma_f32_16x16x32_f16 (rows = heads, cols = channels)
// The group's query heads share every packed byte read (page "TurboQuant vs
// OSCAR vs EpiCache", KV-cache memory bottleneck section: decode is bound by
// streaming the cache), and scores never leave registers.
//
// FP4 element values: an E2M1 code times its bf16 group scale has at most 10
// significant bits, so it is exact in fp16 while |x| stays within the fp16
// range; products with the bf16 query (exact in fp16 in range) accumulate in
// fp32.  Softmax weights enter the PV product as fp16 (relative error 2^-11).
//
// QJL keys: the logit is sqrt(pi/2)/m * n * <S q, sigma> with sigma = +-1 from
// the sketch bits (page "TurboQuant vs OSCAR vs EpiCache", section
// "quantization frontiers", stage two).  <S q, sigma> = 2 <S q, b> - sum(S q)
// for the bits b; each bit enters the product as the fp16 value 1.0 or 0 and
// S q as an exact fp16 hi + lo pair, so the sum is exact up to fp32 rounding.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_kernels.h"

namespace kvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

namespace {

constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

template <int SEL>
__device__ __forceinline__ h2_t fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ h2_t bf16x2_to_h2(uint32_t lo_hi) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(lo_hi << 16),
                                                            __uint_as_float(lo_hi & 0xFFFF0000u)));
}

__device__ __forceinline__ h2_t splat_bf16(uint32_t s) {
  const float f = __uint_as_float(s << 16);
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(f, f));
}

__device__ __forceinline__ h8_t h8_from(h2_t a, h2_t b, h2_t c, h2_t d) {
  h8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 E2M1 codes (one dword) times one scale -> 8 fp16 (A-operand k-slots in order).
__device__ __forceinline__ h8_t dequant8(uint32_t w, h2_t s) {
  return h8_from(fp4x2<0>(w) * s, fp4x2<1>(w) * s, fp4x2<2>(w) * s, fp4x2<3>(w) * s);
}

// One bit per nibble of a 32-bit key word, as the FP4 operand of a scaled
// product: dword d holds bits d, d + 4, ..., d + 28 (element 8 d + n = bit 4 n + d).
__device__ __forceinline__ i8_t bit_nibbles(uint32_t w) {
  const uint32_t m = 0x11111111u;
  return i8_t{(int)(w & m), (int)((w >> 1) & m), (int)((w >> 2) & m), (int)((w >> 3) & m), 0, 0, 0, 0};
}

// v_mfma_scale_f32_16x16x128_f8f6f4: A = key bits (FP4, 0 or 0.5, block scale
// 2), B = FP8 pieces with their block scales.  A lane quarter's 32 elements
// form one k-block; B lane quarter qb holds k-blocks qb / 2 and 2 + qb / 2
// (elements 16 (qb % 2) .. + 15 of each) and the scale of k-block qb.
__device__ __forceinline__ f4_t key_product(i8_t a, i8_t b, int scale_b, f4_t acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 0, 0, 128, 0, scale_b);
}

// x of lane (l & ~15) | ((l + N) & 15), 0 < N < 16: DPP row_ror:(16 - N) (a
// rotation right by k hands lane l the value of lane l - k within its row).
template <int N>
__device__ __forceinline__ float row_fetch(float x) {
  static_assert(N > 0 && N < 16, "rotation within a 16-lane row");
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + (16 - N), 0xF, 0xF, false));
}

// A-operand row c of a 16-token block holds token 4*(c%4) + c/4, so that the
// C rows 4*q4 + v of a lane quarter are the tokens 4*v + q4.
__device__ __forceinline__ int row_token(int c) { return 4 * (c & 3) + (c >> 2); }

// ---------------------------------------------------------------- key policies

// FP4 keys: codes (64 B per token) and scales (16 B per token).
struct KeysFp4 {
  static constexpr int kBytes = 2560;  // codes 2048 | scales 512
  static constexpr int kDma = 4;       // direct-to-LDS loads issue() makes
  struct Q {
    h8_t f[4];  // lane (q4, c): head c, channels 32*q4 + 8*i + j for MFMA i
  };
  struct R {
    __amdgpu_buffer_rsrc_t kc, ks;
  };
  struct Frag {
    uint4 kw[2];
    uint32_t s2[2];
  };
  template <int G>
  __device__ static void load_q(Q& q, const MfmaDecodeArgs& a, int b, int h, int q4, int c, int col0) {
    // column col0 + c of the launch: pair c0 + col0 + c = query token j, head g
    // (columns from ncol on hold none)
    const int pc = a.c0 + col0 + c;
    const bool live = col0 + c < a.ncol;
    const int jq = live ? pc / a.gr : 0, head = live ? pc % a.gr : 0;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((size_t)b * a.nq + jq) * a.Hq + (size_t)h * a.gr + head) * 128 + 32 * q4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + 8 * i);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h2_t v = bf16x2_to_h2(wd[j]);
        q.f[i][2 * j] = live ? v[0] : (_Float16)0.f;
        q.f[i][2 * j + 1] = live ? v[1] : (_Float16)0.f;
      }
    }
  }
  // over nrows token rows from row0
  __device__ static R resources(const MfmaDecodeArgs& a, size_t row0, int nrows) {
    return R{rsrc(a.k_codes + row0 * 64, (size_t)nrows * 64), rsrc(a.k_scale + row0 * 8, (size_t)nrows * 16)};
  }
  __device__ static void issue(uint8_t* st, int lane, int t0, const R& r) {
    const int co = t0 * 64 + lane * 16, so = t0 * 16 + lane * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st), 16, co, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + 1024), 16, co + 1024, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ks, (lds_ptr_t)(st + 2048), 4, so, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ks, (lds_ptr_t)(st + 2304), 4, so + 256, 0, 0, 0);
  }
  // gather: the lane's rows of the two 16-token halves are pa and pb (-1: none,
  // reads zeros); the same stage layout as issue()
  __device__ static void issue_rows(uint8_t* st, int lane, int pa, int pb, int, const R& r) {
    const uint32_t ca = pa < 0 ? ~0u : (uint32_t)pa * 64u + (lane & 3) * 16, cb = pb < 0 ? ~0u : (uint32_t)pb * 64u + (lane & 3) * 16;
    const uint32_t sa = pa < 0 ? ~0u : (uint32_t)pa * 16u + (lane & 3) * 4, sb = pb < 0 ? ~0u : (uint32_t)pb * 16u + (lane & 3) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st), 16, ca, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + 1024), 16, cb, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ks, (lds_ptr_t)(st + 2048), 4, sa, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ks, (lds_ptr_t)(st + 2304), 4, sb, 0, 0, 0);
  }
  __device__ static void read(Frag& f, const uint8_t* st, int q4, int c) {
    int ko = row_token(c) * 64 + 16 * q4, kso = row_token(c) * 16 + 4 * q4;
    asm volatile("" : "+v"(ko), "+v"(kso));
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f.kw[blk] = *reinterpret_cast<const uint4*>(st + ko + 1024 * blk);
      f.s2[blk] = *reinterpret_cast<const uint32_t*>(st + kso + 2048 + 256 * blk);
    }
  }
  // raw logits of the lane's 8 (token, column) pairs per column block nb:
  // [nb][blk][v] for token 16 blk + 4 v + q4; the blocks share the dequantised keys
  template <int NB>
  __device__ static void logits(const Frag& f, const Q* q, f4_t (*sacc)[2]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const h2_t s_lo = splat_bf16(f.s2[blk] & 0xFFFFu), s_hi = splat_bf16(f.s2[blk] >> 16);
      const h8_t k0 = dequant8(f.kw[blk].x, s_lo), k1 = dequant8(f.kw[blk].y, s_lo);
      const h8_t k2 = dequant8(f.kw[blk].z, s_hi), k3 = dequant8(f.kw[blk].w, s_hi);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, q[nb].f[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, q[nb].f[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k2, q[nb].f[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k3, q[nb].f[3], acc, 0, 0, 0);
        sacc[nb][blk] = acc;
      }
    }
  }
};

// 1-bit QJL keys: 128 sketch bits (16 B per token) and the fp16 key norm.  The
// key product runs on the scaled FP4 x FP8 instruction: A = the token's sketch
// bits (lane quarter q4: sketch dword q4, one bit per nibble), B = FP8 pieces of
// S q (4 pieces, prepared once per decode).  Column c carries piece c / G of
// head c % G while pieces fit (16 / G of them per product), so 4 / (16 / G)
// products (1 for G <= 4) cover the 4 pieces, and rotations within each 16-lane
// row add a head's pieces onto its column.
struct KeysQjl {
  static constexpr int kBytes = 768;  // sketch 512 | norms, one per dword: 128 (+ 128 zeros)
  static constexpr int kDma = 3;      // direct-to-LDS loads issue() makes
  template <int G>
  static constexpr int kSlots = G >= 16 ? 1 : (G >= 8 ? 2 : 4);  // pieces per product
  struct Q {
    i8_t bq[4];  // B operands of up to 4 products
    int bs[4];   // their block scales
    float sumq;  // sum of the head's 128 projected-query values
  };
  struct R {
    __amdgpu_buffer_rsrc_t sk, nm;
    int nm_end;  // byte size of the norm resource: an offset that reads zeros
  };
  struct Frag {
    uint32_t w[2];   // sketch rows 32*q4 .. 32*q4 + 31 of token row_token(c)
    uint32_t n[8];   // fp16 norm bits of tokens 16 blk + 4 v + q4
  };
  template <int G>
  __device__ static void load_q(Q& q, const MfmaDecodeArgs& a, int b, int h, int q4, int c, int) {
    constexpr int NS = kSlots<G>, NP = 4 / NS;
    // column c holds piece slot c / G of pair c0 + c % G = query token j, head g
    const int slot = c / G, pair = a.c0 + c % G;
    const bool live = slot < NS && c % G < a.ncol;
    const size_t qrow =
        ((size_t)b * a.nq + (live ? pair / a.gr : 0)) * a.Hq + (size_t)h * a.gr + (live ? pair % a.gr : 0);
    const uint8_t* pc = a.qpieces + qrow * kQjlPieceBytes;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = i * NS + (live ? slot : 0);
      const uint8_t* base = pc + p * 144 + 16 * (q4 & 1);
      const uint4 lo4 = *reinterpret_cast<const uint4*>(base + 32 * (q4 >> 1));
      const uint4 hi4 = *reinterpret_cast<const uint4*>(base + 32 * (2 + (q4 >> 1)));
      q.bq[i] = live ? i8_t{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w, (int)hi4.x, (int)hi4.y, (int)hi4.z,
                            (int)hi4.w}
                     : i8_t{0, 0, 0, 0, 0, 0, 0, 0};
      q.bs[i] = live ? (int)pc[p * 144 + 128 + q4] : 127;
    }
    const float* qp = static_cast<const float*>(a.q) + qrow * 128 + 32 * q4;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 32; ++x) s += qp[x];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    q.sumq = s;
  }
  __device__ static R resources(const MfmaDecodeArgs& a, size_t row0, int nrows) {
    return R{rsrc(a.k_sketch + row0 * 16, (size_t)nrows * 16), rsrc(a.k_norm + row0, (size_t)nrows * 2), nrows * 2};
  }
  __device__ static void issue(uint8_t* st, int lane, int t0, const R& r) {
    const int so = t0 * 16 + lane * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st), 4, so, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st + 256), 4, so + 256, 0, 0, 0);
    // one 2-byte norm per lane for lanes 0..31 (a 2-byte load lands in its lane's
    // dword of LDS, zero-extended); lanes 32..63 read past the resource and write
    // zeros.  2-byte granules keep the range check exact: a dword holding the
    // last token of an odd capacity would straddle the end and read as zero.
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.nm, (lds_ptr_t)(st + 512), 2, lane < 32 ? t0 * 2 + lane * 2 : r.nm_end,
                                             0, 0, 0);
  }
  // gather: sketch rows pa, pb of the lane's two halves, norm row pn (lanes < 32)
  __device__ static void issue_rows(uint8_t* st, int lane, int pa, int pb, int pn, const R& r) {
    const uint32_t sa = pa < 0 ? ~0u : (uint32_t)pa * 16u + (lane & 3) * 4, sb = pb < 0 ? ~0u : (uint32_t)pb * 16u + (lane & 3) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st), 4, sa, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st + 256), 4, sb, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.nm, (lds_ptr_t)(st + 512), 2,
                                             lane < 32 && pn >= 0 ? (uint32_t)pn * 2u : (uint32_t)r.nm_end, 0, 0, 0);
  }
  __device__ static void read(Frag& f, const uint8_t* st, int q4, int c) {
    int so = row_token(c) * 16 + 4 * q4, no = 512 + 4 * q4;
    asm volatile("" : "+v"(so), "+v"(no));
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) f.w[blk] = *reinterpret_cast<const uint32_t*>(st + so + 256 * blk);
#pragma unroll
    for (int j = 0; j < 8; ++j) f.n[j] = *reinterpret_cast<const uint16_t*>(st + no + 16 * j);
  }
  template <int G>
  __device__ static void logits(const Frag& f, const Q& q, float kappa, f4_t sacc[2]) {
    constexpr int NS = kSlots<G>, NP = 4 / NS;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const i8_t A = bit_nibbles(f.w[blk]);
      f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NP; ++i) acc = key_product(A, q.bq[i], q.bs[i], acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = acc[v];
        if constexpr (NS >= 2) x += row_fetch<G>(x);      // + column c + G
        if constexpr (NS >= 4) x += row_fetch<2 * G>(x);  // + columns c + 2G, c + 3G
        const float n = f16_to_f32((uint16_t)f.n[4 * blk + v]);
        // x = <S q, b>: <S q, sigma> = 2 x - sum(S q)
        acc[v] = kappa * n * fmaf(2.f, x, -q.sumq);
      }
      sacc[blk] = acc;
    }
  }
};

// ---------------------------------------------------------------- the kernel

template <int G, int NB>
__device__ __forceinline__ void logits_of(const KeysFp4::Frag& f, const KeysFp4::Q* q, const MfmaDecodeArgs&,
                                          f4_t (*sacc)[2]) {
  KeysFp4::logits<NB>(f, q, sacc);
}
template <int G, int NB>
__device__ __forceinline__ void logits_of(const KeysQjl::Frag& f, const KeysQjl::Q* q, const MfmaDecodeArgs& a,
                                          f4_t (*sacc)[2]) {
  static_assert(NB == 1, "one column block for QJL keys");
  KeysQjl::logits<G>(f, q[0], a.kappa, sacc[0]);
}

// V region of a stage (after the keys): codes 2048 | scales 512.
template <class KP>
struct Stage {
  static constexpr int kVc = KP::kBytes, kVs = KP::kBytes + 2048, kBytes = KP::kBytes + 2560;
};

struct VRsrc {
  __amdgpu_buffer_rsrc_t vc, vs;
};

// Where the next tile's loads go: resources over the token rows of its page (a
// contiguous cache: the (sequence, KV head)'s rows) and its first row in them.
template <class KP>
struct TileSrc {
  typename KP::R kr;
  VRsrc vr;
  int t;
};

// Direct-to-LDS loads of one tile: lane i moves bytes [size*i, size*i + size) of
// each chunk.  The token offset travels in the bounds-checked VGPR offset, so a
// tile past the end of the resource (including the no-tile sentinel, t0 =
// capacity) reads zeros and touches no memory.
template <class KP>
__device__ __forceinline__ void issue_tile(uint8_t* st, int lane, int t0, const typename KP::R& kr,
                                           const VRsrc& vr) {
  KP::issue(st, lane, t0, kr);
  const int co = t0 * 64 + lane * 16, so = t0 * 16 + lane * 4;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vc, (lds_ptr_t)(st + Stage<KP>::kVc), 16, co, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vc, (lds_ptr_t)(st + Stage<KP>::kVc + 1024), 16, co + 1024, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vs, (lds_ptr_t)(st + Stage<KP>::kVs), 4, so, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vs, (lds_ptr_t)(st + Stage<KP>::kVs + 256), 4, so + 256, 0, 0, 0);
}

// Gather form of issue_tile: slot rel of the staged positions starts the tile
// (rel < 0: no tile).  Lane rows: slots lane / 4 and 16 + lane / 4 (codes, scales,
// sketch), slot lane (QJL norms); the number of loads is issue_tile's.
template <class KP>
__device__ __forceinline__ void issue_tile_rows(uint8_t* st, int lane, int rel, const int* pos,
                                                const typename KP::R& kr, const VRsrc& vr) {
  const int pa = rel < 0 ? -1 : pos[rel + (lane >> 2)];
  const int pb = rel < 0 ? -1 : pos[rel + 16 + (lane >> 2)];
  const int pn = rel < 0 ? -1 : pos[rel + (lane & 31)];
  KP::issue_rows(st, lane, pa, pb, pn, kr);
  const uint32_t ca = pa < 0 ? ~0u : (uint32_t)pa * 64u + (lane & 3) * 16, cb = pb < 0 ? ~0u : (uint32_t)pb * 64u + (lane & 3) * 16;
  const uint32_t sa = pa < 0 ? ~0u : (uint32_t)pa * 16u + (lane & 3) * 4, sb = pb < 0 ? ~0u : (uint32_t)pb * 16u + (lane & 3) * 4;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vc, (lds_ptr_t)(st + Stage<KP>::kVc), 16, ca, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vc, (lds_ptr_t)(st + Stage<KP>::kVc + 1024), 16, cb, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vs, (lds_ptr_t)(st + Stage<KP>::kVs), 4, sa, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr.vs, (lds_ptr_t)(st + Stage<KP>::kVs + 256), 4, sb, 0, 0, 0);
}

// Everything one wave carries across tiles, per block of 16 columns.
template <class KP, int NB>
struct WaveState {
  typename KP::Q q[NB];
  float m_run[NB], l_run[NB];
  f4_t o[NB][8];
};

// This lane's token limit per column block (its column's query sees the first
// L - (nq - 1 - j) tokens, capped by the split's end).
template <int NB>
struct Limits {
  int v[NB];
};

// One tile: read this lane's fragments from the stage, then (once the reads
// have returned) refill the stage from `nx` (a row past its resources when there
// is no next tile, so that the refill is unconditional and the compiler's wait
// counts stay exact), then compute.  Tokens below a.t_lo are masked.
// SP: gather mode, nx.t the next tile's first staged slot in pos; `valid` bit j:
// the tile's slot j holds a position.
template <int G, int NS, class KP, int NB, bool SP = false>
__device__ __forceinline__ void tile_step(WaveState<KP, NB>& w, uint8_t* st, int lane, int t0, int t_full,
                                          const Limits<NB>& lim, const TileSrc<KP>& nx, const MfmaDecodeArgs& a,
                                          const int* pos = nullptr, uint32_t valid = ~0u) {
  const int q4 = lane >> 4, c = lane & 15;
  // This stage's tile has landed once at most the other NS - 1 stages' refills
  // are outstanding.  Waited for explicitly: the compiler's own wait for loads
  // into LDS is not placed reliably across the loop back-edge.
  constexpr int kOther = (NS - 1) * (KP::kDma + 4);  // key loads + 4 value loads per stage
  static_assert(kOther < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kOther & 15) | ((kOther >> 4) << 14));
  typename KP::Frag kf;
  KP::read(kf, st, q4, c);
  // Lane byte offsets into the stage; opaque to the optimiser so that every read
  // below is one base register plus an immediate offset, instead of a hoisted
  // register per read.
  int vo = q4 * 64 + 4 * c, vso = q4 * 16 + 2 * (c >> 1);
  asm volatile("" : "+v"(vo), "+v"(vso));
  uint32_t dv[8], sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // the lane's token j is tile row 4j + q4
    dv[j] = *reinterpret_cast<const uint32_t*>(st + vo + Stage<KP>::kVc + 256 * j);
    sc[j] = *reinterpret_cast<const uint16_t*>(st + vso + Stage<KP>::kVs + 64 * j);
  }
  // the reads above must have returned before the stage is overwritten
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  if constexpr (SP) issue_tile_rows<KP>(st, lane, nx.t, pos, nx.kr, nx.vr);
  else issue_tile<KP>(st, lane, nx.t, nx.kr, nx.vr);

  // ---------------- logits: S^T = K Q^T for the two 16-token blocks
  f4_t sacc[NB][2];
  logits_of<G, NB>(kf, w.q, a, sacc);
  // ---------------- online softmax (this lane: column 16 nb + c, tokens t0 + 16*blk + 4*v + q4)
  h8_t pf[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float sv[8];
    float tmax = -INFINITY;
    if (t0 + 32 <= t_full && t0 >= a.t_lo && valid == ~0u) {  // a whole tile for every column: nothing to mask
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          sv[4 * blk + v] = sacc[nb][blk][v] * a.scale_log2;
          tmax = fmaxf(tmax, sv[4 * blk + v]);
        }
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tok = t0 + 16 * blk + 4 * v + q4;
          const bool in = tok < lim.v[nb] && tok >= a.t_lo && ((valid >> (tok - t0)) & 1u);
          const float sx = in ? sacc[nb][blk][v] * a.scale_log2 : -INFINITY;
          sv[4 * blk + v] = sx;
          tmax = fmaxf(tmax, sx);
        }
    }
    tmax = max_xor16(tmax);
    tmax = max_xor32(tmax);
    // The reference max moves only when the tile max exceeds it by more than 2^8
    // (weights up to 256 are exact enough in fp16 and cannot overflow), so the
    // accumulator rescale below is rare.
    const bool bump = tmax > w.m_run[nb] + 8.f;
    const float m_new = bump ? tmax : w.m_run[nb];
    const float alpha = bump ? __builtin_amdgcn_exp2f(w.m_run[nb] - m_new) : 1.f;
    // a column with several queries can meet a tile before its first visible token
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(sv[j] - m_ref);
      psum += p;
      pf[nb][j] = (_Float16)p;
    }
    w.l_run[nb] = w.l_run[nb] * alpha + psum;
    w.m_run[nb] = m_new;
    // O rows are columns 4*q4 + v; column hh's alpha lives in lane hh (quarter 0)
    if (__ballot(bump && 16 * nb + c < a.ncol)) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float av = __shfl(alpha, (4 * q4 + v) & 15);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) w.o[nb][nt][v] *= av;
      }
    }
  }
  // ---------------- values: lane (q4, c) takes channels 8c..8c+7 of its 8 tokens.
  // Byte i of X[p] holds the codes of (token 2p, token 2p+1) for channel 8c + 2i,
  // of Y[p] for channel 8c + 2i + 1; one converted byte is one k-slot pair of the
  // PV B operand, so N-tile 2i (2i+1) is built from byte i of X (Y).
  uint32_t X[4], Y[4];
  h2_t sp[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    X[p] = (dv[2 * p] & 0x0F0F0F0Fu) | ((dv[2 * p + 1] & 0x0F0F0F0Fu) << 4);
    Y[p] = ((dv[2 * p] >> 4) & 0x0F0F0F0Fu) | (dv[2 * p + 1] & 0xF0F0F0F0u);
    sp[p] = bf16x2_to_h2((sc[2 * p] & 0xFFFFu) | (sc[2 * p + 1] << 16));
  }
#define KVQ_PV_BYTE(I)                                                                                   \
  {                                                                                                      \
    const h8_t bx = h8_from(fp4x2<I>(X[0]) * sp[0], fp4x2<I>(X[1]) * sp[1], fp4x2<I>(X[2]) * sp[2],     \
                            fp4x2<I>(X[3]) * sp[3]);                                                     \
    for (int nb = 0; nb < NB; ++nb)                                                                      \
      w.o[nb][2 * I] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[nb], bx, w.o[nb][2 * I], 0, 0, 0);      \
    const h8_t by = h8_from(fp4x2<I>(Y[0]) * sp[0], fp4x2<I>(Y[1]) * sp[1], fp4x2<I>(Y[2]) * sp[2],     \
                            fp4x2<I>(Y[3]) * sp[3]);                                                     \
    for (int nb = 0; nb < NB; ++nb)                                                                      \
      w.o[nb][2 * I + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[nb], by, w.o[nb][2 * I + 1], 0, 0, 0); \
  }
  KVQ_PV_BYTE(0)
  KVQ_PV_BYTE(1)
  KVQ_PV_BYTE(2)
  KVQ_PV_BYTE(3)
#undef KVQ_PV_BYTE
  // keep the scheduler from interleaving two tiles (register pressure)
  __builtin_amdgcn_sched_barrier(0);
}

// LDS arrays that exist only in the kernels that use them (a function-scope
// __shared__ array is allocated only where its function is instantiated), so
// that the two-stage kernels use exactly two stages of LDS.
template <int N>
struct LdsBytes {
  __device__ static uint8_t* get() {
    __shared__ __attribute__((aligned(16))) uint8_t buf[N];
    return buf;
  }
};
template <>
struct LdsBytes<0> {
  __device__ static uint8_t* get() { return nullptr; }
};

#ifndef KVQ_MFMA_WAVES_PER_EU
#define KVQ_MFMA_WAVES_PER_EU 3  // waves per SIMD the register budget is cut for
#endif
#ifndef KVQ_MFMA_STAGES
#define KVQ_MFMA_STAGES 2  // LDS ring depth per wave (tiles in flight + 1)
#endif

// Waves per SIMD the register budget is cut for: 1-bit QJL keys with G <= 4 fit
// four (128 registers), two column blocks take two.
template <int G, class KP, int NB>
constexpr int kWavesPerEu = NB > 1 ? 2 : (std::is_same<KP, KeysQjl>::value && G <= 4 ? 4 : KVQ_MFMA_WAVES_PER_EU);

// NB blocks of G = 16 columns when NB > 1 (FP4 keys): the blocks share every
// dequantised key and value operand; twice the accumulators cut the waves per SIMD.
// PAGED: the token rows live in pool pages named by the block table; each tile's
// resources cover its page (tiles start on 32-token boundaries and pages, a power
// of two of at least 32 tokens, hold whole tiles).
// SPARSE (contiguous caches, one query): split slot i reads position
// a.sel[b][t_begin + i], staged in LDS; slots without a valid position are masked.
template <int G, class KP, int NB, bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kWavesPerEu<G, KP, NB>, kWavesPerEu<G, KP, NB>)))
decode_mfma_kernel(MfmaDecodeArgs a) {
  static_assert(NB == 1 || G == 16, "column blocks are 16 wide");
  constexpr int kStage = Stage<KP>::kBytes;
  constexpr int NS = KVQ_MFMA_STAGES;
  static_assert(NS == 2 || NS == 3, "ring depth");
  // LDS stages per wave, as separate arrays so that the compiler can tell which
  // stage a direct-to-LDS load writes and wait only for that one
  __shared__ __attribute__((aligned(16))) uint8_t stA[4][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stB[4][kStage];
  uint8_t* stC = LdsBytes<NS == 3 ? 4 * kStage : 0>::get();  // third stage, NS == 3 only
  // the waves' running max / sum are combined through stage-B memory, their
  // outputs through stage-A memory when they fit there, else through a buffer
  // of their own; both stages are idle by then
  constexpr bool kAliasA = sizeof(float) * 4 * G * 129 <= sizeof(stA);
  uint8_t* sm_own = LdsBytes<kAliasA ? 0 : sizeof(float) * 4 * G * 129>::get();
  float (*sm_o)[G][129] = reinterpret_cast<float (*)[G][129]>(kAliasA ? (void*)&stA[0][0] : (void*)sm_own);
  float (*sm_m)[16] = reinterpret_cast<float (*)[16]>(&stB[0][0]);
  float (*sm_l)[16] = reinterpret_cast<float (*)[16]>(&stB[0][0] + 4 * 16 * sizeof(float));
  static_assert(2 * 4 * 16 * sizeof(float) <= sizeof(stB), "stage B too small");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.H + h;
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  // tiles start on 32-token boundaries; tokens [t_lo & ~31, t_lo) are masked
  const int t_begin = (a.t_lo & ~31) + split * a.per_split;
  const int t_end = min(max(a.t_lo, L - a.recent), t_begin + a.per_split);
  // this lane's column 16 nb + lane % 16 is query token j = (c0 + column) / gr,
  // which sees the first L - (nq - 1 - j) tokens; a tile below t_full is whole
  // for every column of the launch
  // (QJL keys: column c is pair c0 + c % G, its piece slots replicated)
  const int lane_col = std::is_same<KP, KeysQjl>::value ? (lane & 15) % G : (lane & 15);
  Limits<NB> lim;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) lim.v[nb] = min(t_end, L - (a.nq - 1 - (a.c0 + 16 * nb + lane_col) / a.gr));
  const int t_full = min(t_end, L - (a.nq - 1 - a.c0 / a.gr));

  static_assert(!(PAGED && SPARSE), "gather mode reads contiguous caches");
  static_assert(!SPARSE || NS == 2, "gather mode runs the two-stage ring");
  __shared__ int spos[SPARSE ? kMfmaSparseSlots : 1];
  __shared__ uint32_t svalid[SPARSE ? kMfmaSparseSlots / 32 : 1];  // bit j: slot j of the tile is valid
  if constexpr (SPARSE) {
    const int32_t* sb = a.sel + (size_t)b * a.sel_stride;
    for (int i = threadIdx.x; i < a.per_split; i += 256) {
      const int slot = t_begin + i;
      const int p = slot < t_end ? sb[slot] : -1;
      spos[i] = p >= 0 && p < a.cap ? p : -1;
    }
    __syncthreads();
    for (int ti = threadIdx.x; ti < a.per_split / 32; ti += 256) {
      uint32_t m = 0;
      for (int j = 0; j < 32; ++j) m |= (spos[ti * 32 + j] >= 0 ? 1u : 0u) << j;
      svalid[ti] = m;
    }
    __syncthreads();
  }
  // the tile's validity mask (gather mode; tiles at or past t_end have none)
  auto valid_of = [&](int t) -> uint32_t {
    if constexpr (SPARSE) return t < t_end ? svalid[(t - t_begin) >> 5] : 0u;
    return ~0u;
  };

  // Buffer resources over this (sequence, KV head)'s rows, or over one page's:
  // 32-bit offsets, and a read past the end of a resource returns zeros instead
  // of faulting (a missing tile reads past the end; a page outside the pool has
  // empty resources).
  const typename KP::R kr = KP::resources(a, bh * a.cap, a.cap);
  const VRsrc vr{rsrc(a.v_codes + bh * a.cap * 64, (size_t)a.cap * 64),
                 rsrc(a.v_scale + bh * a.cap * 8, (size_t)a.cap * 16)};
  // table entry of tile t (-1: no tile), checked against the pool where it is used
  auto page_for = [&](int t) { return PAGED && t < t_end ? page_entry_uniform(a.pm, b, t) : -1; };
  // the loads of tile t, whose table entry the caller looked up
  auto tile_at = [&](int t, int entry) {
    TileSrc<KP> s;
    if constexpr (SPARSE) {
      s.kr = kr;
      s.vr = vr;
      s.t = t < t_end ? t - t_begin : -1;  // a staged slot
    } else if constexpr (!PAGED) {
      s.kr = kr;
      s.vr = vr;
      s.t = t < t_end ? t : a.cap;
    } else {
      const int pg = page_checked(a.pm, entry);
      const int nrows = pg < 0 ? 0 : a.pm.tokens;
      const size_t row0 = ((size_t)(pg < 0 ? 0 : pg) * a.H + h) * a.pm.tokens;
      s.kr = KP::resources(a, row0, nrows);
      s.vr = VRsrc{rsrc(a.v_codes + row0 * 64, (size_t)nrows * 64), rsrc(a.v_scale + row0 * 8, (size_t)nrows * 16)};
      s.t = pg < 0 ? 0 : t & (a.pm.tokens - 1);
    }
    return s;
  };
  auto tile_or_none = [&](int t) { return tile_at(t, page_for(t)); };

  uint8_t* sa = stA[wave];
  uint8_t* sb = stB[wave];
  int t0 = t_begin + wave * 32;
  {
    // A contiguous cache's first two tiles are issued before the sequence
    // length has arrived (and before the query): tiles past the end are read
    // from the cache's own rows and weighted by zero, or never used.
    auto first = [&](int t) {
      if constexpr (PAGED || SPARSE) return tile_or_none(t);
      return TileSrc<KP>{kr, vr, t < a.cap ? t : a.cap};
    };
    const TileSrc<KP> s0 = first(t0), s1 = first(t0 + 128);
    if constexpr (SPARSE) {
      issue_tile_rows<KP>(sa, lane, s0.t, spos, s0.kr, s0.vr);
      issue_tile_rows<KP>(sb, lane, s1.t, spos, s1.kr, s1.vr);
    } else {
      issue_tile<KP>(sa, lane, s0.t, s0.kr, s0.vr);
      issue_tile<KP>(sb, lane, s1.t, s1.kr, s1.vr);
    }
  }
  WaveState<KP, NB> w;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    KP::template load_q<G>(w.q[nb], a, b, h, lane >> 4, lane & 15, 16 * nb);
    w.m_run[nb] = -INFINITY;
    w.l_run[nb] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) w.o[nb][nt] = f4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (NS == 2) {
    for (; t0 < t_end; t0 += 256) {
      // the second tile of a pair may lie past t_end: all its tokens are masked
      tile_step<G, NS, KP, NB, SPARSE>(w, sa, lane, t0, t_full, lim, tile_or_none(t0 + 256), a, spos, valid_of(t0));
      tile_step<G, NS, KP, NB, SPARSE>(w, sb, lane, t0 + 128, t_full, lim, tile_or_none(t0 + 384), a, spos,
                                       valid_of(t0 + 128));
    }
  } else {
    uint8_t* sc = stC + wave * kStage;
    {
      const TileSrc<KP> s2 = tile_or_none(t0 + 256);
      issue_tile<KP>(sc, lane, s2.t, s2.kr, s2.vr);
    }
    while (t0 < t_end) {
      tile_step<G, NS, KP, NB>(w, sa, lane, t0, t_full, lim, tile_or_none(t0 + 384), a);
      if (t0 + 128 >= t_end) break;
      tile_step<G, NS, KP, NB>(w, sb, lane, t0 + 128, t_full, lim, tile_or_none(t0 + 512), a);
      if (t0 + 256 >= t_end) break;
      tile_step<G, NS, KP, NB>(w, sc, lane, t0 + 256, t_full, lim, tile_or_none(t0 + 640), a);
      t0 += 384;
    }
  }
  // drain the refills still in flight before the waves' LDS is reused or the wave exits
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---------------- combine the four waves, write this split's partial result
  // (lane indices are recomputed here rather than kept live across the loop)
  __syncthreads();  // every wave is done with its stages before they hold outputs
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int q4e = lane_e >> 4, ce = lane_e & 15;
  const int tid_e = wave * 64 + lane_e;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {  // one column block at a time through the same LDS
    if (nb) __syncthreads();          // the previous block's partials are written
    float l_run = w.l_run[nb];
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (q4e == 0) {
      sm_m[wave][ce] = w.m_run[nb];
      sm_l[wave][ce] = l_run;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 4 * q4e + v;
      if (hh < G) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) sm_o[wave][hh][8 * ce + nt] = w.o[nb][nt][v];
      }
    }
    __syncthreads();
    for (int e = tid_e; e < G * 128; e += 256) {
      const int hh = e >> 7, ch = e & 127;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][hh]);
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = sm_m[ww][hh];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        Ls += f * sm_l[ww][hh];
        O += f * sm_o[ww][hh][ch];
      }
      if (16 * nb + hh >= a.ncol) continue;  // a column with no query
      const int pc = a.c0 + 16 * nb + hh;
      const size_t row = ((size_t)b * a.nq + pc / a.gr) * a.Hq + (size_t)h * a.gr + pc % a.gr;
      float* p = a.part + (row * a.part_splits + split) * 130;
      p[2 + ch] = O;
      if (ch == 0) {
        p[0] = M;
        p[1] = Ls;
      }
    }
  }
}

template <class KP, bool PAGED, bool SPARSE = false>
int launch_g(const MfmaDecodeArgs& a, int B, int G, hipStream_t st) {
  dim3 grid(a.splits, a.H, B);
  switch (G) {
    case 1: decode_mfma_kernel<1, KP, 1, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 2: decode_mfma_kernel<2, KP, 1, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 4: decode_mfma_kernel<4, KP, 1, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 8: decode_mfma_kernel<8, KP, 1, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 16: decode_mfma_kernel<16, KP, 1, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 32:
      if constexpr (std::is_same<KP, KeysFp4>::value && !SPARSE) {
        decode_mfma_kernel<16, KP, 2, PAGED, false><<<grid, 256, 0, st>>>(a);
        break;
      }
      return KV_EUNSUPPORTED;
    default: return KV_EUNSUPPORTED;
  }
  return KV_OK;
}

}  // namespace

int launch_decode_mfma(const MfmaDecodeArgs& a, int format, int B, int G, hipStream_t st) {
  const bool paged = a.pm.table != nullptr;
  if (a.sel) {  // gather mode: contiguous caches
    if (paged) return KV_EUNSUPPORTED;
    if (format == KV_FMT_FP4) return launch_g<KeysFp4, false, true>(a, B, G, st);
    if (format == KV_FMT_QJL1_FP4V) return launch_g<KeysQjl, false, true>(a, B, G, st);
    return KV_EUNSUPPORTED;
  }
  if (format == KV_FMT_FP4) return paged ? launch_g<KeysFp4, true>(a, B, G, st) : launch_g<KeysFp4, false>(a, B, G, st);
  if (format == KV_FMT_QJL1_FP4V)
    return paged ? launch_g<KeysQjl, true>(a, B, G, st) : launch_g<KeysQjl, false>(a, B, G, st);
  return KV_EUNSUPPORTED;
}

}  // namespace kvq
