// TurboQuant decode attention on the matrix cores (gfx950).
//
// Keys: 2-bit Lloyd-Max codes of the rotated unit key u~, a 128-bit QJL sign
// sketch of the residual, and fp16 norms n (key) and gamma (residual); values:
// 2-bit codes of the rotated unit value and its fp16 norm (page "TurboQuant vs
// OSCAR vs EpiCache", section "quantization frontiers": rotation, a scalar
// Lloyd-Max stage, then the 1-bit QJL stage on the residual).  The logit is
//   n * ( <R q, u~> + sqrt(pi/2)/m * gamma * <S R q, sigma> ).
//
// A symmetric 4-level codebook (levels -l2, -l1, l1, l2 by code 0..3) makes a
// code's level linear in its two bits b1 (high) and b0 (low):
//   level = a0 + a1 b1 + a2 b0,  a0 = lv0, a1 = lv2 - lv0, a2 = lv1 - lv0,
// because the b1 b0 term, lv3 - lv2 - lv1 + lv0, vanishes.  So the key
// products become exact 0/1 bit-plane products on the matrix cores:
//   <q, u~>      = a0 sum(q) + <a1 q, b1> + <a2 q, b0>
//   <qS, sigma>  = 2 <qS, b> - sum(qS)
// (key bits as FP4 operands against FP6 pieces of the query side; the query
// preparation folds the softmax scale (log2 units) and sqrt(pi/2)/m into the
// pieces and the two constant terms, which start the accumulators).  So the
// logit of a token is n (L + gamma Q) with L, Q the two products' sums, two
// mixed-precision FMAs on the fp16 norms.
//
// Columns of every product are (query, head) pairs of one KV head, 16 per
// launch, each column taking the 4 query pieces in 4 steps of the same
// accumulator; so a sequence's draft queries share every tile the cache
// streams, and nothing is combined across lanes.  The value product O = P' V~,
// P' = p n_v, takes each value code's level itself as an fp16 operand of
// v_mfma_f32_16x16x32_f16 (rows of P' are the pairs): a code selects its
// level's low and high bytes from two tables and a third permute pairs them.
// Value codes are transposed to token-major order by ds_read_b64_tr_b4 (a 16 x
// 16 nibble transpose within each 16-lane group).
//
// Softmax: a running reference m per pair (log2 units), raised only when one
// of the pair's logits passes m + 8 (then that pair's sums are scaled down), so
// p <= 2^8 and P' stays in fp16 for value norms below 2^8; a pair's weights are
// never measured against another pair's logits.
//
// Layout per workgroup: 4 waves, each streaming its own 32-token tiles through
// a four-stage LDS ring filled by direct-to-LDS loads three tiles ahead, one
// (sequence, KV head, split) per workgroup; the output stays in the rotated
// basis (the split merge applies R^T).  A tile's LDS reads are one inline-asm
// block that waits for them itself: the compiler cannot tell them from the
// loads still landing in the other stages and would otherwise wait for all.
#include <hip/hip_runtime.h>

#include <utility>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_kernels.h"

namespace kvq {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i2_t __attribute__((ext_vector_type(2)));
typedef int i8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kRsrcFlags = 0x00020000;
// stage layout (bytes) for 32 tokens; the loads of the sketch and the norms
// run on the lanes that carry data only (a direct-to-LDS load writes lane l's
// bytes at 4 l or 16 l from its base, inactive lanes write nothing)
constexpr int kSK = 0;      // key codes, 32 B per token
constexpr int kSS = 1024;   // sketch, 16 B per token
// norms (fp16): token pair (2 i, 2 i + 1) in dword i, or (per-token loads:
// gather mode, an odd capacity) token t in the low half of dword t
constexpr int kSN = 1536;   // key norm
constexpr int kSR = 1664;   // residual norm
constexpr int kSVN = 1792;  // value norm
constexpr int kSV = 1920;   // value codes, 32 B per token
constexpr int kStage = 2944;
constexpr int kStages = 4;  // ring depth per wave: loads run kStages - 1 tiles ahead

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

// s_waitcnt immediate for vmcnt(n) alone (gfx9: vmcnt bits [3:0] and [15:14]).
constexpr int vmcnt_only(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

// fp16 levels of the 8 two-bit codes at bits [s, s + 2) of the nibbles of w,
// in the value product's k-slot order: nibbles 0, 2, 4, 6, 1, 3, 5, 7.
// v_perm_b32 picks byte k of the pair {src0 : src1} (bytes 0..3 from src1):
// with a zero src0 a code c picks byte c of a table, here the low (t_lo) and
// high (t_hi) bytes of the four levels; a second permute interleaves the two.
__device__ __forceinline__ h8_t levels8(uint32_t w, int s, uint32_t t_lo, uint32_t t_hi) {
  const uint32_t e = (w >> s) & 0x03030303u, o = (w >> (s + 4)) & 0x03030303u;
  const uint32_t le = __builtin_amdgcn_perm(0u, t_lo, e), he = __builtin_amdgcn_perm(0u, t_hi, e);
  const uint32_t lo = __builtin_amdgcn_perm(0u, t_lo, o), ho = __builtin_amdgcn_perm(0u, t_hi, o);
  const uint4 d{__builtin_amdgcn_perm(he, le, 0x05010400u), __builtin_amdgcn_perm(he, le, 0x07030602u),
                __builtin_amdgcn_perm(ho, lo, 0x05010400u), __builtin_amdgcn_perm(ho, lo, 0x07030602u)};
  return __builtin_bit_cast(h8_t, d);
}

// QK A-operand row rho of block b (16 rows) holds token 8 (rho / 4) + 4 b + rho % 4:
// then the result rows a lane holds (4 (lane / 16) + v) in blocks 0 and 1 are the
// tokens 8 (lane / 16) + j, j = 4 b + v = 0..7: the PV k-slots of that lane.
__device__ __forceinline__ int qk_token(int rho, int b) { return 8 * (rho >> 2) + 4 * b + (rho & 3); }

struct Res {
  __amdgpu_buffer_rsrc_t kc, sk, kn, kr, vc, vn;
};

// The next tile's loads: resources over its page's token rows (a contiguous
// cache: the (sequence, KV head)'s rows) and its first row in them.
struct TileSrc {
  Res r;
  int t;
};

constexpr int kDmaPerTile = 6;  // direct-to-LDS loads issue_tile makes

// Tile t0 (32-aligned) of a contiguous row range: lane l loads 16 bytes of
// codes, lanes < 32 a token's sketch, and lanes < 16 a token pair's norms
// (PAIRS; the range's length must be even: a pair that straddles its end
// would read as zeros) or lanes < 32 a token's.
template <bool PAIRS>
__device__ __forceinline__ void issue_tile(uint8_t* st, int lane, int t0, const Res& r) {
  const int c16 = t0 * 32 + lane * 16;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + kSK), 16, c16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + kSV), 16, c16, 0, 0, 0);
  if (lane < 32) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st + kSS), 16, t0 * 16 + lane * 16, 0, 0, 0);
    if constexpr (PAIRS) {
      if (lane < 16) {
        const int nb = t0 * 2 + lane * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kn, (lds_ptr_t)(st + kSN), 4, nb, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kr, (lds_ptr_t)(st + kSR), 4, nb, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vn, (lds_ptr_t)(st + kSVN), 4, nb, 0, 0, 0);
      }
    } else {
      const int nb = t0 * 2 + lane * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kn, (lds_ptr_t)(st + kSN), 2, nb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kr, (lds_ptr_t)(st + kSR), 2, nb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vn, (lds_ptr_t)(st + kSVN), 2, nb, 0, 0, 0);
    }
  }
}

// Gather form of issue_tile: staged slot rel starts the tile (rel < 0: none);
// lane rows: slot lane / 2 (codes), slot lane for lanes < 32 (sketch, norms).
// Every wave issues as many loads as issue_tile.
__device__ __forceinline__ void issue_tile_rows(uint8_t* st, int lane, int rel, const int* pos, const Res& r) {
  const int pa = rel < 0 ? -1 : pos[rel + (lane >> 1)];
  const uint32_t c16 = pa < 0 ? ~0u : (uint32_t)pa * 32u + (lane & 1) * 16;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + kSK), 16, c16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + kSV), 16, c16, 0, 0, 0);
  if (lane < 32) {
    const int pn = rel < 0 ? -1 : pos[rel + lane];
    const uint32_t s16 = pn < 0 ? ~0u : (uint32_t)pn * 16u, nb = pn < 0 ? ~0u : (uint32_t)pn * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st + kSS), 16, s16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kn, (lds_ptr_t)(st + kSN), 2, nb, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kr, (lds_ptr_t)(st + kSR), 2, nb, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vn, (lds_ptr_t)(st + kSVN), 2, nb, 0, 0, 0);
  }
}

// One bit per nibble of a key word, as the FP4 operand of a scaled product:
// dword d holds bits d, d + 4, ..., d + 28 (element 8 d + n = bit 4 n + d),
// each left where it is in its nibble (E2M1 0.5, 1 or 2 for d = 0, 1, 2) but
// bit 3, the E2M1 sign, moved to bit 2; so element 8 d + n is the bit times
// 1, 2, 4, 4 (block scale 2), which the query pieces divide back out.
__device__ __forceinline__ i8_t bit_nibbles(uint32_t w) {
  return i8_t{(int)(w & 0x11111111u), (int)(w & 0x22222222u), (int)(w & 0x44444444u), (int)((w >> 1) & 0x44444444u),
              0, 0, 0, 0};
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max of 8 values (none NaN)
__device__ __forceinline__ float max8(const float (&x)[8]) {
  return max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), fmaxf(x[6], x[7]));
}

// Key products on v_mfma_scale_f32_16x16x128_f8f6f4: A = key bits (FP4, 0 or
// 0.5, block scale 2), B = FP6 (E2M3) piece P of the query operand, whose block
// scale is byte P of `scales`.  With these formats lane quarter q of either
// operand holds k-block q (its 32 elements in order; FP6 packed 6 bits each
// into 6 dwords) and the scale of k-block q.  FP6 runs at the FP4 rate.
template <int P>
__device__ __forceinline__ f4_t key_product(i8_t a, i8_t b, int scales, f4_t acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 2, 0, 128, P, scales);
}

// Value of lane (l & ~15) | ((l + 8) & 15): the other half of this lane's
// 16-lane row (a DPP row rotation by 8, the same in either direction).
__device__ __forceinline__ float row_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// fp16 half h (0: low, 1: high) of w
__device__ __forceinline__ float half_f16(uint32_t w, int h) { return (float)__builtin_bit_cast(h2_t, w)[h]; }

// STEPS = 4: column c is pair c0 + c and takes the 4 query pieces in 4 steps;
// STEPS = 2 (at most 8 pairs): columns c and c + 8 are pair c0 + c, taking
// pieces 0, 1 and 2, 3, and each adds the other's sums (one row rotation).
template <int STEPS>
struct WaveState {
  // B operands of the key products (6 dwords of FP6 used): [product (code
  // words 0..3, 4..7, sketch)][step] of this lane's column
  i8_t bq[3][STEPS];
  int bs[3];           // their block scales, byte s = step s
  float lc, qc;        // accumulator starts of L and Q (the two constant terms)
  float m_run;         // running reference (log2 units) of this lane's pair
  float l_run;         // this lane's part of its pair's sum of p
  f4_t o[8];           // O rows 4 (lane / 16) + v (pairs), channels of N-tile nt
  uint32_t t_lo, t_hi;  // low / high bytes of the four levels as fp16, byte c for code c
};

// Per-tile masks: a lane's pair sees positions [t_lo, lim); `valid` bit j:
// slot j of the tile holds a position (gather mode).
struct TileMask {
  int t_lo, lim;
  bool live;  // the lane's column is a pair of this launch
};

// A tile's part of this lane: key words q4 and 4 + q4 of its A-operand tokens
// (block 1's token is 4 after block 0's: 128 bytes of codes, 64 of sketch),
// norms of tokens 8 q4 + [0, 8) as fp16 pairs (token 8 q4 + j in half j % 2 of
// dword j / 2), value codes through the transpose.
struct TileRegs {
  uint32_t kw00, kw01, kw10, kw11, sw0, sw1;
  uint4 nk, nr, nv;
  i2_t vx0, vx1;
};

// Addresses are this lane's in the tile's stage.  GATHER: the norms came one
// token per dword (low half); pair them.
template <bool GATHER>
__device__ __forceinline__ void read_stage(TileRegs& r, uint32_t a_key, uint32_t a_sk, uint32_t a_nrm,
                                           uint32_t a_val) {
  constexpr int o = 0;
  if constexpr (!GATHER) {
    asm volatile(
        "ds_read_b32 %0, %11 offset:%c15\n\t"
        "ds_read_b32 %1, %11 offset:%c16\n\t"
        "ds_read_b32 %2, %11 offset:%c17\n\t"
        "ds_read_b32 %3, %11 offset:%c18\n\t"
        "ds_read_b32 %4, %12 offset:%c19\n\t"
        "ds_read_b32 %5, %12 offset:%c20\n\t"
        "ds_read_b128 %6, %13 offset:%c21\n\t"
        "ds_read_b128 %7, %13 offset:%c22\n\t"
        "ds_read_b128 %8, %13 offset:%c23\n\t"
        "ds_read_b64_tr_b4 %9, %14 offset:%c24\n\t"
        "ds_read_b64_tr_b4 %10, %14 offset:%c25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.kw00), "=&v"(r.kw01), "=&v"(r.kw10), "=&v"(r.kw11), "=&v"(r.sw0), "=&v"(r.sw1), "=&v"(r.nk),
          "=&v"(r.nr), "=&v"(r.nv), "=&v"(r.vx0), "=&v"(r.vx1)
        : "v"(a_key), "v"(a_sk), "v"(a_nrm), "v"(a_val), "i"(o + kSK), "i"(o + kSK + 128), "i"(o + kSK + 16),
          "i"(o + kSK + 144), "i"(o + kSS), "i"(o + kSS + 64), "i"(o + kSN), "i"(o + kSR), "i"(o + kSVN),
          "i"(o + kSV), "i"(o + kSV + 16));
  } else {
    uint4 n[6];
    asm volatile(
        "ds_read_b32 %0, %14 offset:%c18\n\t"
        "ds_read_b32 %1, %14 offset:%c19\n\t"
        "ds_read_b32 %2, %14 offset:%c20\n\t"
        "ds_read_b32 %3, %14 offset:%c21\n\t"
        "ds_read_b32 %4, %15 offset:%c22\n\t"
        "ds_read_b32 %5, %15 offset:%c23\n\t"
        "ds_read_b128 %6, %16 offset:%c24\n\t"
        "ds_read_b128 %7, %16 offset:%c25\n\t"
        "ds_read_b128 %8, %16 offset:%c26\n\t"
        "ds_read_b128 %9, %16 offset:%c27\n\t"
        "ds_read_b128 %10, %16 offset:%c28\n\t"
        "ds_read_b128 %11, %16 offset:%c29\n\t"
        "ds_read_b64_tr_b4 %12, %17 offset:%c30\n\t"
        "ds_read_b64_tr_b4 %13, %17 offset:%c31\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.kw00), "=&v"(r.kw01), "=&v"(r.kw10), "=&v"(r.kw11), "=&v"(r.sw0), "=&v"(r.sw1), "=&v"(n[0]),
          "=&v"(n[1]), "=&v"(n[2]), "=&v"(n[3]), "=&v"(n[4]), "=&v"(n[5]), "=&v"(r.vx0), "=&v"(r.vx1)
        : "v"(a_key), "v"(a_sk), "v"(a_nrm), "v"(a_val), "i"(o + kSK), "i"(o + kSK + 128), "i"(o + kSK + 16),
          "i"(o + kSK + 144), "i"(o + kSS), "i"(o + kSS + 64), "i"(o + kSN), "i"(o + kSN + 16), "i"(o + kSR),
          "i"(o + kSR + 16), "i"(o + kSVN), "i"(o + kSVN + 16), "i"(o + kSV), "i"(o + kSV + 16));
    // the low halves of dwords (x, y) -> one dword: v_perm bytes 0, 1 of y then of x
    auto pk = [](uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); };
    r.nk = uint4{pk(n[0].x, n[0].y), pk(n[0].z, n[0].w), pk(n[1].x, n[1].y), pk(n[1].z, n[1].w)};
    r.nr = uint4{pk(n[2].x, n[2].y), pk(n[2].z, n[2].w), pk(n[3].x, n[3].y), pk(n[3].z, n[3].w)};
    r.nv = uint4{pk(n[4].x, n[4].y), pk(n[4].z, n[4].w), pk(n[5].x, n[5].y), pk(n[5].z, n[5].w)};
  }
}

// The value product of a tile whose weights are pa (PV k-slot order) and whose
// transposed value codes are vx: N-tile nt = 2 chunk + parity; column c <->
// channel 32 chunk + 2 c + parity, whose code is bits [2 parity, 2 parity + 2)
// of each nibble (nibble n = token 8 q4 + n).
template <int STEPS>
__device__ __forceinline__ void value_product(WaveState<STEPS>& w, h8_t pa, i2_t vx0, i2_t vx1) {
  const uint32_t vx[4] = {(uint32_t)vx0[0], (uint32_t)vx0[1], (uint32_t)vx1[0], (uint32_t)vx1[1]};
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int nt = 2 * ch + par;
      w.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, levels8(vx[ch], 2 * par, w.t_lo, w.t_hi), w.o[nt], 0, 0, 0);
    }
  }
}

// f(integral_constant<int, K>) for K in the sequence, in order.
template <typename F, int... K>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, K...>, F&& f) {
  (f(std::integral_constant<int, K>{}), ...);
}

// The key products of a tile, S^T = K Q^T per 16-token block: L from the two
// code-word products and Q from the sketch, in four independent chains (two
// blocks), product k of step p = k / 6 on block k % 2 and product (k / 2) % 3.
// A wave issues in order and vector work overlaps only a matrix product issued
// before it, so the schedule is written out in fenced groups: each computes on
// the vector ALU what a later product needs (a key word's bit planes during
// the first step, then, with PV, the code lookups of the pending tile's value
// N-tile j) and then issues its products (key product k, value product j).
template <int STEPS, bool PV>
__device__ __forceinline__ void key_products(WaveState<STEPS>& w, const TileRegs& r, f4_t (&L)[2], f4_t (&Q)[2],
                                             h8_t pa, i2_t vx0, i2_t vx1) {
  constexpr int NK = 6 * STEPS;
  const uint32_t kw[2][3] = {{r.kw00, r.kw10, r.sw0}, {r.kw01, r.kw11, r.sw1}};  // [block][product]
  const uint32_t vx[4] = {(uint32_t)vx0[0], (uint32_t)vx0[1], (uint32_t)vx1[0], (uint32_t)vx1[1]};
  i8_t a[2][3];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    L[b] = f4_t{w.lc, w.lc, w.lc, w.lc};
    Q[b] = f4_t{w.qc, w.qc, w.qc, w.qc};
  }
  auto kp = [&](auto K) {
    constexpr int k = decltype(K)::value, p = k / 6, b = k % 2, m = (k / 2) % 3;
    if constexpr (m < 2) L[b] = key_product<p>(a[b][m], w.bq[m][p], w.bs[m], L[b]);
    else Q[b] = key_product<p>(a[b][m], w.bq[m][p], w.bs[m], Q[b]);
  };
  h8_t vb;  // B operand of the value N-tile in hand
  auto group = [&](auto K) {
    constexpr int k = decltype(K)::value;  // group k: key product k (if any), value N-tile j = k - 6
    constexpr int j = k - 6;
    if constexpr (k < 6) a[k % 2][k / 2] = bit_nibbles(kw[k % 2][k / 2]);
    if constexpr (PV && j >= 0 && j < 8) vb = levels8(vx[j >> 1], 2 * (j & 1), w.t_lo, w.t_hi);
    if constexpr (k < NK) kp(std::integral_constant<int, k>{});
    if constexpr (PV && j >= 0 && j < 8) w.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, w.o[j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int NG = NK > 14 ? NK : 14;  // groups: every key product, value N-tiles 0..7 from group 6
  for_each_index(std::make_integer_sequence<int, NG>{}, group);
}

// Softmax step of a tile: logits n (L + gamma Q) of the lane's tokens 8 q4 + 4 b
// + v, the pair's running reference and sum, and the weights P' = p n_v (fp16,
// rounded to nearest) in the PV k-slot order (tokens 0, 2, 4, 6, 1, 3, 5, 7 of
// the lane's eight).  `full`: every token of the tile counts for every pair.
template <int STEPS>
__device__ __forceinline__ h8_t softmax_step(WaveState<STEPS>& w, const TileRegs& r, const f4_t (&L)[2], const f4_t (&Q)[2],
                                             int q4, int t0, bool full, const TileMask& mk, uint32_t valid) {

  const uint32_t nkw[4] = {r.nk.x, r.nk.y, r.nk.z, r.nk.w}, nrw[4] = {r.nr.x, r.nr.y, r.nr.z, r.nr.w};
  const uint32_t nvw[4] = {r.nv.x, r.nv.y, r.nv.z, r.nv.w};
  auto nk = [&](int j) { return half_f16(nkw[j >> 1], j & 1); };
  auto nv = [&](int j) { return half_f16(nvw[j >> 1], j & 1); };
  float t[8], s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    t[j] = __builtin_fmaf(half_f16(nrw[j >> 1], j & 1), Q[j >> 2][j & 3], L[j >> 2][j & 3]);
    if constexpr (STEPS == 2) t[j] += row_ror8(t[j]);  // the other column half's pieces
    s[j] = __builtin_fmaf(nk(j), t[j], -w.m_run);
  }
  // masked positions (only boundary tiles) take -inf
  auto mask = [&](float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = t0 + 8 * q4 + j;
      const bool in = tok >= mk.t_lo && tok < mk.lim && ((valid >> (8 * q4 + j)) & 1u);
      x[j] = in ? x[j] : -INFINITY;
    }
  };
  if (!full) mask(s);
  const float mx = max8(s);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(mk.live && mx > 8.f) != 0, 0)) {
    // raise each pair's reference to its largest logit so far (the max over the
    // pair's four lanes, l and l ^ 16, l ^ 32) and rescale its sums; output row
    // r of this lane (4 q4 + v) is the pair of lane r
    float sa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sa[j] = nk(j) * t[j];
    if (!full) mask(sa);
    const float ma = max_xor32(max_xor16(max8(sa)));
    const float m_new = mk.live ? fmaxf(ma, w.m_run) : 0.f;
    // a pair that has seen no position yet keeps -inf and scales by 1
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(w.m_run - m_new);
    w.l_run *= alpha;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, 4 * q4 + v);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) w.o[nt][v] *= av;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = m_new == -INFINITY ? -INFINITY : sa[j] - m_new;
    w.m_run = m_new;
  }
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(s[j]);
    w.l_run += p[j];
  }
  h8_t pa;
  constexpr int order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
  for (int k = 0; k < 8; ++k) pa[k] = (_Float16)__builtin_fmaf(nv(order[k]), p[order[k]], 0.f);
  return pa;
}

// Waves per SIMD the register budget is cut for: three with two pieces per
// column (the ring of three workgroups fits the LDS), two with four.
#ifndef KVQ_TURBO_WAVES_PER_EU
#define KVQ_TURBO_WAVES_PER_EU 3
#endif
#ifndef KVQ_TURBO_WAVES_PER_EU_4STEP
#define KVQ_TURBO_WAVES_PER_EU_4STEP 2
#endif

// PAGED: token rows in pool pages named by the block table, resources per tile.
// SPARSE (contiguous caches): split slot i reads position a.sel[b][t_begin + i],
// staged in LDS; slots without a valid position are masked.  PAIRS: norms load
// as token pairs (row ranges of even length: not SPARSE).  STEPS: see WaveState.
template <bool PAGED, bool SPARSE, bool PAIRS, int STEPS>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(STEPS == 2 ? KVQ_TURBO_WAVES_PER_EU : KVQ_TURBO_WAVES_PER_EU_4STEP,
                                   STEPS == 2 ? KVQ_TURBO_WAVES_PER_EU : KVQ_TURBO_WAVES_PER_EU_4STEP)))
decode_turbo_kernel(TurboDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][kStages][kStage];
  __shared__ float sm_m[4][16], sm_l[4][16];
  // after the loop the rings hold the four waves' outputs
  float (*sm_o)[16][129] = reinterpret_cast<float (*)[16][129]>(&ring[0][0][0]);
  static_assert(sizeof(ring) >= 4 * 16 * 129 * sizeof(float), "outputs fit the rings");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.H + h;
  const int q4 = lane >> 4, c = lane & 15;
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  // pairs c0 .. c0 + ncol - 1 of this KV head: pair j G + g is query j, head g;
  // query j sees the first L - (nq - 1 - j) tokens
  const int G = a.gr;
  const int j_first = a.c0 / G, j_last = (a.c0 + a.ncol - 1) / G;
  // packed tokens [t_lo, L - recent): tiles start 32-aligned below t_lo
  const int t_begin = (a.t_lo & ~31) + split * a.per_split;
  const int t_pack = max(a.t_lo, L - a.recent);
  const int t_stop = min(t_pack, L - (a.nq - 1 - j_last));
  const int t_end = t_stop <= a.t_lo ? t_begin : min(t_stop, t_begin + a.per_split);
  // tiles below t_full hold no position any live pair must skip
  const int t_full = min(t_end, L - (a.nq - 1 - j_first));


  // resources over nrows token rows from row0 (nrows 0: every read is zeros)
  auto res_at = [&](size_t row0, int nrows) {
    return Res{rsrc(a.k_codes + row0 * 32, (size_t)nrows * 32), rsrc(a.k_sketch + row0 * 16, (size_t)nrows * 16),
               rsrc(a.k_norm + row0, (size_t)nrows * 2),        rsrc(a.k_rnorm + row0, (size_t)nrows * 2),
               rsrc(a.v_codes + row0 * 32, (size_t)nrows * 32), rsrc(a.v_norm + row0, (size_t)nrows * 2)};
  };
  const Res res = res_at(bh * a.cap, a.cap);
  static_assert(!(PAGED && SPARSE), "gather mode reads contiguous caches");
  __shared__ int spos[SPARSE ? kMfmaSparseSlots : 1];
  __shared__ uint32_t svalid[SPARSE ? kMfmaSparseSlots / 32 : 1];
  if constexpr (SPARSE) {
    const int32_t* sbp = a.sel + (size_t)b * a.sel_stride;
    for (int i = threadIdx.x; i < a.per_split; i += 256) {
      const int slot = t_begin + i;
      const int p = slot < t_end ? sbp[slot] : -1;
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
  auto valid_of = [&](int t) -> uint32_t {
    if constexpr (SPARSE) return t < t_end ? svalid[(t - t_begin) >> 5] : 0u;
    return ~0u;
  };
  // a missing tile reads past the end of its resources: zeros, no memory traffic
  auto tile_or_none = [&](int t) {
    TileSrc s;
    if constexpr (SPARSE) {
      s.r = res;
      s.t = t < t_end ? t - t_begin : -1;  // a staged slot
    } else if constexpr (!PAGED) {
      s.r = res;
      s.t = t < t_end ? t : a.cap;
    } else {
      const int pg = t < t_end ? page_of_uniform(a.pm, b, t) : -1;
      s.r = res_at(((size_t)(pg < 0 ? 0 : pg) * a.H + h) * a.pm.tokens, pg < 0 ? 0 : a.pm.tokens);
      s.t = pg < 0 ? 0 : t & (a.pm.tokens - 1);
    }
    return s;
  };
  uint8_t* my_ring = &ring[wave][0][0];
  auto issue = [&](int stage, int t) {
    const TileSrc s = tile_or_none(t);
    uint8_t* st = my_ring + stage * kStage;
    if constexpr (SPARSE) issue_tile_rows(st, lane, s.t, spos, s.r);
    else issue_tile<PAIRS>(st, lane, s.t, s.r);
  };
  // this lane's LDS addresses in stage 0 (stage s: s * kStage further)
  const uint32_t ring0 = (uint32_t)(uintptr_t)my_ring;
  uint32_t a_key = ring0 + qk_token(c, 0) * 32 + 4 * q4;
  uint32_t a_sk = ring0 + qk_token(c, 0) * 16 + 4 * q4;
  uint32_t a_nrm = ring0 + (PAIRS ? 16 : 32) * q4;
  uint32_t a_val = ring0 + (8 * q4 + (c & 7)) * 32 + 8 * (c >> 3);
  asm volatile("" : "+v"(a_key), "+v"(a_sk), "+v"(a_nrm), "+v"(a_val));

  // wave w takes tiles t_begin + 32 w + 128 i, i = 0, 1, ...; tile i in stage
  // i % 4.  Software pipeline: the key products of tile i + 1 run beside the
  // value product of tile i (matrix-core and vector work of one wave overlap),
  // then tile i + 1's softmax.
  const int t_first = t_begin + wave * 32;
  if constexpr (PAGED || SPARSE) {
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) issue(i, t_first + 128 * i);
  } else {
    // A contiguous cache's first tiles are issued before the sequence length
    // and the query have arrived: a tile past the end is read from the cache's
    // own rows and never used, and a partial tile's extra tokens are masked.
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) {
      const int t = t_first + 128 * i;
      issue_tile<PAIRS>(my_ring + i * kStage, lane, t < a.cap ? t : a.cap, res);
    }
  }
  WaveState<STEPS> w;
  TileMask mk;
  constexpr int kCols = STEPS == 2 ? 8 : 16;  // distinct pairs per launch
  {
    const int col = c % kCols;
    const int pair = a.c0 + col;
    mk.live = col < a.ncol;
    const int jq = (mk.live ? pair : a.c0) / G, g = (mk.live ? pair : a.c0) % G;
    mk.t_lo = a.t_lo;
    mk.lim = min(t_end, L - (a.nq - 1 - jq));
    const size_t qrow = ((size_t)b * a.nq + jq) * a.Hq + (size_t)h * G + g;
    const uint8_t* pc = a.qpieces + qrow * kTurboPieceBytes;
    const int p0 = STEPS == 2 && c >= 8 ? 2 : 0;  // this column's first piece
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      int sc = 0;
#pragma unroll
      for (int p = 0; p < STEPS; ++p) {
        const uint8_t* base = pc + (m * 4 + p0 + p) * 144;
        const uint4 lo4 = *reinterpret_cast<const uint4*>(base + 32 * q4);
        const uint2 hi2 = *reinterpret_cast<const uint2*>(base + 32 * q4 + 16);
        w.bq[m][p] = mk.live ? i8_t{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w, (int)hi2.x, (int)hi2.y, 0, 0}
                             : i8_t{0, 0, 0, 0, 0, 0, 0, 0};
        sc |= (mk.live ? (int)base[128 + q4] : 127) << (8 * p);
      }
      w.bs[m] = sc;
    }
    const float2 cst = *reinterpret_cast<const float2*>(pc + kTurboPieceConstOff);
    w.lc = mk.live && p0 == 0 ? cst.x : 0.f;  // the constant terms once per pair
    w.qc = mk.live && p0 == 0 ? cst.y : 0.f;
    w.t_lo = 0;
    w.t_hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)a.levels[k]);
      w.t_lo |= (hb & 0xFFu) << (8 * k);
      w.t_hi |= (hb >> 8) << (8 * k);
    }
  }
  w.m_run = mk.live ? -INFINITY : 0.f;  // a column past the launch's pairs never moves
  w.l_run = 0.f;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) w.o[nt] = f4_t{0.f, 0.f, 0.f, 0.f};
  h8_t pa;        // weights of the tile whose value product is pending
  i2_t vx0, vx1;  // its value codes
  // tile t0 in stage st: refill the stage read last (its reads have completed)
  // kStages - 1 tiles ahead, wait for this tile's loads, read it, and run its
  // key products beside the pending value product (none before the first tile)
  auto step = [&](auto PV, int st, int t0) {
    issue((st + kStages - 1) % kStages, t0 + 128 * (kStages - 1));
    __builtin_amdgcn_s_waitcnt(vmcnt_only((kStages - 1) * kDmaPerTile));
    TileRegs r;
    const uint32_t so = st * kStage;
    read_stage<!PAIRS>(r, a_key + so, a_sk + so, a_nrm + so, a_val + so);
    const uint32_t valid = valid_of(t0);
    const bool full = t0 >= a.t_lo && t0 + 32 <= t_full && valid == ~0u;
    f4_t L[2], Q[2];
    key_products<STEPS, decltype(PV)::value>(w, r, L, Q, pa, vx0, vx1);
    pa = softmax_step(w, r, L, Q, q4, t0, full, mk, valid);
    vx0 = r.vx0;
    vx1 = r.vx1;
  };
  if (t_first < t_end) {
    step(std::false_type{}, 0, t_first);
    int st = 1;
    for (int t0 = t_first + 128; t0 < t_end; t0 += 128) {
      step(std::true_type{}, st, t0);
      st = st + 1 == kStages ? 0 : st + 1;
    }
    value_product(w, pa, vx0, vx1);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));  // the refills past the last tile have landed

  // ---------------- combine the four waves, write this split's partial rows
  __syncthreads();
  float l_run = w.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (q4 == 0) {  // (STEPS 2: columns c and c + 8 hold the same)
    sm_m[wave][c] = w.m_run;
    sm_l[wave][c] = l_run;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * q4 + v;
    if (row < a.ncol) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) sm_o[wave][row][32 * (nt >> 1) + 2 * c + (nt & 1)] = w.o[nt][v];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.ncol * 128; e += 256) {
    const int row = e >> 7, ch = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][row]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = sm_m[ww][row];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      Ls += f * sm_l[ww][row];
      O += f * sm_o[ww][row][ch];
    }
    const int pair = a.c0 + row;
    const size_t qrow = ((size_t)b * a.nq + pair / G) * a.Hq + (size_t)h * G + pair % G;
    float* p = a.part + (qrow * a.part_splits + split) * 130;
    p[2 + ch] = O;
    if (ch == 0) {
      p[0] = M;
      p[1] = Ls;
    }
  }
}

}  // namespace

namespace {
template <bool PAGED, bool SPARSE, bool PAIRS>
int launch_turbo(const TurboDecodeArgs& a, int B, hipStream_t st) {
  static_assert(!(SPARSE && PAIRS), "gathered norms load per token");
  dim3 grid(a.splits, a.H, B);
  if (a.ncol <= 8) decode_turbo_kernel<PAGED, SPARSE, PAIRS, 2><<<grid, 256, 0, st>>>(a);
  else decode_turbo_kernel<PAGED, SPARSE, PAIRS, 4><<<grid, 256, 0, st>>>(a);
  return KV_OK;
}
}  // namespace

int launch_decode_turbo(const TurboDecodeArgs& a, int B, hipStream_t st) {
  if (a.ncol < 1 || a.ncol > 16) return KV_EINVAL;
  if (a.sel) return a.pm.table ? KV_EUNSUPPORTED : launch_turbo<false, true, false>(a, B, st);
  // pool pages hold page_tokens (a power of two >= 32) rows; a contiguous
  // cache's row ranges are the capacity long
  if (a.pm.table) return launch_turbo<true, false, true>(a, B, st);
  return a.cap % 2 == 0 ? launch_turbo<false, false, true>(a, B, st) : launch_turbo<false, false, false>(a, B, st);
}

}  // namespace kvq
