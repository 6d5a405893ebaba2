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
// (key bits as FP4 operands against FP6 pieces of the query side, below).  The
// value product O = P' V~, P' = p n_v, takes each value code's level itself as
// an fp16 operand of v_mfma_f32_16x16x32_f16: two byte permutes look a code up
// in a table of the four levels' low and high bytes.  Value codes are transposed
// to token-major order by ds_read_b64_tr_b4 (a 16 x 16 nibble transpose within
// each 16-lane group).
//
// Layout per workgroup, as in the FP4 kernel: 4 waves, each streaming its own
// 32-token tiles through a two-stage LDS ring filled by direct-to-LDS loads,
// one (sequence, KV head, split) per workgroup; the output stays in the rotated
// basis (the split merge applies R^T).
#include <hip/hip_runtime.h>

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
// stage layout (bytes) for 32 tokens
constexpr int kSK = 0;      // key codes, 32 B per token
constexpr int kSS = 1024;   // sketch, 16 B per token (lanes 32..63 of its load write zeros up to 2048)
constexpr int kSN = 2048;   // key norm: token t in the low half of dword t (then zeros)
constexpr int kSR = 2304;   // residual norm, same form
constexpr int kSV = 2560;   // value codes, 32 B per token
constexpr int kSVN = 3584;  // value norm, same form as the key norm
constexpr int kStage = 3840;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

// fp16 levels of the 8 two-bit codes at bits [s, s + 2) of the nibbles of w,
// in the value product's k-slot order: nibbles 0, 2, 4, 6, 1, 3, 5, 7.
// v_perm_b32 picks byte k of the pair {src0 : src1} (bytes 4..7 from src0):
// the first permute turns codes c, c' into the selector (c, c + 4, c', c' + 4),
// the second reads the low and high bytes of levels c and c' from the tables.
__device__ __forceinline__ h8_t levels8(uint32_t w, int s, uint32_t t_lo, uint32_t t_hi) {
  const uint32_t e = (w >> s) & 0x03030303u, o = (w >> (s + 4)) & 0x03030303u;
  const uint32_t e4 = e | 0x04040404u, o4 = o | 0x04040404u;
  const uint4 d{__builtin_amdgcn_perm(t_hi, t_lo, __builtin_amdgcn_perm(e4, e, 0x05010400u)),
                __builtin_amdgcn_perm(t_hi, t_lo, __builtin_amdgcn_perm(e4, e, 0x07030602u)),
                __builtin_amdgcn_perm(t_hi, t_lo, __builtin_amdgcn_perm(o4, o, 0x05010400u)),
                __builtin_amdgcn_perm(t_hi, t_lo, __builtin_amdgcn_perm(o4, o, 0x07030602u))};
  return __builtin_bit_cast(h8_t, d);
}

// Value of lane (l & ~15) | ((l + 8) & 15): the other half of this lane's
// 16-lane row (a DPP row rotation by 8, the same in either direction).
__device__ __forceinline__ float row_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t row_ror8(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);
}

// QK A-operand row rho of block b (16 rows) holds token 8 (rho / 4) + 4 b + rho % 4:
// then the result rows a lane holds (4 (lane / 16) + v) in blocks 0 and 1 are the
// tokens 8 (lane / 16) + j, j = 4 b + v = 0..7: the PV k-slots of that lane.
__device__ __forceinline__ int qk_token(int rho, int b) { return 8 * (rho >> 2) + 4 * b + (rho & 3); }

struct Res {
  __amdgpu_buffer_rsrc_t kc, sk, kn, kr, vc, vn;
  int n_end;  // a byte offset past every norm resource
};

// The next tile's loads: resources over its page's token rows (a contiguous
// cache: the (sequence, KV head)'s rows) and its first row in them.
struct TileSrc {
  Res r;
  int t;
};

constexpr int kDmaPerTile = 6;  // direct-to-LDS loads issue_tile makes

__device__ __forceinline__ void issue_tile(uint8_t* st, int lane, int t0, const Res& r) {
  const int c16 = t0 * 32 + lane * 16;
  const int nb = lane < 32 ? t0 * 2 + lane * 2 : r.n_end;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + kSK), 16, c16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st + kSS), 16, lane < 32 ? t0 * 16 + lane * 16 : r.n_end,
                                           0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kn, (lds_ptr_t)(st + kSN), 2, nb, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kr, (lds_ptr_t)(st + kSR), 2, nb, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + kSV), 16, c16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vn, (lds_ptr_t)(st + kSVN), 2, nb, 0, 0, 0);
}

// Gather form of issue_tile: staged slot rel starts the tile (rel < 0: none);
// lane rows: slot lane / 2 (codes), slot lane for lanes < 32 (sketch, norms).
// The number of loads is issue_tile's.
__device__ __forceinline__ void issue_tile_rows(uint8_t* st, int lane, int rel, const int* pos, const Res& r) {
  const int pa = rel < 0 ? -1 : pos[rel + (lane >> 1)];
  const int pn = rel < 0 || lane >= 32 ? -1 : pos[rel + lane];
  const uint32_t c16 = pa < 0 ? ~0u : (uint32_t)pa * 32u + (lane & 1) * 16;
  const uint32_t s16 = pn < 0 ? ~0u : (uint32_t)pn * 16u, nb = pn < 0 ? ~0u : (uint32_t)pn * 2u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + kSK), 16, c16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.sk, (lds_ptr_t)(st + kSS), 16, s16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kn, (lds_ptr_t)(st + kSN), 2, nb, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kr, (lds_ptr_t)(st + kSR), 2, nb, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + kSV), 16, c16, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vn, (lds_ptr_t)(st + kSVN), 2, nb, 0, 0, 0);
}

struct Consts {
  float a0;            // level of code 0
  uint32_t t_lo, t_hi;  // low / high bytes of the four levels as fp16, byte c for code c
};

// One bit per nibble of a key word, as the FP4 operand of a scaled product:
// dword d holds bits d, d + 4, ..., d + 28 (element 8 d + n = bit 4 n + d).
__device__ __forceinline__ i8_t bit_nibbles(uint32_t w) {
  const uint32_t m = 0x11111111u;
  return i8_t{(int)(w & m), (int)((w >> 1) & m), (int)((w >> 2) & m), (int)((w >> 3) & m), 0, 0, 0, 0};
}

// Key products on v_mfma_scale_f32_16x16x128_f8f6f4: A = key bits (FP4, 0 or
// 0.5, block scale 2), B = FP6 (E2M3) pieces of the query operand with their
// block scales.  With these formats lane quarter q of either operand holds
// k-block q (its 32 elements in order; FP6 packed 6 bits each into 6 dwords)
// and the scale of k-block q.  FP6 runs at the FP4 rate, faster than FP8.
__device__ __forceinline__ f4_t key_product(i8_t a, i8_t b, int scale_b, f4_t acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 2, 0, 128, 0, scale_b);
}

template <int G>
struct WaveState {
  // B operands of the key products (6 dwords of FP6 used): [product (code
  // words 0..3, 4..7, sketch)][piece set]: columns 0..7 carry pieces 2 s,
  // columns 8..15 pieces 2 s + 1
  i8_t bq[3][2];
  int bs[3][2];  // their block scales
  float cst;     // a0 * sum(R q) for this lane's head
  float sqs;     // sum(S R q)
  float m_run, l_run;  // running max, sum of p
  f4_t o[8];
};

// One 32-token tile (see tile_step of the FP4 kernel for the ring protocol).
// SP: gather mode (nx.t a staged slot of pos); `valid` bit j: slot j of the tile
// holds a position.
template <int G, bool SP = false>
__device__ __forceinline__ void tile_step(WaveState<G>& w, uint8_t* st, int lane, int t0, int t_end,
                                          const TileSrc& nx, const TurboDecodeArgs& a, const Consts& k,
                                          const int* pos = nullptr, uint32_t valid = ~0u) {
  const int q4 = lane >> 4, c = lane & 15;
  // This stage's tile has landed once at most the other stage's refill (the
  // kDmaPerTile loads issued after it) is outstanding.  Waited for explicitly:
  // the compiler's own wait for loads into LDS is not placed reliably across
  // the loop back-edge.
  __builtin_amdgcn_s_waitcnt(0x0F70 | kDmaPerTile);  // vmcnt(kDmaPerTile)
  // ---- fragments of this lane
  int ko = qk_token(c, 0) * 32, so = qk_token(c, 0) * 16, no = 4 * 8 * q4;
  int vo = (8 * q4 + (c & 7)) * 32 + 8 * (c >> 3);
  asm volatile("" : "+v"(ko), "+v"(so), "+v"(no), "+v"(vo));
  // this lane's key words of its A-operand token: code words q4 and 4 + q4,
  // sketch dword q4 (block 1's token is 4 after block 0's: 128 bytes of codes,
  // 64 of sketch)
  uint32_t kw0[2], kw1[2], sw[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    kw0[b] = *reinterpret_cast<const uint32_t*>(st + kSK + ko + 128 * b + 4 * q4);
    kw1[b] = *reinterpret_cast<const uint32_t*>(st + kSK + ko + 128 * b + 16 + 4 * q4);
    sw[b] = *reinterpret_cast<const uint32_t*>(st + kSS + so + 64 * b + 4 * q4);
  }
  // Norms of the 4 tokens this lane scores after the hi + lo combine (below):
  // columns 0..7 take tokens 8 q4 + [0, 4), columns 8..15 tokens 8 q4 + [4, 8).
  const int nofs = no + (c >= 8 ? 16 : 0);
  const uint4 nk = *reinterpret_cast<const uint4*>(st + kSN + nofs);
  const uint4 nr = *reinterpret_cast<const uint4*>(st + kSR + nofs);
  const uint4 nv = *reinterpret_cast<const uint4*>(st + kSVN + nofs);
  const i2_t vx0 = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) i2_t*)(st + kSV + vo));
  const i2_t vx1 = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) i2_t*)(st + kSV + vo + 16));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage may be refilled
  if constexpr (SP) issue_tile_rows(st, lane, nx.t, pos, nx.r);
  else issue_tile(st, lane, nx.t, nx.r);

  // ---- logits: S^T = K Q^T, code-bit steps then sketch steps, per 16-token block
  f4_t lm[2], qj[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const i8_t a0 = bit_nibbles(kw0[b]), a1 = bit_nibbles(kw1[b]), as = bit_nibbles(sw[b]);
    lm[b] = f4_t{0.f, 0.f, 0.f, 0.f};
    qj[b] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      lm[b] = key_product(a0, w.bq[0][ps], w.bs[0][ps], lm[b]);
      lm[b] = key_product(a1, w.bq[1][ps], w.bs[1][ps], lm[b]);
      qj[b] = key_product(as, w.bq[2][ps], w.bs[2][ps], qj[b]);
    }
  }
  // Column c < 8 holds pieces 0 and 2 of head c, column c + 8 pieces 1 and 3.
  // Each lane keeps one block and adds the partner column's part of that block:
  // columns 0..7 finish block 0, columns 8..15 block 1, both for head c % 8.
  const bool upper = c >= 8;
  float sv[4];
  float tmax = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float l_ = (upper ? lm[1][v] : lm[0][v]) + row_ror8(upper ? lm[0][v] : lm[1][v]);
    const float q_ = (upper ? qj[1][v] : qj[0][v]) + row_ror8(upper ? qj[0][v] : qj[1][v]);
    const float n = f16_to_f32((uint16_t)(&nk.x)[v]), gm = f16_to_f32((uint16_t)(&nr.x)[v]);
    const float logit = n * ((l_ + w.cst) + a.kappa * gm * fmaf(2.f, q_, -w.sqs));
    const int tok = t0 + 8 * q4 + (upper ? 4 : 0) + v;
    float s = tok < t_end && ((valid >> (tok - t0)) & 1u) ? logit * a.scale_log2 : -INFINITY;
    if ((c & 7) >= G) s = 0.f;  // columns past the group hold no head: keep them finite
    sv[v] = s;
    tmax = fmaxf(tmax, s);
  }
  tmax = fmaxf(tmax, row_ror8(tmax));
  tmax = max_xor16(tmax);
  tmax = max_xor32(tmax);
  const bool bump = tmax > w.m_run + 8.f;
  const float m_new = bump ? tmax : w.m_run;
  const float alpha = bump ? __builtin_amdgcn_exp2f(w.m_run - m_new) : 1.f;
  float psum = 0.f, pv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float p = __builtin_amdgcn_exp2f(sv[v] - m_new);
    pv[v] = p * f16_to_f32((uint16_t)(&nv.x)[v]);
    psum += p;
  }
  // this lane's 4 weights P' as fp16 pairs (tokens 0 and 2, 1 and 3 of its 4),
  // rounded to nearest (a truncating pack would bias every weight low)
  const uint32_t own02 = __builtin_bit_cast(uint32_t, h2_t{(_Float16)pv[0], (_Float16)pv[2]});
  const uint32_t own13 = __builtin_bit_cast(uint32_t, h2_t{(_Float16)pv[1], (_Float16)pv[3]});
  w.l_run = w.l_run * alpha + psum;
  w.m_run = m_new;
  // PV A operand of row c (head c for c < 8): tokens 8 q4 + [0, 8) = this lane's
  // 4 and the partner column's 4 in the k-slot order of levels8 (0, 2, 4, 6, 1,
  // 3, 5, 7); rows 8..15 are not heads and are discarded
  h8_t pa;
  {
    const uint32_t oth02 = row_ror8(own02), oth13 = row_ror8(own13);
    pa = __builtin_bit_cast(h8_t, upper ? uint4{oth02, own02, oth13, own13} : uint4{own02, oth02, own13, oth13});
  }
  if (__ballot(bump && c < G)) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, (4 * q4 + v) & 15);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) w.o[nt][v] *= av;
    }
  }
  // ---- values: N-tile nt = 2 chunk + parity; column c <-> channel 32 chunk + 2 c + parity,
  // whose code is bits [2 parity, 2 parity + 2) of each nibble (nibble n = token 8 q4 + n)
  const uint32_t vx[4] = {(uint32_t)vx0[0], (uint32_t)vx0[1], (uint32_t)vx1[0], (uint32_t)vx1[1]};
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int nt = 2 * ch + par;
      w.o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, levels8(vx[ch], 2 * par, k.t_lo, k.t_hi), w.o[nt], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

#ifndef KVQ_TURBO_WAVES_PER_EU
#define KVQ_TURBO_WAVES_PER_EU 3  // waves per SIMD the register budget is cut for
#endif

// PAGED: token rows in pool pages named by the block table, resources per tile.
// SPARSE (contiguous caches): split slot i reads position a.sel[b][t_begin + i],
// staged in LDS; slots without a valid position are masked.
template <int G, bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(KVQ_TURBO_WAVES_PER_EU, KVQ_TURBO_WAVES_PER_EU))) decode_turbo_kernel(TurboDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t stA[4][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stB[4][kStage];
  __shared__ float sm_o[4][G][129];
  float (*sm_m)[16] = reinterpret_cast<float (*)[16]>(&stB[0][0]);
  float (*sm_l)[16] = reinterpret_cast<float (*)[16]>(&stB[0][0] + 4 * 16 * sizeof(float));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.H + h;
  // several queries per sequence: this launch takes query j = a.qj of a.nq,
  // which sees the first L - (nq - 1 - j) tokens
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  const size_t qrow0 = ((size_t)b * a.nq + a.qj) * a.Hq;  // its first query / output row
  // packed tokens [t_lo, L - recent) this query sees; a split none of whose
  // tokens reach t_lo has no work (its tiles would be masked whole)
  const int t_begin = (a.t_lo & ~31) + split * a.per_split;
  const int t_stop = min(L - (a.nq - 1 - a.qj), max(a.t_lo, L - a.recent));
  const int t_end = t_stop <= a.t_lo ? t_begin : min(t_stop, t_begin + a.per_split);
  const int q4 = lane >> 4, c = lane & 15;

  Consts k;
  {
    k.a0 = a.levels[0];
    k.t_lo = 0;
    k.t_hi = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)a.levels[c]);
      k.t_lo |= (hb & 0xFFu) << (8 * c);
      k.t_hi |= (hb >> 8) << (8 * c);
    }
  }
  WaveState<G> w;
  {
    // prepared query: [R q (128) | S R q (128)] fp32 per query head, and the FP8
    // pieces of the key-product operands (layout of prepared_query_pieces)
    const int head = c % 8;
    const bool live = head < G;
    const size_t qrow = qrow0 + (size_t)h * G + (live ? head : 0);
    const float* qp = a.q + qrow * 256;
    const uint8_t* pc = a.qpieces + qrow * kTurboPieceBytes;
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        const uint8_t* base = pc + (m * 4 + 2 * ps + (c >> 3)) * 144;
        const uint4 lo4 = *reinterpret_cast<const uint4*>(base + 32 * q4);
        const uint2 hi2 = *reinterpret_cast<const uint2*>(base + 32 * q4 + 16);
        w.bq[m][ps] = live ? i8_t{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w, (int)hi2.x, (int)hi2.y, 0, 0}
                           : i8_t{0, 0, 0, 0, 0, 0, 0, 0};
        w.bs[m][ps] = live ? (int)base[128 + q4] : 127;
      }
    // per-head sums over all 128 entries: this lane's 32 + the other quarters'
    float sr = 0.f, ss = 0.f;
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      sr += live ? qp[32 * q4 + x] : 0.f;
      ss += live ? qp[128 + 32 * q4 + x] : 0.f;
    }
    sr += __shfl_xor(sr, 16);
    sr += __shfl_xor(sr, 32);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    w.cst = k.a0 * sr;
    w.sqs = ss;
  }
  w.m_run = -INFINITY;
  w.l_run = 0.f;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) w.o[nt] = f4_t{0.f, 0.f, 0.f, 0.f};

  // resources over nrows token rows from row0 (nrows 0: every read is zeros)
  auto res_at = [&](size_t row0, int nrows) {
    return Res{rsrc(a.k_codes + row0 * 32, (size_t)nrows * 32), rsrc(a.k_sketch + row0 * 16, (size_t)nrows * 16),
               rsrc(a.k_norm + row0, (size_t)nrows * 2),        rsrc(a.k_rnorm + row0, (size_t)nrows * 2),
               rsrc(a.v_codes + row0 * 32, (size_t)nrows * 32), rsrc(a.v_norm + row0, (size_t)nrows * 2),
               nrows * 32};
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
    return t >= a.t_lo ? ~0u : a.t_lo - t >= 32 ? 0u : ~0u << (a.t_lo - t);  // below t_lo: the bf16 sink's
  };
  uint8_t* sa = stA[wave];
  uint8_t* sb = stB[wave];
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
  int t0 = t_begin + wave * 32;
  {
    const TileSrc s0 = tile_or_none(t0), s1 = tile_or_none(t0 + 128);
    if constexpr (SPARSE) {
      issue_tile_rows(sa, lane, s0.t, spos, s0.r);
      issue_tile_rows(sb, lane, s1.t, spos, s1.r);
    } else {
      issue_tile(sa, lane, s0.t, s0.r);
      issue_tile(sb, lane, s1.t, s1.r);
    }
  }
  for (; t0 < t_end; t0 += 256) {
    tile_step<G, SPARSE>(w, sa, lane, t0, t_end, tile_or_none(t0 + 256), a, k, spos, valid_of(t0));
    tile_step<G, SPARSE>(w, sb, lane, t0 + 128, t_end, tile_or_none(t0 + 384), a, k, spos, valid_of(t0 + 128));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---------------- combine the four waves, write this split's partial result
  __syncthreads();
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int q4e = lane_e >> 4, ce = lane_e & 15;
  const int tid_e = wave * 64 + lane_e;
  float l_run = w.l_run;
  l_run += row_ror8(l_run);  // the two column halves scored disjoint tokens
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (q4e == 0) {
    sm_m[wave][ce] = w.m_run;
    sm_l[wave][ce] = l_run;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int hh = 4 * q4e + v;
    if (hh < G) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int ch = 32 * (nt >> 1) + 2 * ce + (nt & 1);
        sm_o[wave][hh][ch] = w.o[nt][v];
      }
    }
  }
  __syncthreads();
  const size_t row0 = qrow0 + (size_t)h * G;
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
    float* p = a.part + ((row0 + hh) * a.part_splits + split) * 130;
    p[2 + ch] = O;
    if (ch == 0) {
      p[0] = M;
      p[1] = Ls;
    }
  }
}

}  // namespace

namespace {
template <bool PAGED, bool SPARSE = false>
int launch_turbo(const TurboDecodeArgs& a, int B, int G, hipStream_t st) {
  dim3 grid(a.splits, a.H, B);
  switch (G) {
    case 1: decode_turbo_kernel<1, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 2: decode_turbo_kernel<2, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 4: decode_turbo_kernel<4, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 8: decode_turbo_kernel<8, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    default: return KV_EUNSUPPORTED;
  }
  return KV_OK;
}
}  // namespace

int launch_decode_turbo(const TurboDecodeArgs& a, int B, int G, hipStream_t st) {
  if (a.sel) return a.pm.table ? KV_EUNSUPPORTED : launch_turbo<false, true>(a, B, G, st);
  return a.pm.table ? launch_turbo<true>(a, B, G, st) : launch_turbo<false>(a, B, G, st);
}

}  // namespace kvq
