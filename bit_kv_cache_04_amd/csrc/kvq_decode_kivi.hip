// Decode attention on the matrix cores (gfx950) for KIVI-2 caches with D = 64
// or 128 channels: keys quantised per channel over groups of 32 tokens, values
// per token over groups of 32 channels, 2-bit codes with fp32 scale and zero
// (page "TurboQuant vs OSCAR vs EpiCache", section "quantization frontiers",
// KIVI paragraph).
//
// One workgroup = 4 waves over one (sequence, KV head, context split); each
// wave streams its own 32-token tiles (one key group each) from HBM into a
// private two-stage LDS ring with direct-to-LDS loads and keeps the online
// softmax of 16 (query, head) columns.  Per tile and wave:
//   keys    S_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c for the group's scale
//           s and zero z.  The codes (0..3) are exact fp16 operands, q_c s_c an
//           exact fp16 hi + lo pair: D / 8 v_mfma_f32_16x16x32_f16 (rows =
//           tokens, columns = heads); the zero term is an fp32 sum per column.
//   softmax per column = per lane column, the reference max moving only when
//           a tile max passes it by 2^8.
//   values  v_tc = code_tc s_t + z_t for the token's 32-channel group, made in
//           fp32 and rounded once to fp16 (nearest) as the B operand of D / 16
//           PV products.
// With fewer than 16 (query, head) pairs per launch the 16 columns carry each
// pair S = 16 / P times (P pair slots, S at most D / 32), column c taking pair
// c % P over the channel part c / P only, and rotations within each 16-lane row
// add the parts: each lane scales D / S query channels per tile instead of D.
// Tokens of a sequence's incomplete last group are not coded yet (their keys
// wait in staging); they take one more split in fp32: on small grids a last
// column of workgroups of the same launch, else the general kernel.
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_kernels.h"

namespace kvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

namespace {

constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcFlags);
}

// Stage of one 32-token tile of a D-channel cache (bytes): key codes (D / 4 per
// token row), the group's D key scales and zeros, value codes, and the tokens'
// value scales and zeros (D / 32 per token).
template <int D>
struct Stage {
  static constexpr int kKc = 0, kKs = 8 * D, kKz = 12 * D, kVc = 16 * D, kVs = 24 * D, kVz = 28 * D, kBytes = 32 * D;
  static constexpr int kDma = D == 128 ? 10 : 8;  // direct-to-LDS loads per tile
};

struct Res {
  __amdgpu_buffer_rsrc_t kc, ks, kz, vc, vs, vz;
};

// The tile from token t0 (a multiple of 32; t0 = capacity: no tile, every load
// reads past its resource and writes zeros): lane l moves bytes [s l, s l + s)
// of each chunk (D = 128: 16-byte code chunks; D = 64: 4-byte pieces throughout).
template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* st, int lane, int t0, const Res& r) {
  using G = Stage<D>;
  const int go = (t0 >> 5) * (4 * D) + lane * 4, vo = t0 * (D / 8) + lane * 4;
  if constexpr (D == 128) {
    const int co = t0 * 32 + lane * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + G::kKc), 16, co, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + G::kVc), 16, co, 0, 0, 0);
  } else {
    const int co = t0 * 16 + lane * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + G::kKc), 4, co, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kc, (lds_ptr_t)(st + G::kKc + 256), 4, co + 256, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + G::kVc), 4, co, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vc, (lds_ptr_t)(st + G::kVc + 256), 4, co + 256, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {  // 4 D bytes each: 256 per load
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ks, (lds_ptr_t)(st + G::kKs + 256 * i), 4, go + 256 * i, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.kz, (lds_ptr_t)(st + G::kKz + 256 * i), 4, go + 256 * i, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vs, (lds_ptr_t)(st + G::kVs + 256 * i), 4, vo + 256 * i, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.vz, (lds_ptr_t)(st + G::kVz + 256 * i), 4, vo + 256 * i, 0, 0, 0);
  }
}

// Codes 0..3 in nibbles as the exact fp16 values: an E2M1 nibble 0..3 is
// 0, 0.5, 1, 1.5, and the conversion's power-of-two scale 2 restores the code.
template <int SEL>
__device__ __forceinline__ h2_t code_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, SEL);
}

// 8 two-bit codes (bits 2 i, 2 i + 1 of x) into the low bits of 8 nibbles (nibble i).
__device__ __forceinline__ uint32_t spread_codes(uint32_t x) {
  uint32_t t = (x | (x << 8)) & 0x00FF00FFu;
  t = (t | (t << 4)) & 0x0F0F0F0Fu;
  return (t | (t << 2)) & 0x33333333u;
}

__device__ __forceinline__ h8_t h8_from(h2_t a, h2_t b, h2_t c, h2_t d) {
  h8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 codes (16 bits) as the fp16 A operand of a key product, in k-slot order.
__device__ __forceinline__ h8_t codes8(uint32_t x16) {
  const uint32_t n = spread_codes(x16);
  return h8_from(code_pair<0>(n), code_pair<1>(n), code_pair<2>(n), code_pair<3>(n));
}

// A-operand row c of a 16-token block holds token 4*(c%4) + c/4, so that the
// C rows 4*q4 + v of a lane quarter are the tokens 4*v + q4.
__device__ __forceinline__ int row_token(int c) { return 4 * (c & 3) + (c >> 2); }

// x of lane (l & ~15) | ((l + N) & 15), 0 < N < 16: DPP row_ror:(16 - N) (a
// rotation right by k hands lane l the value of lane l - k within its row).
template <int N>
__device__ __forceinline__ float row_fetch(float x) {
  static_assert(N > 0 && N < 16, "rotation within a 16-lane row");
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + (16 - N), 0xF, 0xF, false));
}

// Everything one wave carries across tiles.
template <int D>
struct WaveState {
  float q[D / 32][8];  // prepared query of the lane's column: its part's k-steps kp, channels 32 kk + 8 q4 + i
  float m_run, l_run;
  f4_t o[D / 16];      // O rows = columns 4 q4 + v; N-tile nt = channels (D / 16) c + nt
};

// One tile: read this lane's fragments from the stage, refill the stage from
// tile `next` once the reads have returned, then compute.  lim: the lane
// column's token limit; t_full: a tile below it is whole for every column.
// S: channel parts per pair (column c: pair c % (16 / S), k-steps of part c / (16 / S)).
template <int D, int S>
__device__ __forceinline__ void tile_step(WaveState<D>& w, uint8_t* st, int lane, int t0, int t_full, int lim,
                                          int next, const Res& r, const MfmaDecodeArgs& a) {
  using G = Stage<D>;
  constexpr int NK = D / 32, NT = D / 16, CL = D / 16;  // k-steps, value N-tiles, value channels per lane
  constexpr int P = 16 / S, KP = NK / S;                  // pair slots, k-steps per part
  static_assert(KP >= 1, "a part holds at least one k-step");
  const int q4 = lane >> 4, c = lane & 15;
  const int part = c / P;
  const int pc = c % P;
  // This stage's tile has landed once at most the other stage's refill is
  // outstanding (explicit: the compiler's own wait for loads into LDS is not
  // placed reliably across the loop back-edge).
  static_assert(G::kDma < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | G::kDma);
  // key codes: row c of block blk, channels 32 kk + 8 q4 + [0, 8) (bytes 8 kk + 2 q4, +1)
  uint32_t kx[2][NK];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    int ko = (16 * blk + row_token(c)) * (D / 4) + 2 * q4;
    asm volatile("" : "+v"(ko));
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kx[blk][kk] = *reinterpret_cast<const uint16_t*>(st + G::kKc + ko + 8 * kk);
  }
  // the group's key scales and zeros of the lane's channels: 8 per k-step of its part
  float ks[KP][8], kz[KP][8];
#pragma unroll
  for (int kk = 0; kk < KP; ++kk) {
    const int ch = 32 * (KP * part + kk) + 8 * q4;
    const float4* ps = reinterpret_cast<const float4*>(st + G::kKs + 4 * ch);
    const float4* pz = reinterpret_cast<const float4*>(st + G::kKz + 4 * ch);
    const float4 s0 = ps[0], s1 = ps[1], z0 = pz[0], z1 = pz[1];
    ks[kk][0] = s0.x; ks[kk][1] = s0.y; ks[kk][2] = s0.z; ks[kk][3] = s0.w;
    ks[kk][4] = s1.x; ks[kk][5] = s1.y; ks[kk][6] = s1.z; ks[kk][7] = s1.w;
    kz[kk][0] = z0.x; kz[kk][1] = z0.y; kz[kk][2] = z0.z; kz[kk][3] = z0.w;
    kz[kk][4] = z1.x; kz[kk][5] = z1.y; kz[kk][6] = z1.z; kz[kk][7] = z1.w;
  }
  // the lane's 8 tokens j (tile row 16 (j / 4) + 4 (j % 4) + q4): value codes of
  // channels CL c .. CL c + CL - 1 (CL / 4 bytes from CL c / 4) and the scale and
  // zero of their group CL c / 32
  uint32_t vx[8];
  float vs[8], vz[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = 16 * (j >> 2) + 4 * (j & 3) + q4;
    if constexpr (CL == 8) vx[j] = *reinterpret_cast<const uint16_t*>(st + G::kVc + tok * (D / 4) + 2 * c);
    else vx[j] = st[G::kVc + tok * (D / 4) + c];
    const int vg = tok * (D / 8) + 4 * ((CL * c) >> 5);
    vs[j] = *reinterpret_cast<const float*>(st + G::kVs + vg);
    vz[j] = *reinterpret_cast<const float*>(st + G::kVz + vg);
  }
  // the reads above must have returned before the stage is overwritten
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  issue_tile<D>(st, lane, next, r);

  // ---------------- keys: B = q s as an fp16 hi + lo pair, A = the codes.  The
  // lane scales its part's k-steps only (the others hold zeros): k-step kk of
  // part u is kk = KP u + kp.
  h8_t bh[NK], bl[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    bh[kk] = h8_t{};
    bl[kk] = h8_t{};
  }
  float zs = 0.f;
  h8_t ph[KP], pl[KP];
#pragma unroll
  for (int kp = 0; kp < KP; ++kp) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float x0 = w.q[kp][i] * ks[kp][i], x1 = w.q[kp][i + 1] * ks[kp][i + 1];
      const h2_t hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
      const h2_t lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(x0 - (float)hi[0], x1 - (float)hi[1]));
      ph[kp][i] = hi[0];
      ph[kp][i + 1] = hi[1];
      pl[kp][i] = lo[0];
      pl[kp][i + 1] = lo[1];
      zs = __builtin_fmaf(w.q[kp][i], kz[kp][i], zs);
      zs = __builtin_fmaf(w.q[kp][i + 1], kz[kp][i + 1], zs);
    }
  }
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (kk / KP == part) {  // place the part's operands at their k-steps
      bh[kk] = ph[kk % KP];
      bl[kk] = pl[kk % KP];
    }
  }
  zs += __shfl_xor(zs, 16);
  zs += __shfl_xor(zs, 32);  // the column part's zero term, in every lane of the column
  f4_t sacc[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    f4_t acc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const h8_t A = codes8(kx[blk][kk]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[kk], acc, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {  // the pair's logit: its parts summed along the row
      float x = acc[v] + zs;
      if constexpr (S >= 2) x += row_fetch<P>(x);
      if constexpr (S >= 4) x += row_fetch<2 * P>(x);
      acc[v] = x;
    }
    sacc[blk] = acc;
  }

  // ---------------- online softmax (this lane: column c, tokens t0 + 16 blk + 4 v + q4)
  float sv[8];
  float tmax = -INFINITY;
  if (t0 + 32 <= t_full) {  // a whole tile for every column: nothing to mask
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[4 * blk + v] = sacc[blk][v] * a.scale_log2;
        tmax = fmaxf(tmax, sv[4 * blk + v]);
      }
  } else {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = t0 + 16 * blk + 4 * v + q4;
        const float sx = tok < lim ? sacc[blk][v] * a.scale_log2 : -INFINITY;
        sv[4 * blk + v] = sx;
        tmax = fmaxf(tmax, sx);
      }
  }
  tmax = max_xor16(tmax);
  tmax = max_xor32(tmax);
  const bool bump = tmax > w.m_run + 8.f;
  const float m_new = bump ? tmax : w.m_run;
  const float alpha = bump ? __builtin_amdgcn_exp2f(w.m_run - m_new) : 1.f;
  const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // a column with no visible token yet
  float psum = 0.f;
  h8_t pf;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(sv[j] - m_ref);
    psum += p;
    pf[j] = (_Float16)p;
  }
  w.l_run = w.l_run * alpha + psum;
  w.m_run = m_new;
  // O rows are columns 4 q4 + v; column hh's alpha lives in lane hh (quarter 0)
  if (__ballot(bump && pc < a.ncol)) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float av = __shfl(alpha, (4 * q4 + v) & 15);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w.o[nt][v] *= av;
    }
  }

  // ---------------- values: B of N-tile nt = channel CL c + nt over the lane's 8 tokens.
  // e_j byte k = nibble k of token j's codes (channels CL c + 2k, CL c + 2k + 1);
  // X[p] byte k pairs channel CL c + 2k of tokens 2p and 2p + 1, Y[p] channel CL c + 2k + 1.
  uint32_t X[4], Y[4];
  auto nibble_bytes = [](uint32_t x) {
    if constexpr (CL == 8) {
      const uint32_t t = (x | (x << 8)) & 0x00FF00FFu;
      return (t | (t << 4)) & 0x0F0F0F0Fu;
    } else {
      return (x | (x << 4)) & 0x0F0Fu;
    }
  };
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t e0 = nibble_bytes(vx[2 * p]), e1 = nibble_bytes(vx[2 * p + 1]);
    X[p] = (e0 & 0x03030303u) | ((e1 & 0x03030303u) << 4);
    Y[p] = ((e0 >> 2) & 0x03030303u) | ((e1 << 2) & 0x30303030u);
  }
  // tokens 2 p, 2 p + 1 of byte K of x: code s + z in fp32, rounded once to fp16
  auto vpair = [&](uint32_t x, int p, auto K) {
    const auto c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 2.0f, decltype(K)::value);
    h2_t r;
    r[0] = (_Float16)__builtin_fmaf(c2[0], vs[2 * p], vz[2 * p]);
    r[1] = (_Float16)__builtin_fmaf(c2[1], vs[2 * p + 1], vz[2 * p + 1]);
    return r;
  };
#define KVQ_KIVI_PV(K)                                                                                          \
  {                                                                                                             \
    constexpr std::integral_constant<int, K> k{};                                                               \
    const h8_t bx = h8_from(vpair(X[0], 0, k), vpair(X[1], 1, k), vpair(X[2], 2, k), vpair(X[3], 3, k));        \
    w.o[2 * K] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, bx, w.o[2 * K], 0, 0, 0);                           \
    const h8_t by = h8_from(vpair(Y[0], 0, k), vpair(Y[1], 1, k), vpair(Y[2], 2, k), vpair(Y[3], 3, k));        \
    w.o[2 * K + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, by, w.o[2 * K + 1], 0, 0, 0);                   \
  }
  KVQ_KIVI_PV(0)
  KVQ_KIVI_PV(1)
  if constexpr (CL == 8) {
    KVQ_KIVI_PV(2)
    KVQ_KIVI_PV(3)
  }
#undef KVQ_KIVI_PV
  // keep the scheduler from interleaving two tiles (register pressure)
  __builtin_amdgcn_sched_barrier(0);
}

// The staged tokens [kstage, L) of a sequence's incomplete key group (keys still
// fp32 in staging, token t in row t mod 32; values coded) for the launch's
// pairs, written as partial split a.splits: fp32 logits, softmax and value sums.
// kbuf: 32 x D floats of LDS, sbuf: 16 x 32 + 32 floats.
template <int D>
__device__ void staged_tail(const MfmaDecodeArgs& a, int b, int h, float* kbuf, float* sbuf) {
  const int tid = threadIdx.x;
  const size_t bh = (size_t)b * a.H + h;
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  const float* stg = a.k_stage + bh * (4 + 32 * D);
  const int t0 = reinterpret_cast<const int*>(stg)[0] & ~31;
  const int n = max(0, L - t0);  // below 32: the coded groups end at t0
  float* sm = sbuf;              // [16][32] logits, then weights
  float* mm = sbuf + 16 * 32;    // [16] max, [16] sum
  for (int e = tid; e < n * D; e += 256) kbuf[e] = stg[4 + ((t0 + e / D) & 31) * D + e % D];
  __syncthreads();
  for (int e = tid; e < a.ncol * 32; e += 256) {
    const int pc = e >> 5, i = e & 31, pair = a.c0 + pc, j = pair / a.gr;
    float x = -INFINITY;
    if (i < n && t0 + i < L - (a.nq - 1 - j)) {  // query j sees the first L - (nq - 1 - j) tokens
      const size_t qrow = ((size_t)b * a.nq + j) * a.Hq + (size_t)h * a.gr + pair % a.gr;
      const float* q = static_cast<const float*>(a.q) + qrow * D;
      float acc = 0.f;
#pragma unroll 4
      for (int ch = 0; ch < D; ++ch) acc = fmaf(q[ch], kbuf[i * D + ch], acc);
      x = acc * a.scale_log2;
    }
    sm[e] = x;
  }
  __syncthreads();
  if (tid < a.ncol) {
    float M = -INFINITY, l = 0.f;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) M = fmaxf(M, sm[tid * 32 + i]);
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
      const float p = M == -INFINITY ? 0.f : exp2f(sm[tid * 32 + i] - M);
      sm[tid * 32 + i] = p;
      l += p;
    }
    mm[tid] = M;
    mm[16 + tid] = l;
  }
  // the staged tokens' values, dequantised in place of the keys
  for (int e = tid; e < n * D; e += 256) {
    const size_t row = bh * a.cap + t0 + e / D;
    const int ch = e % D;
    const uint32_t code = (a.v_codes[row * (D / 4) + ch / 4] >> (2 * (ch & 3))) & 3u;
    const size_t g = row * (D / 32) + ch / 32;
    kbuf[e] = fmaf((float)code, a.v_scale_f[g], a.v_zero_f[g]);
  }
  __syncthreads();
  for (int e = tid; e < a.ncol * D; e += 256) {
    const int pc = e / D, ch = e % D, pair = a.c0 + pc;
    float O = 0.f;
#pragma unroll 4
    for (int i = 0; i < n; ++i) O = fmaf(sm[pc * 32 + i], kbuf[i * D + ch], O);
    const size_t row = ((size_t)b * a.nq + pair / a.gr) * a.Hq + (size_t)h * a.gr + pair % a.gr;
    float* p = a.part + (row * a.part_splits + a.splits) * (D + 2);
    p[2 + ch] = O;
    if (ch == 0) {
      p[0] = mm[pc];
      p[1] = mm[16 + pc];
    }
  }
}

// TAIL: the grid has one more column of workgroups, which take the staged
// tokens (staged_tail); else the caller runs them separately.
template <int D, int S, bool TAIL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_kivi_kernel(MfmaDecodeArgs a) {
  constexpr int NK = D / 32, NT = D / 16, CL = D / 16;  // k-steps, value N-tiles, value channels per lane
  constexpr int P = 16 / S, KP = NK / S;                  // pair slots, k-steps per channel part
  // LDS stages per wave, as separate arrays so that the compiler can tell which
  // stage a direct-to-LDS load writes
  __shared__ __attribute__((aligned(16))) uint8_t stA[4][Stage<D>::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stB[4][Stage<D>::kBytes];
  // the waves' running max / sum are combined through stage-B memory, their
  // outputs through stage-A memory, 8 columns x D floats per wave at a time
  float (*sm_o)[8][D] = reinterpret_cast<float (*)[8][D]>(&stA[0][0]);
  float (*sm_m)[16] = reinterpret_cast<float (*)[16]>(&stB[0][0]);
  float (*sm_l)[16] = reinterpret_cast<float (*)[16]>(&stB[0][0] + 4 * 16 * sizeof(float));
  static_assert(sizeof(float) * 4 * 8 * D <= sizeof(stA), "stage A too small");
  static_assert(2 * 4 * 16 * sizeof(float) <= sizeof(stB), "stage B too small");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  static_assert(sizeof(float) * 32 * D <= sizeof(stA) && sizeof(float) * (16 * 32 + 32) <= sizeof(stB),
                "the staged tail fits the stages");
  if constexpr (TAIL) {
    if (split == a.splits) {  // the grid's last column: the staged tokens
      staged_tail<D>(a, b, h, reinterpret_cast<float*>(&stA[0][0]), reinterpret_cast<float*>(&stB[0][0]));
      return;
    }
  }
  const size_t bh = (size_t)b * a.H + h;
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap);
  // the coded tokens end at the first token of the incomplete group
  const int kstage = reinterpret_cast<const int*>(a.k_stage)[bh * (4 + 32 * D)] & ~31;
  const int t_begin = split * a.per_split;
  const int t_end = min(min(L, kstage), t_begin + a.per_split);
  // column c is (query j, head g) pair c0 + c % P; query j sees the first L - (nq - 1 - j) tokens
  const int c = lane & 15, q4 = lane >> 4;
  const int pc = c % P, part = c / P;
  const int lim = min(t_end, L - (a.nq - 1 - (a.c0 + pc) / a.gr));
  const int t_full = min(t_end, L - (a.nq - 1 - a.c0 / a.gr));


  // Buffer resources over this (sequence, KV head)'s rows: a read past the end
  // of a resource returns zeros instead of faulting (a missing tile reads past
  // the end).
  const size_t row0 = bh * a.cap;
  const Res r{rsrc(a.k_codes + row0 * (D / 4), (size_t)a.cap * (D / 4)),
              rsrc(reinterpret_cast<const uint8_t*>(a.k_scale_f) + row0 / 32 * (4 * D), (size_t)a.cap / 32 * (4 * D)),
              rsrc(reinterpret_cast<const uint8_t*>(a.k_zero_f) + row0 / 32 * (4 * D), (size_t)a.cap / 32 * (4 * D)),
              rsrc(a.v_codes + row0 * (D / 4), (size_t)a.cap * (D / 4)),
              rsrc(reinterpret_cast<const uint8_t*>(a.v_scale_f) + row0 * (D / 8), (size_t)a.cap * (D / 8)),
              rsrc(reinterpret_cast<const uint8_t*>(a.v_zero_f) + row0 * (D / 8), (size_t)a.cap * (D / 8))};
  auto tile_or_none = [&](int t) { return t < t_end ? t : a.cap; };

  uint8_t* sa = stA[wave];
  uint8_t* sb = stB[wave];
  int t0 = t_begin + wave * 32;
  // The first two tiles are issued before the sequence length, the staging
  // marker and the query have arrived: a tile past the end is read from the
  // cache's own rows and never used, or has all its tokens masked.
  issue_tile<D>(sa, lane, t0 < a.cap ? t0 : a.cap, r);
  issue_tile<D>(sb, lane, t0 + 128 < a.cap ? t0 + 128 : a.cap, r);
  WaveState<D> w;
  {
    const int pair = a.c0 + pc;
    const bool live = pc < a.ncol;
    const size_t qrow = ((size_t)b * a.nq + (live ? pair / a.gr : 0)) * a.Hq + (size_t)h * a.gr + (live ? pair % a.gr : 0);
    const float* qp = static_cast<const float*>(a.q) + qrow * D + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      if (kk >= KP) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w.q[kk][i] = 0.f;
        continue;
      }
      const int k = KP * part + kk;
      const float4 x0 = *reinterpret_cast<const float4*>(qp + 32 * k);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + 32 * k + 4);
      w.q[kk][0] = live ? x0.x : 0.f; w.q[kk][1] = live ? x0.y : 0.f;
      w.q[kk][2] = live ? x0.z : 0.f; w.q[kk][3] = live ? x0.w : 0.f;
      w.q[kk][4] = live ? x1.x : 0.f; w.q[kk][5] = live ? x1.y : 0.f;
      w.q[kk][6] = live ? x1.z : 0.f; w.q[kk][7] = live ? x1.w : 0.f;
    }
  }
  w.m_run = -INFINITY;
  w.l_run = 0.f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) w.o[nt] = f4_t{0.f, 0.f, 0.f, 0.f};
  for (; t0 < t_end; t0 += 256) {
    // the second tile of a pair may lie past t_end: all its tokens are masked
    tile_step<D, S>(w, sa, lane, t0, t_full, lim, tile_or_none(t0 + 256), r, a);
    tile_step<D, S>(w, sb, lane, t0 + 128, t_full, lim, tile_or_none(t0 + 384), r, a);
  }
  // drain the refills still in flight before the waves' LDS is reused or the wave exits
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---------------- combine the four waves, write this split's partial result
  __syncthreads();  // every wave is done with its stages before they hold outputs
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int q4e = lane_e >> 4, ce = lane_e & 15;
  const int tid_e = wave * 64 + lane_e;
  float l_run = w.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (q4e == 0) {
    sm_m[wave][ce] = w.m_run;
    sm_l[wave][ce] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {  // columns 8 r .. 8 r + 7 (rows 4 q4 + v of lane quarters 2 r, 2 r + 1)
    if (r) __syncthreads();       // the previous round's outputs are read
    if ((q4e >> 1) == r) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sm_o[wave][4 * (q4e & 1) + v][CL * ce + nt] = w.o[nt][v];
      }
    }
    __syncthreads();
    for (int e = tid_e; e < 8 * D; e += 256) {
      const int hh = 8 * r + e / D, ch = e % D;
      if (hh >= P || hh >= a.ncol) continue;  // a column with no query, or a pair's copy
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][hh]);
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = sm_m[ww][hh];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        Ls += f * sm_l[ww][hh];
        O += f * sm_o[ww][hh - 8 * r][ch];
      }
      const int pc = a.c0 + hh;
      const size_t row = ((size_t)b * a.nq + pc / a.gr) * a.Hq + (size_t)h * a.gr + pc % a.gr;
      float* p = a.part + (row * a.part_splits + split) * (D + 2);
      p[2 + ch] = O;
      if (ch == 0) {
        p[0] = M;
        p[1] = Ls;
      }
    }
  }
}

}  // namespace

template <bool TAIL>
static void launch_kivi(const MfmaDecodeArgs& a, int d, int B, hipStream_t st) {
  const dim3 grid(a.splits + (TAIL ? 1 : 0), a.H, B);
  if (d == 128) {
    if (a.ncol <= 4) decode_kivi_kernel<128, 4, TAIL><<<grid, 256, 0, st>>>(a);
    else if (a.ncol <= 8) decode_kivi_kernel<128, 2, TAIL><<<grid, 256, 0, st>>>(a);
    else decode_kivi_kernel<128, 1, TAIL><<<grid, 256, 0, st>>>(a);
  } else {
    if (a.ncol <= 8) decode_kivi_kernel<64, 2, TAIL><<<grid, 256, 0, st>>>(a);
    else decode_kivi_kernel<64, 1, TAIL><<<grid, 256, 0, st>>>(a);
  }
}

int launch_decode_kivi(const MfmaDecodeArgs& a, int d, bool tail, int B, hipStream_t st) {
  if (a.pm.table || a.sel || a.ncol < 1 || a.ncol > 16 || (d != 64 && d != 128)) return KV_EUNSUPPORTED;
  if (tail) launch_kivi<true>(a, d, B, st);
  else launch_kivi<false>(a, d, B, st);
  return KV_OK;
}

}  // namespace kvq
