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
// One workgroup = one (sequence, context split), all Hq = 32 * NW query heads,
// NW waves, one per SIMD.  Wave w owns heads [32 w, 32 w + 32) end to end: its
// query operand (144 registers) and its 32 x 512 fp32 output accumulators (256
// registers) stay in registers for the whole split.  Per 32-token tile:
//   1. the packed tile (codes, scales, RoPE) arrives by direct-to-LDS loads,
//      issued two tiles ahead;
//   2. all threads dequantise it once into a token-major tile Kt (fp16 latent,
//      bf16 RoPE); the PV operand reads it back transposed (ds_read_b64_tr_b16);
//   3. each wave computes S^T = K Q^T for its heads (36 MFMAs);
//   4. online softmax per head (each lane pair holds one head), P to fp16;
//   5. O += P V (32 MFMAs).
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
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kTile = 32;
constexpr int kLat = 512, kRope = 64;
// packed stage: codes 32 x 256 | scales 32 x 64 | RoPE 32 x 128
constexpr int kStCodes = 0, kStScale = 8192, kStRope = 10240, kStBytes = 14336;
// Kt: 32 token rows of 576 halves (fp16 latent, then bf16 RoPE), row stride
// 73 x 16 bytes.  Token t = 16 c + 8 h + 4 h2 + e (e < 4) lives in row
// kt_phys(t) = 16 c + 8 h2 + 2 e + h, chosen so that both readers see distinct
// bank groups: the QK operand (lanes of 8 read 8 rows differing in e and h) and
// the transposing PV reads (4 rows differing in e, 32 bytes each).
constexpr int kKtStride = kLat + kRope + 8;
constexpr int kRsrcFlags = 0x00020000;

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

__device__ __forceinline__ h2_t bf16x2_to_h2(uint32_t lo_hi) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(lo_hi << 16),
                                                            __uint_as_float(lo_hi & 0xFFFF0000u)));
}

// Row rho of the QK A operand holds token qk_token(rho) (bits 2 and 3 of rho
// swapped): then the result rows a lane holds (i % 4 + 8 (i / 4) + 4 (lane / 32),
// i = 0..15) are the tokens 16 (i / 8) + 8 (lane / 32) + i % 8, exactly the
// k-slots that lane supplies as the A operand of the two 16-token PV products.
__device__ __forceinline__ int qk_token(int rho) { return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

__device__ __forceinline__ int kt_phys(int t) {
  return (t & 16) | ((t & 4) << 1) | ((t & 3) << 1) | ((t >> 3) & 1);
}

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4_t* lds_s4_ptr;

// Transposing LDS read: within each 16-lane group, lane i gets element i % 4 of
// the 8-byte chunks addressed by lanes 4 e + i / 4, e = 0..3.
__device__ __forceinline__ s4_t read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(p));
}

// s_waitcnt immediate that waits for vmcnt <= n and nothing else
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

struct Res {
  __amdgpu_buffer_rsrc_t codes, scale, rope;
};

// A tile's loads: resources over its page's token rows (a contiguous cache: the
// sequence's rows) and its first row in them.
struct TileSrc {
  Res r;
  int t;
};

// Direct-to-LDS loads of one packed tile, spread evenly over the NW waves
// (32 / NW loads each).  The token offset rides in the range-checked VGPR
// offset: a tile at or past the end of the resources reads zeros.
template <int NW>
__device__ __forceinline__ void issue_tile(uint8_t* st, int wave, int lane, int t0, const Res& r) {
#pragma unroll
  for (int k = 0; k < 8 / NW; ++k) {
    const int c = wave + k * NW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.codes, (lds_ptr_t)(st + kStCodes + c * 1024), 16,
                                             t0 * 256 + c * 1024 + lane * 16, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 8 / NW; ++k) {
    const int c = wave + k * NW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.scale, (lds_ptr_t)(st + kStScale + c * 256), 4,
                                             t0 * 64 + c * 256 + lane * 4, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 16 / NW; ++k) {
    const int c = wave + k * NW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rope, (lds_ptr_t)(st + kStRope + c * 256), 4,
                                             t0 * 128 + c * 256 + lane * 4, 0, 0, 0);
  }
}

// Sparse decode: the tile's slots read the staged positions pos[rel .. rel + 32)
// (-1: none; rel < 0: no tile), each lane its own token row of the chunk it
// loads (as issue_tile: codes and scales 4 c + lane / 16, RoPE 2 c + lane / 32).
// A missing position reads past the end of the resources: zeros.
template <int NW>
__device__ __forceinline__ void issue_tile_sparse(uint8_t* st, int wave, int lane, int rel, const int* pos,
                                                  const Res& r) {
  auto tok = [&](int slot) { return rel < 0 ? -1 : pos[rel + slot]; };
#pragma unroll
  for (int k = 0; k < 8 / NW; ++k) {
    const int c = wave + k * NW;
    const int p = tok(4 * c + (lane >> 4));
    const uint32_t oc = p < 0 ? 0xFFFFFFFFu : (uint32_t)p * 256u + (lane & 15) * 16;
    const uint32_t os = p < 0 ? 0xFFFFFFFFu : (uint32_t)p * 64u + (lane & 15) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.codes, (lds_ptr_t)(st + kStCodes + c * 1024), 16, oc, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.scale, (lds_ptr_t)(st + kStScale + c * 256), 4, os, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 16 / NW; ++k) {
    const int c = wave + k * NW;
    const int p = tok(2 * c + (lane >> 5));
    const uint32_t orp = p < 0 ? 0xFFFFFFFFu : (uint32_t)p * 128u + (lane & 31) * 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rope, (lds_ptr_t)(st + kStRope + c * 256), 4, orp, 0, 0, 0);
  }
}

// o *= f for one accumulator held in an AGPR, without the compiler staging the
// whole accumulator array through arch VGPRs.
__device__ __forceinline__ void scale_acc(float& x, float f) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(t)
               : "v"(f));
}

// PAGED: token rows in pool pages named by the block table, resources per tile.
// SPARSE (contiguous caches): the split's slots read the positions a.sel names,
// staged in LDS; slots without a valid position are masked.
template <int NW, bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(1, 1))) decode_latent_kernel(MfmaDecodeArgs a) {
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint8_t stA[kStBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stB[kStBytes];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[kTile * kKtStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x, b = blockIdx.y;
  // several queries per sequence: this launch takes query j = a.c0 of a.nq,
  // which sees the first L - (nq - 1 - j) tokens
  const int L = min(min(a.seq_lens[b], a.max_len), a.cap) - (a.nq - 1 - a.c0);
  const size_t qrow0 = ((size_t)b * a.nq + a.c0) * a.Hq;  // its first query / output row
  const int t_begin = split * a.per_split;
  const int t_end = min(L, t_begin + a.per_split);
  const int col = lane & 31, half = lane >> 5;
  static_assert(!(PAGED && SPARSE), "sparse decode reads contiguous caches");
  __shared__ int spos[SPARSE ? kLatentSparseSlots : 1];
  __shared__ uint32_t svalid[SPARSE ? kLatentSparseSlots / kTile : 1];  // bit j: slot j of the tile is valid
  if constexpr (SPARSE) {
    const int32_t* sb = a.sel + (size_t)b * a.sel_stride;
    for (int i = tid; i < a.per_split; i += NT) {
      const int slot = t_begin + i;
      int p = slot < t_end ? sb[slot] : -1;
      spos[i] = p >= 0 && p < a.cap ? p : -1;
    }
    __syncthreads();
    for (int ti = tid; ti < a.per_split / kTile; ti += NT) {
      uint32_t m = 0;
      for (int j = 0; j < kTile; ++j) m |= (spos[ti * kTile + j] >= 0 ? 1u : 0u) << j;
      svalid[ti] = m;
    }
    __syncthreads();
  }

  // ---------------- the query operand: 32 fp16 latent steps, 4 bf16 RoPE steps
  h8_t ql[32];
  b8_t qr[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow0 + 32 * wave + col) * (kLat + kRope);
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * s + 8 * half);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h2_t v = bf16x2_to_h2(wd[j]);
        ql[s][2 * j] = v[0];
        ql[s][2 * j + 1] = v[1];
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + kLat + 16 * s + 8 * half);
      qr[s] = __builtin_bit_cast(b8_t, raw);
    }
  }

  f16v_t o[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) o[n] = f16v_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // resources over nrows token rows from row0 (nrows 0: every read is zeros)
  auto res_at = [&](size_t row0, int nrows) {
    return Res{rsrc(a.k_codes + row0 * 256, (size_t)nrows * 256), rsrc(a.k_scale + row0 * 32, (size_t)nrows * 64),
               rsrc(a.rope + row0 * 64, (size_t)nrows * 128)};
  };
  const Res res = res_at((size_t)b * a.cap, a.cap);
  // a missing tile reads past the end of its resources
  auto tile_or_none = [&](int t) {
    TileSrc s;
    if constexpr (!PAGED) {
      s.r = res;
      s.t = t < t_end ? t : a.cap;
    } else {
      const int pg = t < t_end ? page_of_uniform(a.pm, b, t) : -1;
      s.r = res_at((size_t)(pg < 0 ? 0 : pg) * a.pm.tokens, pg < 0 ? 0 : a.pm.tokens);
      s.t = pg < 0 ? 0 : t & (a.pm.tokens - 1);
    }
    return s;
  };

  // the loads of tile t into stage st
  auto issue_at = [&](uint8_t* st, int t) {
    if constexpr (SPARSE) {
      issue_tile_sparse<NW>(st, wave, lane, t < t_end ? t - t_begin : -1, spos, res);
    } else {
      const TileSrc s = tile_or_none(t);
      issue_tile<NW>(st, wave, lane, s.t, s.r);
    }
  };
  issue_at(stA, t_begin);
  issue_at(stB, t_begin + kTile);

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
  constexpr int kH2 = 8 * kKtStride;   // h2 = 1: token + 4 -> row + 8
  constexpr int kC = 16 * kKtStride;   // c = 1: token + 16 -> row + 16

  for (int t0 = t_begin; t0 < t_end; t0 += 2 * kTile) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int tt = t0 + sub * kTile;
      uint8_t* st = sub == 0 ? stA : stB;
      // -------- 1. this wave's loads into this stage have landed (the other
      // stage's are still in flight); the barrier then covers every wave's, and
      // every wave is done with the previous tile's Kt
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(32 / NW));
      __syncthreads();
      // -------- 2. dequantise: item = (token quad, channel octet); a wave's lanes
      // take consecutive channel octets of one token quad
      for (int it = tid; it < 8 * 64; it += NT) {
        const int tq = it >> 6, co = it & 63;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tok = 4 * tq + k;
          const uint32_t cw = *reinterpret_cast<const uint32_t*>(st + kStCodes + tok * 256 + 4 * co);
          const h2_t sc = splat_bf16(*reinterpret_cast<const uint16_t*>(st + kStScale + tok * 64 + 2 * (co >> 1)));
          *reinterpret_cast<uint4*>(&Kt[kt_phys(tok) * kKtStride + 8 * co]) =
              uint4{__builtin_bit_cast(uint32_t, fp4x2<0>(cw) * sc), __builtin_bit_cast(uint32_t, fp4x2<1>(cw) * sc),
                    __builtin_bit_cast(uint32_t, fp4x2<2>(cw) * sc), __builtin_bit_cast(uint32_t, fp4x2<3>(cw) * sc)};
        }
      }
      for (int it = tid; it < kTile * 8; it += NT) {  // RoPE: 32 tokens x 8 x 16 bytes
        const int tok = it >> 3, part = it & 7;
        *reinterpret_cast<uint4*>(&Kt[kt_phys(tok) * kKtStride + kLat + 8 * part]) =
            *reinterpret_cast<const uint4*>(st + kStRope + tok * 128 + 16 * part);
      }
      __syncthreads();
      // -------- the stage is free: refill it two tiles ahead
      issue_at(st, tt + 2 * kTile);
      // -------- 3. S^T = K Q^T for this wave's 32 heads (two accumulation chains)
      f16v_t s = f16v_t{}, s2 = f16v_t{};
#pragma unroll
      for (int k = 0; k < 32; k += 2) {
        const h8_t kf0 = *reinterpret_cast<const h8_t*>(&Kt[ka + 16 * k]);
        const h8_t kf1 = *reinterpret_cast<const h8_t*>(&Kt[ka + 16 * k + 16]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf0, ql[k], s, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf1, ql[k + 1], s2, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
        const b8_t kf0 = *reinterpret_cast<const b8_t*>(&Kt[ka + kLat + 16 * k]);
        const b8_t kf1 = *reinterpret_cast<const b8_t*>(&Kt[ka + kLat + 16 * k + 16]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qr[k], s, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qr[k + 1], s2, 0, 0, 0);
      }
      // a few fragments in flight: 3 reads ahead, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int k = 0; k < 33; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_barrier(0);
      s += s2;
      // -------- 4. online softmax for head 32 wave + col over this lane's 16 tokens
      float tmax = -INFINITY;
      const uint32_t valid = SPARSE ? svalid[(tt - t_begin) / kTile] : 0xFFFFFFFFu;
      if (tt + kTile <= t_end && valid == 0xFFFFFFFFu) {  // a whole tile: nothing to mask
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = s[i] * a.scale_log2;
          tmax = fmaxf(tmax, s[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = 16 * (i >> 3) + 8 * half + (i & 7);
          s[i] = tt + j < t_end && ((valid >> j) & 1u) ? s[i] * a.scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, s[i]);
        }
      }
      tmax = max_xor32(tmax);
      // the reference max moves only when the tile max passes it by more than 2^8
      const bool bump = tmax > m_run + 8.f;
      const float m_new = bump ? tmax : m_run;
      const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      h8_t pf[2];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_new);
        psum += p;
        pf[i >> 3][i & 7] = (_Float16)p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__ballot(bump)) {
        // output rows are heads i % 4 + 8 (i / 4) + 4 half; head r's alpha is in
        // lane r.  The products are issued well after the last MFMA wrote the
        // accumulators (the whole QK product and softmax lie between).
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float ar = __shfl(alpha, (i & 3) + 8 * (i >> 2) + 4 * half);
#pragma unroll
          for (int n = 0; n < 16; ++n) {
            float x = o[n][i];
            scale_acc(x, ar);
            o[n][i] = x;
          }
        }
        asm volatile("s_nop 7");  // VALU writes of the accumulators, then MFMA reads of them
      }
      // -------- 5. O += P V
#pragma unroll
      for (int n = 0; n < 16; ++n) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const s4_t lo = read_tr16(&Kt[vb + c * kC + 32 * n]);
          const s4_t hi = read_tr16(&Kt[vb + c * kC + kH2 + 32 * n]);
          const h8_t vf = __builtin_bit_cast(h8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pf[c], vf, o[n], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int k = 0; k < 30; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the workgroup

  // ---------------- partial result of this split
  l_run += __shfl_xor(l_run, 32);
  const size_t row0 = qrow0 + 32 * wave;
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int col_e = lane_e & 31, half_e = lane_e >> 5;
  if (half_e == 0) {
    float* p = a.part + ((row0 + col_e) * a.splits + split) * (kLat + 2);
    p[0] = m_run;
    p[1] = l_run;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int head = (i & 3) + 8 * (i >> 2) + 4 * half_e;
    float* p = a.part + ((row0 + head) * a.splits + split) * (kLat + 2) + 2 + col_e;
#pragma unroll
    for (int n = 0; n < 16; ++n) p[32 * n] = o[n][i];
  }
}

}  // namespace

namespace {
template <bool PAGED, bool SPARSE>
int launch_latent(const MfmaDecodeArgs& a, int B, hipStream_t st) {
  dim3 grid(a.splits, B);
  switch (a.Hq) {
    case 32: decode_latent_kernel<1, PAGED, SPARSE><<<grid, 64, 0, st>>>(a); break;
    case 64: decode_latent_kernel<2, PAGED, SPARSE><<<grid, 128, 0, st>>>(a); break;
    case 128: decode_latent_kernel<4, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    default: return KV_EUNSUPPORTED;
  }
  return KV_OK;
}
}  // namespace

int launch_decode_latent(const MfmaDecodeArgs& a, int B, hipStream_t st) {
  if (a.sel) return a.pm.table ? KV_EUNSUPPORTED : launch_latent<false, true>(a, B, st);
  return a.pm.table ? launch_latent<true, false>(a, B, st) : launch_latent<false, false>(a, B, st);
}

}  // namespace kvq
