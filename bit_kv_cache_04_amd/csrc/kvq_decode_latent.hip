// Decode attention on the matrix cores over a shared latent cache: every query
// head attends to one 512-channel latent per token (FP4 E2M1, one bf16 scale per
// 16 channels) plus a 64-channel bf16 RoPE key; the value is the latent itself
// (page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2", CSA2
// section: one 512-channel latent shared by the heads, with a 64-channel RoPE
// part).
//
// With 128 query heads on one latent the per-token work is a dense contraction
// (2 x 128 x (576 + 512) flop per 448 packed bytes), far past the HBM ridge, so
// the whole tile math runs on v_mfma_f32_16x16x32_{f16,bf16}.
//
// One workgroup = one (sequence, context split), all Hq = 16 * NW query heads,
// NW waves: with 128 heads, 8 waves, two per SIMD, so that one wave's
// dequantisation, softmax and LDS reads overlap the other's matrix products.
// Wave w owns heads [16 w, 16 w + 16) end to end: its query operand (72
// registers) and its 16 x 512 fp32 output accumulators (128 registers) stay in
// registers for the whole split.  Per 32-token tile i, after one workgroup
// barrier:
//   1. the loads of tile i + 3 are issued into the stage tile i has freed
//      (direct-to-LDS, three stages in flight);
//   2. every thread dequantises its share of tile i + 1 into the other of two
//      token-major fp16 tiles (RoPE copied as bf16);
//   3. S^T = K Q^T for the wave's heads: 2 x 18 products on tile i;
//   4. online softmax per head (each head's 32 logits spread over 4 lanes);
//   5. O += P V: 32 products, V read transposed from tile i (ds_read_b64_tr_b16).
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
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s4_t* lds_s4_ptr;

constexpr int kTile = 32;
constexpr int kLat = 512, kRope = 64;
constexpr int kStages = 3;
// packed stage: codes 32 x 256 | scales 32 x 64 | RoPE 32 x 128
constexpr int kStCodes = 0, kStScale = 8192, kStRope = 10240, kStBytes = 14336;
// Kt: 32 token rows of 576 halves (fp16 latent, then bf16 RoPE), row stride
// 73 x 16 bytes.  Token t lives in row kt_phys(t): tokens 8j..8j+7 of each
// 16-token half on the even (j even) or odd (j odd) rows of that half.  Then the
// 16 rows a QK operand read touches (tokens 0-15 or 16-31) fall in 16 distinct
// 16-byte bank groups, and the 8 rows of a transposing PV read's 32 lanes
// (tokens 8j..8j+7) start on 8 distinct even (or odd) bank groups, their 32-byte
// spans disjoint.
constexpr int kKtStride = kLat + kRope + 8;
constexpr int kKtHalves = kTile * kKtStride;
constexpr int kRsrcFlags = 0x00020000;

__host__ __device__ constexpr int kt_phys(int t) { return (t & 16) | ((t & 7) << 1) | ((t >> 3) & 1); }

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

// Dequantise one packed stage into a token-major fp16 tile: item (token t,
// channel octet o) per thread and step, a wave's lanes the 64 octets of one
// token; RoPE rows copied through (bf16) by the first 256 threads.  The stage is
// read in one asm block that also waits for the reads (outputs early-clobber, so
// that no result register doubles as an address still to be read): the compiler would
// otherwise make every read of a stage wait for all loads into LDS still in
// flight (it cannot tell the three stages apart), the next tiles' included.
template <int NW>
__device__ __forceinline__ void dequant_tile(const uint8_t* st, uint16_t* kt, int tid) {
  constexpr int NT = 64 * NW;
  constexpr int NI = 2048 / NT;                   // items per thread: 4, 8 or 16
  static_assert(NI == 4 || NI == 8 || NI == 16, "items per thread");
  const int t0 = tid >> 6, o = tid & 63;          // item k: token t0 + (NT / 64) k, octet o
  // stage byte offsets (LDS addresses) of item 0's code word and scale; item k
  // adds k * (NT / 64) tokens: 256 and 64 bytes per token
  const uint32_t ac = (uint32_t)(uintptr_t)(st + kStCodes + t0 * 256 + 4 * o);
  const uint32_t as = (uint32_t)(uintptr_t)(st + kStScale + t0 * 64 + 2 * (o >> 1));
  uint32_t cw[NI], sw[NI];
#pragma unroll
  for (int k0 = 0; k0 < NI; k0 += 4) {
    constexpr int dt = NT / 64;
    asm volatile(
        "ds_read_b32 %0, %8 offset:%c10\n\t"
        "ds_read_u16 %4, %9 offset:%c11\n\t"
        "ds_read_b32 %1, %8 offset:%c12\n\t"
        "ds_read_u16 %5, %9 offset:%c13\n\t"
        "ds_read_b32 %2, %8 offset:%c14\n\t"
        "ds_read_u16 %6, %9 offset:%c15\n\t"
        "ds_read_b32 %3, %8 offset:%c16\n\t"
        "ds_read_u16 %7, %9 offset:%c17\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(cw[k0]), "=&v"(cw[k0 + 1]), "=&v"(cw[k0 + 2]), "=&v"(cw[k0 + 3]), "=&v"(sw[k0]),
          "=&v"(sw[k0 + 1]), "=&v"(sw[k0 + 2]), "=&v"(sw[k0 + 3])
        : "v"(ac), "v"(as), "i"(256 * dt * k0), "i"(64 * dt * k0), "i"(256 * dt * (k0 + 1)),
          "i"(64 * dt * (k0 + 1)), "i"(256 * dt * (k0 + 2)), "i"(64 * dt * (k0 + 2)), "i"(256 * dt * (k0 + 3)),
          "i"(64 * dt * (k0 + 3)));
  }
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int t = t0 + (NT / 64) * k;
    const h2_t sc = splat_bf16(sw[k]);
    *reinterpret_cast<uint4*>(kt + kt_phys(t) * kKtStride + 8 * o) =
        uint4{__builtin_bit_cast(uint32_t, fp4x2<0>(cw[k]) * sc), __builtin_bit_cast(uint32_t, fp4x2<1>(cw[k]) * sc),
              __builtin_bit_cast(uint32_t, fp4x2<2>(cw[k]) * sc), __builtin_bit_cast(uint32_t, fp4x2<3>(cw[k]) * sc)};
  }
  // RoPE: 32 tokens x 8 parts of 16 bytes
#pragma unroll
  for (int k = 0; k < (256 + NT - 1) / NT; ++k) {
    const int it = tid + k * NT;
    if (it < 256) {
      const int t = it >> 3, part = it & 7;
      const uint32_t ar = (uint32_t)(uintptr_t)(st + kStRope + t * 128 + 16 * part);
      uint4 r;
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(ar));
      *reinterpret_cast<uint4*>(kt + kt_phys(t) * kKtStride + kLat + 8 * part) = r;
    }
  }
}

// Per-wave state that lives across tiles.
struct LatentWave {
  h8_t ql[16];   // query, latent part (fp16): B operand of 16 k-steps
  b8_t qr[2];    // query, RoPE part (bf16): 2 k-steps
  f4_t o[32];    // output accumulators, N block nb = channels 16 nb + [0, 16)
  float m_run;   // running max (log2 units) of this lane's head
  float l_part;  // this lane's share of the running sum
};

// QK, softmax and PV of one dequantised tile kt (first token tt, tokens below
// t_end; SPARSE: slot j valid when bit j of `valid`).  The operand reads run D
// k-steps (QK) and E products (PV) ahead of the products that use them: as deep
// as the 256 registers of a wave that shares its SIMD allow without spilling.
template <bool SPARSE, int D, int E>
__device__ __forceinline__ void tile_math(LatentWave& w, const uint16_t* kt, int ka, int vb0, int vb1, int grp,
                                          int tt, int t_end, uint32_t valid, float scale_log2) {
  constexpr int kHalf = kt_phys(16) * kKtStride;  // token 16 + m: row kt_phys(m) + 16
  // -------- S^T = K Q^T: tokens col and 16 + col (rows), this wave's heads (columns).
  h8_t kf[18][2];
  f4_t s0 = f4_t{}, s1 = f4_t{};
  auto kread = [&](int k) {
    kf[k][0] = *reinterpret_cast<const h8_t*>(kt + ka + 32 * k);
    kf[k][1] = *reinterpret_cast<const h8_t*>(kt + ka + kHalf + 32 * k);
  };
#pragma unroll
  for (int k = 0; k < D; ++k) kread(k);
#pragma unroll
  for (int k = 0; k < 18; ++k) {
    if (k + D < 18) kread(k + D);
    if (k < 16) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[k][0], w.ql[k], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[k][1], w.ql[k], s1, 0, 0, 0);
    } else {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, kf[k][0]), w.qr[k - 16], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, kf[k][1]), w.qr[k - 16], s1, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * D, 0);
#pragma unroll
  for (int k = 0; k < 18 - D; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * D, 0);
  __builtin_amdgcn_sched_barrier(0);
  // -------- online softmax for this lane's head: tokens 4 grp + j (s0) and
  // 16 + 4 grp + j (s1), j < 4
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = s0[j], x[4 + j] = s1[j];
  float tmax = -INFINITY;
  if (tt + kTile <= t_end && valid == 0xFFFFFFFFu) {  // a whole tile: nothing to mask
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] *= scale_log2;
      tmax = fmaxf(tmax, x[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 16 * (j >> 2) + 4 * grp + (j & 3);
      x[j] = tt + tok < t_end && ((valid >> tok) & 1u) ? x[j] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[j]);
    }
  }
  tmax = max_xor32(max_xor16(tmax));
  // the reference max moves only when the tile max passes it by more than 2^8
  const bool bump = tmax > w.m_run + 8.f;
  const float m_new = bump ? tmax : w.m_run;
  const float alpha = bump ? __builtin_amdgcn_exp2f(w.m_run - m_new) : 1.f;
  h8_t pf;
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(x[j] - m_new);
    psum += p;
    pf[j] = (_Float16)p;
  }
  w.l_part = w.l_part * alpha + psum;
  w.m_run = m_new;
  if (__ballot(bump)) {
    // output rows are heads 4 grp + r; head h's alpha is in lane h
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int n = 0; n < 32; ++n) w.o[n][r] *= ar;
    }
  }
  // -------- O += P V: A = P (head col, k-slots = tokens 4 grp + [0, 4) and
  // 16 + 4 grp + [0, 4)), B = V (same k-slots, channel 16 nb + col).
  s4_t vf[32][2];
  auto vread = [&](int nb) {
    vf[nb][0] = read_tr16(kt + vb0 + 16 * nb);
    vf[nb][1] = read_tr16(kt + vb1 + 16 * nb);
  };
#pragma unroll
  for (int nb = 0; nb < E; ++nb) vread(nb);
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) {
    if (nb + E < 32) vread(nb + E);
    const h8_t v = __builtin_bit_cast(h8_t, __builtin_shufflevector(vf[nb][0], vf[nb][1], 0, 1, 2, 3, 4, 5, 6, 7));
    w.o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, v, w.o[nb], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * E, 1);
#pragma unroll
  for (int nb = 0; nb < 32 - E; ++nb) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, E, 1);
  __builtin_amdgcn_sched_barrier(0);
}

// PAGED: token rows in pool pages named by the block table, resources per tile.
// SPARSE (contiguous caches): the split's slots read the positions a.sel names,
// staged in LDS; slots without a valid position are masked.
template <int NW, bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW / 4 > 1 ? NW / 4 : 1, NW / 4 > 1 ? NW / 4 : 1))) decode_latent_kernel(
    MfmaDecodeArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int kLoads = 32 / NW;  // direct-to-LDS loads per wave per tile
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStages][kStBytes];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][kKtHalves];

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
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;
  const int col = lane & 15, grp = lane >> 4;  // head of this lane's column, its lane group
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

  // resources over nrows token rows from row0 (nrows 0: every read is zeros)
  auto res_at = [&](size_t row0, int nrows) {
    return Res{rsrc(a.k_codes + row0 * 256, (size_t)nrows * 256), rsrc(a.k_scale + row0 * 32, (size_t)nrows * 64),
               rsrc(a.rope + row0 * 64, (size_t)nrows * 128)};
  };
  const Res res = res_at((size_t)b * a.cap, a.cap);
  // the loads of tile index ti (token t_begin + 32 ti) into stage st; a missing
  // tile reads past the end of its resources
  auto issue_at = [&](uint8_t* st, int ti) {
    const int t = t_begin + ti * kTile;
    if constexpr (SPARSE) {
      issue_tile_sparse<NW>(st, wave, lane, t < t_end ? t - t_begin : -1, spos, res);
    } else if constexpr (!PAGED) {
      issue_tile<NW>(st, wave, lane, t < t_end ? t : a.cap, res);
    } else {
      const int pg = t < t_end ? page_of_uniform(a.pm, b, t) : -1;
      issue_tile<NW>(st, wave, lane, pg < 0 ? 0 : t & (a.pm.tokens - 1),
                     res_at((size_t)(pg < 0 ? 0 : pg) * a.pm.tokens, pg < 0 ? 0 : a.pm.tokens));
    }
  };
#pragma unroll
  for (int s = 0; s < kStages; ++s) issue_at(stage[s], s);

  LatentWave w;
  // ---------------- the query operand: 16 fp16 latent steps, 2 bf16 RoPE steps
  // (B operand of the 16x16x32 products: head col, channels 32 k + 8 grp + [0, 8))
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (qrow0 + 16 * wave + col) * (kLat + kRope);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * grp);
      w.ql[s] = __builtin_bit_cast(h8_t, uint4{bf16x2_to_h2(raw.x), bf16x2_to_h2(raw.y), bf16x2_to_h2(raw.z),
                                               bf16x2_to_h2(raw.w)});
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
      w.qr[s] = __builtin_bit_cast(b8_t, *reinterpret_cast<const uint4*>(qp + kLat + 32 * s + 8 * grp));
  }
#pragma unroll
  for (int n = 0; n < 32; ++n) w.o[n] = f4_t{};
  w.m_run = -INFINITY;
  w.l_part = 0.f;

  // lane constants of the fragment reads (kept opaque so that the compiler does
  // not hoist one address register per read out of the loop)
  // QK A operand: token col (+16), channels 32 k + 8 grp + [0, 8)
  int ka = kt_phys(col) * kKtStride + 8 * grp;
  // transposing PV reads: lane (e = (lane % 16) / 4, q = lane % 4) addresses
  // channels 16 nb + 4 q + [0, 4) of token 4 grp + e (and 16 + 4 grp + e), so
  // that it receives channel 16 nb + col of those four tokens: its PV B operand
  const int e4 = (lane & 15) >> 2, q4 = lane & 3;
  int vb0 = kt_phys(4 * grp + e4) * kKtStride + 4 * q4;
  int vb1 = kt_phys(16 + 4 * grp + e4) * kKtStride + 4 * q4;
  asm volatile("" : "+v"(ka), "+v"(vb0), "+v"(vb1));

  // prologue: tile 0's loads have landed (tiles 1 and 2 may still be in flight)
  if (ntiles > 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * kLoads));
    __syncthreads();
    dequant_tile<NW>(stage[0], Kt[0], tid);
  }

  for (int i = 0; i < ntiles; ++i) {
    // this wave's loads of tile i + 1 have landed (tile i + 2's may still be in
    // flight); the barrier then covers every wave's, the whole of tile i's
    // dequantised copy, and every wave being done with tile i - 1
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(kLoads));
    __syncthreads();
    issue_at(stage[i % kStages], i + kStages);  // the stage of tile i is free: tile i + 3
    if (i + 1 < ntiles) dequant_tile<NW>(stage[(i + 1) % kStages], Kt[(i + 1) & 1], tid);
    tile_math<SPARSE, SPARSE ? 1 : 2, SPARSE ? 2 : 4>(w, Kt[i & 1], ka, vb0, vb1, grp, t_begin + i * kTile, t_end, SPARSE ? svalid[i] : 0xFFFFFFFFu,
                      a.scale_log2);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the workgroup

  // ---------------- partial result of this split
  float l_run = w.l_part + __shfl_xor(w.l_part, 16);
  l_run += __shfl_xor(l_run, 32);
  const size_t row0 = qrow0 + 16 * wave;
  if (grp == 0) {
    float* p = a.part + ((row0 + col) * a.splits + split) * (kLat + 2);
    p[0] = w.m_run;
    p[1] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* p = a.part + ((row0 + 4 * grp + r) * a.splits + split) * (kLat + 2) + 2 + col;
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) p[16 * nb] = w.o[nb][r];
  }
}

}  // namespace

namespace {
template <bool PAGED, bool SPARSE>
int launch_latent(const MfmaDecodeArgs& a, int B, hipStream_t st) {
  dim3 grid(a.splits, B);
  switch (a.Hq) {
    case 32: decode_latent_kernel<2, PAGED, SPARSE><<<grid, 128, 0, st>>>(a); break;
    case 64: decode_latent_kernel<4, PAGED, SPARSE><<<grid, 256, 0, st>>>(a); break;
    case 128: decode_latent_kernel<8, PAGED, SPARSE><<<grid, 512, 0, st>>>(a); break;
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
