// Append kernels: quantise new tokens' keys/values into the packed cache.
//
// FP4 E2M1 groups (page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via
// CSA2", numerical-precision section), KIVI 2-bit (page "TurboQuant vs OSCAR vs
// EpiCache", "quantization frontiers", KIVI paragraph), TurboQuant and QJL
// sign sketches (same section, stages one and two).  The rotation and the QJL
// projection are the only dense contractions here and run on the matrix cores.
#include <hip/hip_runtime.h>

#include <type_traits>

#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// First cache positions of an append: one for every sequence, or one per
// sequence (s[b] for sequence b of the launch, `heads` sequence-head rows each),
// passed by value so that no device memory holds them.
constexpr int kMaxRaggedSeqs = 256;
struct AppendPos {
  int start;   // every sequence's first position when ragged == 0
  int ragged;  // 1: sequence b starts at s[b]
  int heads;   // sequence-head rows per sequence (KV heads; 1 for the latent)
  PageMap pm;  // where the launch's sequences keep their token rows
  int32_t s[kMaxRaggedSeqs];
};
__device__ __forceinline__ int start_of(const AppendPos& p, size_t bh) {
  return p.ragged ? p.s[bh / p.heads] : p.start;
}

// Cache row of sequence-head bh's position t (kNoRow: a page outside the pool,
// whose stores are dropped).
__device__ __forceinline__ size_t seq_row(const AppendPos& pos, size_t bh, int t, int cap) {
  if (!pos.pm.table) return bh * (size_t)cap + t;
  return token_row(pos.pm, pos.heads, (int)(bh / pos.heads), (int)(bh % pos.heads), t);
}

// Token rows of an append are flat indices r in [0, bh_count * n): sequence-head
// bh = r / n, position start_of(bh) + r % n; the input row r starts at x + r * stride.
__device__ __forceinline__ size_t dst_row(size_t r, int n, int cap, const AppendPos& pos) {
  return seq_row(pos, r / n, start_of(pos, r / n) + (int)(r % n), cap);
}

// dst_row with the ragged starts read from an LDS copy (fill_starts): indexing
// the by-value table itself with a per-row index would copy it to scratch in
// every thread.
__device__ __forceinline__ void fill_starts(const AppendPos& pos, int* starts) {
  if (pos.ragged && threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kMaxRaggedSeqs; ++j) starts[j] = pos.s[j];  // constant offsets: kernel-argument reads
  }
  __syncthreads();
}
__device__ __forceinline__ int start_tab(const AppendPos& pos, const int* starts, size_t bh) {
  return pos.ragged ? starts[bh / pos.heads] : pos.start;
}
__device__ __forceinline__ size_t dst_row_tab(size_t r, int n, int cap, const AppendPos& pos, const int* starts) {
  const size_t bh = r / n;
  return seq_row(pos, bh, start_tab(pos, starts, bh) + (int)(r % n), cap);
}

// ---------------------------------------------------------------- FP4

// 16 consecutive input elements, read with 16-byte loads (input rows and group
// offsets are multiples of 16 bytes) and unpacked to fp32 when needed.
template <typename InT>
struct Raw16;
template <>
struct Raw16<uint16_t> {
  uint4 w[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    w[0] = reinterpret_cast<const uint4*>(p)[0];
    w[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void unpack(float (&f)[16]) const {
    const uint32_t u[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Raw16<float> {
  float4 w[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = reinterpret_cast<const float4*>(p)[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = float4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void unpack(float (&f)[16]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[4 * i] = w[i].x;
      f[4 * i + 1] = w[i].y;
      f[4 * i + 2] = w[i].z;
      f[4 * i + 3] = w[i].w;
    }
  }
};

// One 16-value group: s = bf16_RNE(absmax / 6) (the quotient taken in fp64,
// then rounded once), then each element's E2M1 nibble against s by comparing
// |x| with the midpoints times s (exact in fp32: s has 8 significant bits).
__device__ __forceinline__ void fp4_encode_compare(const float (&a)[16], float amax, unsigned long long& packed,
                                                   uint16_t& sb) {
  sb = bf16_from_f64(__ddiv_rn((double)amax, 6.0));
  const float s = bf16_to_f32(sb);
  packed = 0;
  if (s > 0.f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) packed |= (unsigned long long)e2m1_encode(a[i], s) << (4 * i);
  }
}

// x rounded to 16 mantissa bits (halfway away from zero).
__device__ __forceinline__ float snap16(float x) { return __uint_as_float((__float_as_uint(x) + 64u) & ~127u); }

// The same group from bf16 inputs, without fp64 and without per-element
// compares.  x and s both carry 8 significant bits, so x / s either equals an
// E2M1 midpoint exactly or lies at least 2^-12.3 (relative) away from every
// midpoint; likewise absmax / 6 lies at least 2^-10.6 away from every bf16
// midpoint (it is never one).  Hence
//   s = bf16_RNE(fl32(absmax * fl32(1/6)))        (error 2^-23)
//   q = fl32(x * rcp(s)), rounded to 16 bits      (error 2^-22 before rounding;
//                                                  an exact midpoint comes back
//                                                  exactly, nothing else crosses one)
// take the exact-arithmetic decisions, and the hardware E2M1 conversion (ties to
// even, saturating at 6, sign of zero kept) forms each pair of nibbles.  A group
// whose absmax lies outside [2^-100, 2^100], where rcp(s) could leave the normal
// range, takes the compare path.
__device__ __forceinline__ void fp4_encode_bf16(const float (&a)[16], unsigned long long& packed, uint16_t& sb) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(a[i]));
  if (!(amax >= 0x1p-100f && amax <= 0x1p100f)) {
    fp4_encode_compare(a, amax, packed, sb);
    return;
  }
  const uint32_t u = __float_as_uint(amax * (1.0f / 6.0f));
  const uint32_t sbits = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  sb = (uint16_t)sbits;
  const float r = __builtin_amdgcn_rcpf(__uint_as_float(sbits << 16));
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* e = a + 8 * h;
    uint32_t word = 0u;
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, snap16(e[0] * r), snap16(e[1] * r), 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, snap16(e[2] * r), snap16(e[3] * r), 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, snap16(e[4] * r), snap16(e[5] * r), 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, snap16(e[6] * r), snap16(e[7] * r), 1.0f, 3);
    w[h] = word;
  }
  packed = (unsigned long long)w[0] | ((unsigned long long)w[1] << 32);
}

__device__ __forceinline__ void fp4_encode16(const float (&a)[16], unsigned long long& packed, uint16_t& sb,
                                             const uint16_t*) {
  fp4_encode_bf16(a, packed, sb);
}
__device__ __forceinline__ void fp4_encode16(const float (&a)[16], unsigned long long& packed, uint16_t& sb,
                                             const float*) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(a[i]));
  fp4_encode_compare(a, amax, packed, sb);
}

// Encode one group (values already loaded) and store its codes (element 2i in
// the low nibble of byte i) and scale at cache row dr, group g.  `tag` only
// selects the input type's encoder.
template <typename InT>
__device__ __forceinline__ void fp4_store_at(const float (&a)[16], const InT* tag, size_t dr, int g, int d,
                                             uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  unsigned long long packed;
  uint16_t sb;
  fp4_encode16(a, packed, sb, tag);
  if (dr == kNoRow) return;
  *reinterpret_cast<unsigned long long*>(codes + dr * (d / 2) + g * 8) = packed;
  scales[dr * (d / 16) + g] = sb;
}
template <typename InT>
__device__ __forceinline__ void fp4_store_group(const float (&a)[16], const InT* tag, size_t r, int g, int d,
                                                uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, int n,
                                                int cap, const AppendPos& pos, const int* starts) {
  fp4_store_at(a, tag, dst_row_tab(r, n, cap, pos, starts), g, d, codes, scales);
}

// Group gid (= row * (d / 16) + group) of a row-major input with row stride
// `stride` elements.
template <typename InT>
__device__ __forceinline__ void fp4_group(const InT* __restrict__ x, size_t stride, int d,
                                          uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                          size_t rows, int n, int cap, const AppendPos& pos, const int* starts,
                                          size_t gid) {
  const int groups = d / 16;
  if (gid >= rows * groups) return;
  const int g = (int)(gid % groups);
  const size_t r = gid / groups;
  Raw16<InT> raw;
  raw.load(x + r * stride + g * 16);
  float a[16];
  raw.unpack(a);
  fp4_store_group(a, x, r, g, d, codes, scales, n, cap, pos, starts);
}

// K (blockIdx.y = 0) and V (blockIdx.y = 1) of an FP4 cache in one launch.
template <typename InT>
__global__ void __launch_bounds__(256) fp4_append_kernel(const InT* __restrict__ k, const InT* __restrict__ v,
                                                         int d, uint8_t* __restrict__ kc, uint16_t* __restrict__ ks,
                                                         uint8_t* __restrict__ vc, uint16_t* __restrict__ vs,
                                                         size_t rows, int n, int cap, AppendPos pos) {
  __shared__ int starts[kMaxRaggedSeqs];
  fill_starts(pos, starts);
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.y == 0) fp4_group(k, d, d, kc, ks, rows, n, cap, pos, starts, gid);
  else fp4_group(v, d, d, vc, vs, rows, n, cap, pos, starts, gid);
}

// Latent: the 512-wide latent as FP4 groups (blockIdx.y = 0) and the RoPE key
// copied through as bf16, rounded once if the input is fp32 (blockIdx.y = 1).
template <typename InT>
__global__ void __launch_bounds__(256) latent_append_kernel(const InT* __restrict__ x, int d, int rope_dim,
                                                            uint8_t* __restrict__ cc, uint16_t* __restrict__ cs,
                                                            uint16_t* __restrict__ rope, size_t rows, int n,
                                                            int cap, AppendPos pos) {
  __shared__ int starts[kMaxRaggedSeqs];
  fill_starts(pos, starts);
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)d + rope_dim;
  if (blockIdx.y == 0) {
    fp4_group(x, stride, d, cc, cs, rows, n, cap, pos, starts, gid);
  } else if (gid < rows * rope_dim) {
    const int c = (int)(gid % rope_dim);
    const size_t r = gid / rope_dim;
    const float val = load_as_f32(x + r * stride + d, c);
    const size_t dr = dst_row_tab(r, n, cap, pos, starts);
    if (dr != kNoRow) rope[dr * rope_dim + c] = bf16_from_f64((double)val);
  }
}

// ---------------------------------------------------------------- KIVI 2-bit

// codes c = clamp(RNE((x - z) / s), 0, 3) in fp32 with s = (max - min) / 3,
// z = min; c = 0 when s == 0.
// KIVI key staging per sequence-head: word 0 the tokens appended so far, words
// 1..3 unused, then the 32 x d keys of the incomplete last group.
__device__ __forceinline__ float* stage_keys(float* stage, size_t bh, int d) { return stage + bh * (4 + 32 * d) + 4; }
__device__ __forceinline__ void set_appended(float* stage, size_t bh, int d, int appended) {
  reinterpret_cast<int*>(stage)[bh * (4 + 32 * d)] = appended;
}

__device__ __forceinline__ uint32_t kivi_code(float x, float z, float s) {
  if (!(s > 0.f)) return 0;
  float q = rintf(__fdiv_rn(__fsub_rn(x, z), s));
  q = fminf(fmaxf(q, 0.f), 3.f);
  return (uint32_t)q;
}

// One workgroup per (sequence x KV head, 32-token group): the group's keys and
// values are staged in LDS with coalesced loads, then all 256 threads code:
//   keys:   per channel, min / max over the 32 tokens, the tokens split over
//           256 / d threads;
//   values: per (token, 32-channel group), min / max over the group, its
//           channels split over 256 / (d / 32 x 32) threads (16 channels each
//           at d = 128, 8 at d = 64).
constexpr int kKiviMaxD = 128;

__device__ __forceinline__ float4 load4_as_f32(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_as_f32(const uint16_t* p) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  return float4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                __uint_as_float(r.y & 0xFFFF0000u)};
}

template <typename InT>
__global__ void __launch_bounds__(256) kivi_append_kernel(const InT* __restrict__ k, const InT* __restrict__ v,
                                                          int d, uint8_t* kc, float* ks, float* kz, uint8_t* vc,
                                                          float* vs, float* vz, float* stage, int bh_count, int n,
                                                          int cap, AppendPos pos) {
  __shared__ float xk[32][kKiviMaxD + 1];
  __shared__ float xv[32][kKiviMaxD + 1];
  __shared__ int starts[kMaxRaggedSeqs];
  fill_starts(pos, starts);
  const int tid = threadIdx.x;
  const int ngroups = n / 32;
  const int g = blockIdx.x % ngroups;
  const size_t bh = blockIdx.x / ngroups;
  const size_t r0 = bh * n + (size_t)g * 32;  // first input row of the group
  {
    // 32 x d elements as groups of 4 (rows are 16-byte aligned: d is 64 or 128),
    // every load of this thread in flight before the first store
    constexpr int kMaxIt = 32 * kKiviMaxD / 4 / 256;
    float4 a[kMaxIt], bq[kMaxIt];
#pragma unroll
    for (int i = 0; i < kMaxIt; ++i) {
      const int e = 4 * (tid + 256 * i);
      if (e < 32 * d) {
        a[i] = load4_as_f32(k + r0 * d + e);
        bq[i] = load4_as_f32(v + r0 * d + e);
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxIt; ++i) {
      const int e = 4 * (tid + 256 * i);
      if (e < 32 * d) {
        const int t = e / d, c = e % d;
        xk[t][c] = a[i].x, xk[t][c + 1] = a[i].y, xk[t][c + 2] = a[i].z, xk[t][c + 3] = a[i].w;
        xv[t][c] = bq[i].x, xv[t][c + 1] = bq[i].y, xv[t][c + 2] = bq[i].z, xv[t][c + 3] = bq[i].w;
      }
    }
  }
  __syncthreads();
  const int quads = d / 4;
  const int start = start_tab(pos, starts, bh);
  const size_t slot0 = seq_row(pos, bh, start + g * 32, cap);  // cache row of the group's first token
  if (tid == 0 && g == ngroups - 1) set_appended(stage, bh, d, start + n);
  if (slot0 == kNoRow) return;  // a page outside the pool
  // keys: thread (token part kp, channel c), d * kparts = 256; every thread
  // takes its channel's min / max over the 32 tokens, then codes its part's
  // 32 / kparts tokens (lanes c .. c + 3 of a wave pack one byte per token)
  {
    const int kparts = 256 / d, c = tid % d, kp = tid / d, tpp = 32 / kparts;
    float mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < 32; ++t) {
      mn = fminf(mn, xk[t][c]);
      mx = fmaxf(mx, xk[t][c]);
    }
    const float sc = __fdiv_rn(__fsub_rn(mx, mn), 3.0f);
    for (int t = kp * tpp; t < (kp + 1) * tpp; ++t) {
      uint32_t code = kivi_code(xk[t][c], mn, sc) << (2 * (c & 3));
      code |= __shfl_xor(code, 1);
      code |= __shfl_xor(code, 2);
      if ((c & 3) == 0) kc[(slot0 + t) * quads + c / 4] = (uint8_t)code;
    }
    if (kp == 0) {
      const size_t meta = slot0 / 32 * (size_t)d + c;  // pages and the layout hold whole groups
      ks[meta] = sc;
      kz[meta] = mn;
    }
  }
  // values: thread (token t, channel group vg, channel part vp), 32 * vgroups *
  // vparts = 256; every thread takes the group's min / max over its 32 channels
  // and codes its part's 32 / vparts of them
  {
    const int vgroups = d / 32, vparts = 256 / (32 * vgroups), cpp = 32 / vparts;
    const int vp = tid % vparts, vg = (tid / vparts) % vgroups, t = tid / (vparts * vgroups);
    float mn = INFINITY, mx = -INFINITY;
    for (int i = 0; i < 32; ++i) {
      mn = fminf(mn, xv[t][32 * vg + i]);
      mx = fmaxf(mx, xv[t][32 * vg + i]);
    }
    const float sc = __fdiv_rn(__fsub_rn(mx, mn), 3.0f);
    uint32_t packed = 0;
    for (int i = 0; i < cpp; ++i) packed |= kivi_code(xv[t][32 * vg + vp * cpp + i], mn, sc) << (2 * i);
    const size_t dr = slot0 + t;
    uint8_t* dst = vc + dr * (d / 4) + vg * 8 + vp * (cpp / 4);
    if (cpp == 16) *reinterpret_cast<uint32_t*>(dst) = packed;
    else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
    if (vp == 0) {
      vs[dr * vgroups + vg] = sc;
      vz[dr * vgroups + vg] = mn;
    }
  }
}

// Appends that leave or fill an incomplete key group (any start and length).
// Workgroup (sequence-head bh, group index gi) takes group G = start / 32 + gi,
// tokens [32 G, 32 G + 32): its keys before the append come from the staging
// slots, the new ones from the input.  A group the append completes is coded
// as in kivi_append_kernel; an incomplete one keeps its new keys in staging
// (slot t mod 32).  Values are coded per token for the new tokens only.
// Two launches on one stream: phase 0 codes (reading the old staged keys of the
// first group), phase 1 then writes the new staged keys of the last, incomplete
// group.  Both use slots t mod 32, so in one launch a workgroup could overwrite
// slots another workgroup has still to read.
template <typename InT>
__global__ void __launch_bounds__(256) kivi_append_any_kernel(const InT* __restrict__ k, const InT* __restrict__ v,
                                                              int d, uint8_t* kc, float* ks, float* kz, uint8_t* vc,
                                                              float* vs, float* vz, float* stage, int n, int cap,
                                                              AppendPos pos, int phase) {
  __shared__ float xk[32][kKiviMaxD + 1];
  __shared__ float xv[32][kKiviMaxD + 1];
  __shared__ int starts[kMaxRaggedSeqs];
  fill_starts(pos, starts);
  const int tid = threadIdx.x;
  const int ngmax = n / 32 + 2;  // groups an append of n tokens can touch
  const int gi = blockIdx.x % ngmax;
  const size_t bh = blockIdx.x / ngmax;
  const int s = start_tab(pos, starts, bh);
  const int g0 = 32 * (s / 32 + gi);                 // the group's first token
  const int a0 = max(g0, s), a1 = min(g0 + 32, s + n);  // its new tokens
  if (a0 >= a1) return;                              // the whole workgroup: no token of this append
  const bool complete = s + n >= g0 + 32;
  if (phase == 1) {  // the new staged keys of the last, incomplete group, and the appended length
    if (!complete) {
      for (int e = tid; e < (a1 - a0) * d; e += 256) {
        const int t = a0 - g0 + e / d, c = e % d;
        stage_keys(stage, bh, d)[t * d + c] = load_as_f32(k + (bh * n + (g0 + t - s)) * d, c);
      }
    }
    if (tid == 0 && g0 + 32 >= s + n) set_appended(stage, bh, d, s + n);  // the group of the last token
    return;
  }
  for (int e = tid; e < 32 * d; e += 256) {
    const int t = e / d, c = e % d, tok = g0 + t;
    float kx = 0.f, vx = 0.f;
    if (tok < a0) {
      kx = stage_keys(stage, bh, d)[t * d + c];
    } else if (tok < a1) {
      const size_t r = bh * n + (tok - s);
      kx = load_as_f32(k + r * d, c);
      vx = load_as_f32(v + r * d, c);
    }
    xk[t][c] = kx;
    xv[t][c] = vx;
  }
  __syncthreads();
  const int quads = d / 4;
  const size_t slot0 = seq_row(pos, bh, g0, cap);  // cache row of the group's first token
  if (complete) {
    if (tid < quads && slot0 != kNoRow) {
      const int cq = tid;
      float mn[4], mx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) mn[j] = INFINITY, mx[j] = -INFINITY;
      for (int t = 0; t < 32; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mn[j] = fminf(mn[j], xk[t][4 * cq + j]);
          mx[j] = fmaxf(mx[j], xk[t][4 * cq + j]);
        }
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[j] = __fdiv_rn(__fsub_rn(mx[j], mn[j]), 3.0f);
      for (int t = 0; t < 32; ++t) {
        uint32_t byte = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) byte |= kivi_code(xk[t][4 * cq + j], mn[j], sc[j]) << (2 * j);
        kc[(slot0 + t) * quads + cq] = (uint8_t)byte;
      }
      const size_t meta = slot0 / 32 * (size_t)d + 4 * cq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ks[meta + j] = sc[j];
        kz[meta + j] = mn[j];
      }
    }
  }
  const int vgroups = d / 32;
  for (int it = tid; slot0 != kNoRow && it < (a1 - a0) * vgroups; it += 256) {
    const int t = a0 - g0 + it / vgroups, vg = it % vgroups;
    float mn = INFINITY, mx = -INFINITY;
    for (int i = 0; i < 32; ++i) {
      mn = fminf(mn, xv[t][32 * vg + i]);
      mx = fmaxf(mx, xv[t][32 * vg + i]);
    }
    const float sc = __fdiv_rn(__fsub_rn(mx, mn), 3.0f);
    unsigned long long packed = 0;
    for (int i = 0; i < 32; ++i) packed |= (unsigned long long)kivi_code(xv[t][32 * vg + i], mn, sc) << (2 * i);
    const size_t dr = slot0 + t;
    *reinterpret_cast<unsigned long long*>(vc + dr * (d / 4) + vg * 8) = packed;
    vs[dr * vgroups + vg] = sc;
    vz[dr * vgroups + vg] = mn;
  }
}

// ---------------------------------------------------------------- QJL sign sketch (MFMA)

// Split x into bf16 parts whose sum is exactly x (1 part for bf16 input, 3 for fp32).
// A lane's share of a 16-token key tile as the A operand of
// v_mfma_f32_16x16x32_bf16: token (lane & 15), channels ks * 32 + 8 * (lane >> 4)
// + j (j < 8) of the four 32-wide k-steps ks.  A bf16 input is the operand as it
// is; an fp32 input is the exact sum of three bf16 slices (truncations), each
// its own product.  The fragment stays in registers for the fp64 recheck.
template <typename InT>
struct KeyFrag;
template <>
struct KeyFrag<uint16_t> {
  static constexpr int NP = 1;
  uint4 r[4];
  __device__ __forceinline__ void load(const uint16_t* row, int kq) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) r[ks] = *reinterpret_cast<const uint4*>(row + ks * 32 + kq * 8);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) r[ks] = make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ float value(int ks, int j) const {
    const uint32_t w = j < 2 ? r[ks].x : j < 4 ? r[ks].y : j < 6 ? r[ks].z : r[ks].w;
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ __forceinline__ void parts(int ks, bf16x8 (&p)[NP]) const { p[0] = __builtin_bit_cast(bf16x8, r[ks]); }
};
template <>
struct KeyFrag<float> {
  static constexpr int NP = 3;
  float4 r[4][2];
  __device__ __forceinline__ void load(const float* row, int kq) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) r[ks][h] = *reinterpret_cast<const float4*>(row + ks * 32 + kq * 8 + 4 * h);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) r[ks][0] = r[ks][1] = float4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ float value(int ks, int j) const {
    const float4 q = r[ks][j >> 2];
    const int c = j & 3;
    return c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
  }
  __device__ __forceinline__ void parts(int ks, bf16x8 (&p)[NP]) const;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint16_t (&h)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = __builtin_bit_cast(__bf16, h[i]);
  return r;
}

__device__ __forceinline__ void KeyFrag<float>::parts(int ks, bf16x8 (&p)[NP]) const {
  uint16_t h[NP][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v = value(ks, j);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const uint32_t hi = __float_as_uint(v) & 0xFFFF0000u;  // truncation: exact top slice
      h[k][j] = (uint16_t)(hi >> 16);
      v = v - __uint_as_float(hi);                          // exact remainder
    }
  }
#pragma unroll
  for (int k = 0; k < NP; ++k) p[k] = as_bf16x8(h[k]);
}

constexpr int kSPad = 136;  // LDS row pitch (elements) of the staged 128 x 128 bf16 matrix

// 32 consecutive elements (bf16 or fp32, 16-byte aligned) as fp32, with the
// loads issued together.
__device__ __forceinline__ void load32_as_f32(const uint16_t* p, float (&out)[32]) {
  uint4 r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = reinterpret_cast<const uint4*>(p)[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      out[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}
__device__ __forceinline__ void load32_as_f32(const float* p, float (&out)[32]) {
  float4 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = reinterpret_cast<const float4*>(p)[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[4 * i] = r[i].x;
    out[4 * i + 1] = r[i].y;
    out[4 * i + 2] = r[i].z;
    out[4 * i + 3] = r[i].w;
  }
}

// Stage a bf16-valued 128 x 128 fp32 matrix into LDS as bf16 (row pitch kSPad):
// 16 four-float loads per thread, all in flight before the first store.
__device__ __forceinline__ void stage_bf16_matrix(const float* __restrict__ m, uint16_t* dst) {
  const int tid = threadIdx.x;
  float4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = reinterpret_cast<const float4*>(m)[tid + 256 * i];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = 4 * (tid + 256 * i);
    uint2 h;
    h.x = (__float_as_uint(v[i].x) >> 16) | (__float_as_uint(v[i].y) & 0xFFFF0000u);
    h.y = (__float_as_uint(v[i].z) >> 16) | (__float_as_uint(v[i].w) & 0xFFFF0000u);
    *reinterpret_cast<uint2*>(&dst[(e >> 7) * kSPad + (e & 127)]) = h;
  }
}

// x of lane l plus x of lane l ^ 16 (ROW = 16) or l ^ 32 (ROW = 32), in
// registers (v_permlane16_swap / v_permlane32_swap of each half with itself
// leaves the two lanes' halves in the two results, in either order).
template <int ROW>
__device__ __forceinline__ double add_swapped(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t a0, a1, b0, b1;
  if constexpr (ROW == 16) {
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    a0 = l[0]; a1 = l[1]; b0 = h[0]; b1 = h[1];
  } else {
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    a0 = l[0]; a1 = l[1]; b0 = h[0]; b1 = h[1];
  }
  return __builtin_bit_cast(double, (uint64_t)a0 | ((uint64_t)b0 << 32)) +
         __builtin_bit_cast(double, (uint64_t)a1 | ((uint64_t)b1 << 32));
}

// Keys of one wave's 16 tokens [base, base + 16): sketch bit i = [(S k)_i >= 0]
// and the token's fp16 norm.  C = K_tile S^T on v_mfma_f32_16x16x32_bf16 (S^T
// read from LDS, fp32 accumulation of exact products).  Summing n exact
// products in fp32, in any order and grouping, errs by at most (n - 1) 2^-24
// sum_j |s_j k_j| <= (n - 1) 2^-24 ||S_i|| ||k|| (twice that if every addition
// truncated): 2^-17 ||S_i|| ||k|| for n = 128.  Where |y| is within 2^-15
// ||S_i|| ||k|| of zero (2^-12 for three slices, n = 384), about one element
// in 2^12, the sign is recomputed in fp64 from the registers: each of the
// token's four lanes sums its 32 products and the four partial sums are added.
template <typename InT>
__device__ __forceinline__ void qjl_key_tile(const KeyFrag<InT>& fr, size_t base, size_t rows,
                                             const uint16_t* S_lds, const float (&sbound)[8], size_t my_dst,
                                             uint8_t* __restrict__ sketch, uint16_t* __restrict__ knorm) {
  constexpr int NP = KeyFrag<InT>::NP;
  const int lane = threadIdx.x & 63, col = lane & 15, kq = lane >> 4;
  // token norms: the lane's 32 squares, then the four k-quarters held by lanes
  // col, col+16, col+32, col+48
  double ss = 0.0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double v = (double)fr.value(ks, j);
      ss = fma(v, v, ss);
    }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const double nrm = sqrt(ss);  // lane holds the norm of token `col`
  // Lane t < 16 assembles the sketch of token t: its bits sit in rows t & 3 of
  // the C tiles, lanes 16 (t >> 2) .. 16 (t >> 2) + 15 of each ballot.
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  const int my_q = (lane >> 2) & 3, my_i = lane & 3;
  // the norms and validity of the tokens 4 kq + i whose C rows this lane holds
  float tn[4];
  bool tvalid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tn[i] = (float)__shfl(nrm, kq * 4 + i);
    tvalid[i] = base + kq * 4 + i < rows;
  }
  // S rows in two halves of 64 (n-tiles 4 hf .. 4 hf + 3), sketch words 2 hf, 2 hf + 1
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 pa[NP];
      fr.parts(ks, pa);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int srow = (4 * hf + nt) * 16 + col;
        const uint4 braw = *reinterpret_cast<const uint4*>(&S_lds[srow * kSPad + ks * 32 + kq * 8]);
        const bf16x8 b = __builtin_bit_cast(bf16x8, braw);
#pragma unroll
        for (int p = 0; p < NP; ++p)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[p], b, acc[nt], 0, 0, 0);
      }
    }
    // bit 4 i + nt of sgn: the sign bit of element (token 4 kq + i, S row
    // (4 hf + nt) 16 + col); of close: the element lies within the accumulation
    // error bound of zero, and its sign is then recomputed in fp64 (the whole
    // wave takes part, one element at a time)
    uint32_t close = 0u, sgn = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        close |= (fabsf(acc[nt][i]) <= sbound[4 * hf + nt] * tn[i] && tvalid[i] ? 1u : 0u) << (4 * i + nt);
        sgn |= (acc[nt][i] >= 0.f ? 1u : 0u) << (4 * i + nt);
      }
    if (__ballot(close != 0u)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          unsigned long long todo = __ballot((close >> (4 * i + nt)) & 1u);
          while (todo) {
            const int src = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int ct = (src >> 4) * 4 + i;               // token of that element
            const int sr = (4 * hf + nt) * 16 + (src & 15);  // its row of S
            double e = 0.0;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const uint4 sw = *reinterpret_cast<const uint4*>(&S_lds[sr * kSPad + ks * 32 + kq * 8]);
              const uint32_t w[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float sv = __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
                e = fma((double)sv, (double)fr.value(ks, j), e);
              }
            }
            // each lane: its token's four partial sums, (q0 + q1) + (q2 + q3);
            // token ct's is read from lane ct
            const double tot = add_swapped<32>(add_swapped<16>(e));
            const uint32_t tlo = __builtin_amdgcn_readlane((uint32_t)__builtin_bit_cast(uint64_t, tot), ct);
            const uint32_t thi = __builtin_amdgcn_readlane((uint32_t)(__builtin_bit_cast(uint64_t, tot) >> 32), ct);
            const double tct = __builtin_bit_cast(double, (uint64_t)tlo | ((uint64_t)thi << 32));
            if (lane == src) sgn = (sgn & ~(1u << (4 * i + nt))) | ((tct >= 0.0 ? 1u : 0u) << (4 * i + nt));
          }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unsigned long long bal[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bal[nt] = __ballot((sgn >> (4 * i + nt)) & 1u);
      if (my_i == i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t lo = (uint32_t)(bal[2 * j] >> (16 * my_q)) & 0xFFFFu;
          const uint32_t hi = (uint32_t)(bal[2 * j + 1] >> (16 * my_q)) & 0xFFFFu;
          words[2 * hf + j] = lo | (hi << 16);
        }
      }
    }
  }
  if (lane < 16 && base + lane < rows && my_dst != kNoRow) {
    *reinterpret_cast<uint4*>(sketch + my_dst * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    knorm[my_dst] = f16_from_f64_nonneg(nrm);
  }
}

// QJL keys and FP4 values in one persistent launch.  Each workgroup stages S
// once (bf16 in LDS, with its row norms), then takes 64-token tiles: each wave
// does the values and the keys of 16 tokens, both loaded at the start.
#ifndef KVQ_QJL_APPEND_WAVES_PER_EU
#define KVQ_QJL_APPEND_WAVES_PER_EU 3
#endif

template <typename InT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KVQ_QJL_APPEND_WAVES_PER_EU)))
qjl_append_kernel(const InT* __restrict__ k, const InT* __restrict__ v,
                                                         const float* __restrict__ proj,
                                                         uint8_t* __restrict__ sketch, uint16_t* __restrict__ knorm,
                                                         uint8_t* __restrict__ vc, uint16_t* __restrict__ vs,
                                                         size_t rows, int n, int cap, AppendPos pos) {
  __shared__ __align__(16) uint16_t S_lds[128 * kSPad];
  __shared__ float srow_norm[128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  stage_bf16_matrix(proj, S_lds);  // bf16-valued
  __syncthreads();
  {
    // row norms of S from the staged copy: two threads per row, 64 entries each
    const int r = tid >> 1, h = tid & 1;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 w = *reinterpret_cast<const uint4*>(&S_lds[r * kSPad + 64 * h + 8 * c]);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = __uint_as_float(ww[j] << 16), hi = __uint_as_float(ww[j] & 0xFFFF0000u);
        acc = fmaf(lo, lo, acc);
        acc = fmaf(hi, hi, acc);
      }
    }
    acc += __shfl_xor(acc, 1);
    if (h == 0) srow_norm[r] = sqrtf(acc) * 1.0001f;
  }
  __syncthreads();
  // this lane's sign bounds for S rows nt * 16 + (lane & 15), before the token norm
  float sbound[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
    sbound[nt] = (KeyFrag<InT>::NP == 1 ? 0x1p-15f : 0x1p-12f) * srow_norm[nt * 16 + (lane & 15)];
  const size_t tiles = (rows + 63) / 64;
  const size_t vgroups = rows * 8;
  for (size_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const size_t base = t * 64 + (size_t)wave * 16;
    // cache row of tile row j < 16: one division per tile, then at most one wrap
    // into the next sequence-head when n >= 16
    const size_t bh0 = base / (size_t)n;
    const uint32_t p0 = (uint32_t)(base - bh0 * (size_t)n);
    auto tile_dst = [&](uint32_t j) -> size_t {
      uint32_t p = p0 + j;
      size_t bh = bh0;
      if (n >= 16) {
        if (p >= (uint32_t)n) {
          p -= (uint32_t)n;
          ++bh;
        }
      } else {
        bh += p / (uint32_t)n;
        p %= (uint32_t)n;
      }
      return seq_row(pos, bh, start_of(pos, bh) + (int)p, cap);
    };
    // values first: the 128 groups of rows [base, base + 16), two per lane
    // (group g of the flat row-major input starts at v + 16 g), then the key
    // fragment; the values are encoded and stored while the keys are in flight.
    Raw16<InT> va[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t g = base * 8 + lane + 64 * h;
      if (g < vgroups) va[h].load(v + g * 16);
      else va[h].zero();
    }
    const size_t my_row = base + (lane & 15);
    KeyFrag<InT> fr;
    if (my_row < rows) fr.load(k + my_row * 128, lane >> 4);
    else fr.zero();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t g = base * 8 + lane + 64 * h;
      if (g < vgroups) {
        float a[16];
        va[h].unpack(a);
        fp4_store_at(a, v, tile_dst((lane >> 3) + 8 * h), lane & 7, 128, vc, vs);
      }
    }
    if (base < rows) qjl_key_tile(fr, base, rows, S_lds, sbound, tile_dst(lane & 15), sketch, knorm);
  }
}

// ---------------------------------------------------------------- TurboQuant (fp64 MFMA)

// Keys (WITH_SKETCH) or values: n = ||x||; u = R x / n; idx = #{thresholds <= u};
// keys also r = u - levels[idx], gamma = ||r||, sketch = [S r >= 0].  Both
// products run on v_mfma_f64_16x16x4f64: R and S are bf16-valued and x is
// bf16/fp32, so each product term is exact and the fp64 sums match the
// exact-arithmetic decisions except at exact ties.
template <typename InT, bool WITH_SKETCH>
__device__ __forceinline__ void turbo_body(const InT* __restrict__ x, RotArg ra,
                                           const float* __restrict__ proj, const float* __restrict__ levels,
                                           const float* __restrict__ thresh, uint8_t* __restrict__ codes,
                                           uint8_t* __restrict__ sketch, uint16_t* __restrict__ norm_out,
                                           uint16_t* __restrict__ rnorm_out, size_t rows, int n, int cap,
                                           AppendPos pos, uint16_t* R_lds, uint16_t* S_lds,
                                           double (*scratch)[16 * 129], uint8_t (*idx_lds)[16 * 128]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool dense = ra.kind == KV_ROT_DENSE;
  if (dense) stage_bf16_matrix(ra.rot, R_lds);  // bf16-valued
  if (WITH_SKETCH) stage_bf16_matrix(proj, S_lds);
  __syncthreads();
  const double t0 = thresh[0], t1 = thresh[1], t2 = thresh[2];
  const double lv0 = levels[0], lv1 = levels[1], lv2 = levels[2], lv3 = levels[3];
  double* xs = scratch[wave];
  const int col = lane & 15, kq = lane >> 4;
  for (size_t base = ((size_t)blockIdx.x * 4 + wave) * 16; base < rows; base += (size_t)gridDim.x * 64) {
    // stage 16 tokens x 128 as double, zero past the last row: lane takes token
    // lane / 4, channels 32 (lane % 4) + [0, 32), all loads in flight at once
    // (a structured rotation: channel c at position rot_perm(c), its own inverse)
    {
      const int tk = lane >> 2, c0 = 32 * (lane & 3);
      const bool ok = base + tk < rows;
      float xv[32];
      load32_as_f32(x + (base + (ok ? tk : 0)) * 128 + c0, xv);
#pragma unroll
      for (int j = 0; j < 32; ++j) xs[tk * 129 + (dense ? c0 + j : rot_perm(c0 + j, ra.kind))] = ok ? (double)xv[j] : 0.0;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // norms: lane `col` sums its token over the lane quarter kq, then reduce
    double ss = 0.0;
    for (int c = kq * 32; c < kq * 32 + 32; ++c) ss = fma(xs[col * 129 + c], xs[col * 129 + c], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const double nrm = sqrt(ss);
    // Y = X R^T: A[m = token][k] = x, B[k][n = output row] = R[n][k]
    f64x4 acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = f64x4{0.0, 0.0, 0.0, 0.0};
    if (dense) {
      for (int ks = 0; ks < 32; ++ks) {
        const double a = xs[col * 129 + ks * 4 + kq];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const double b = (double)bf16_to_f32(R_lds[(nt * 16 + col) * kSPad + ks * 4 + kq]);
          acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[nt], 0, 0, 0);
        }
      }
    } else {
      // the butterfly over this wave's 16 tokens in place (the norms above have
      // read them), then y = mag (H x') in the product's element order
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      for (int h = 1; h < 128; h <<= 1) {
        hadamard_stage(xs, 16, 129, h, lane, 64);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
      }
      const double mag = (double)ra.mag;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] = mag * xs[(kq + 4 * i) * 129 + nt * 16 + col];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // quantise: the fp64 16x16x4 product leaves y[token kq + 4i][row nt*16 + col]
    // in element i of this lane's accumulators
    double rr[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = kq + 4 * i;
      const double tn = __shfl(nrm, tok);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const double u = tn > 0.0 ? __ddiv_rn(acc[nt][i], tn) : 0.0;
        const int id = (u >= t0) + (u >= t1) + (u >= t2);
        idx_lds[wave][tok * 128 + nt * 16 + col] = (uint8_t)id;
        if (WITH_SKETCH) {
          const double lv = id == 0 ? lv0 : id == 1 ? lv1 : id == 2 ? lv2 : lv3;
          const double r = u - lv;
          xs[tok * 129 + nt * 16 + col] = r;  // residual replaces x (same wave only)
          rr[i] = fma(r, r, rr[i]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // pack the 2-bit codes: lane < 16 owns token `lane`
    if (lane < 16 && base + lane < rows) {
      const size_t dr = dst_row(base + lane, n, cap, pos);
      const uint8_t* ip = &idx_lds[wave][lane * 128];
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) v |= (uint32_t)ip[j * 16 + b] << (2 * b);
        w[j] = v;
      }
      if (dr != kNoRow) {  // else a page outside the pool
        uint4* dst = reinterpret_cast<uint4*>(codes + dr * 32);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        norm_out[dr] = f16_from_f64_nonneg(nrm);
      }
    }
    if (WITH_SKETCH) {
      // gamma^2 per token: rows are spread over the 16 lanes of each quarter
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double v = rr[i];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        rr[i] = v;
      }
      // S r: A[m = token][k] = r, B[k][n = sketch row] = S[n][k]
      f64x4 sacc[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) sacc[nt] = f64x4{0.0, 0.0, 0.0, 0.0};
      for (int ks = 0; ks < 32; ++ks) {
        const double a = xs[col * 129 + ks * 4 + kq];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const double b = (double)bf16_to_f32(S_lds[(nt * 16 + col) * kSPad + ks * 4 + kq]);
          sacc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, sacc[nt], 0, 0, 0);
        }
      }
      unsigned long long ballots[8][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) ballots[nt][i] = __ballot(sacc[nt][i] >= 0.0);
      // lane (kq, col) holds gamma^2 of token kq + 4i in rr[i]; token `lane` needs it
      double g2 = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double v = __shfl(rr[i], (lane & 3) * 16);
        if ((lane >> 2) == i) g2 = v;
      }
      if (lane < 16 && base + lane < rows) {
        const int q = lane & 3, i = lane >> 2;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t lo = (uint32_t)(ballots[2 * j][i] >> (16 * q)) & 0xFFFFu;
          uint32_t hi = (uint32_t)(ballots[2 * j + 1][i] >> (16 * q)) & 0xFFFFu;
          w[j] = lo | (hi << 16);
        }
        const size_t dr = dst_row(base + lane, n, cap, pos);
        if (dr != kNoRow) {
          *reinterpret_cast<uint4*>(sketch + dr * 16) = make_uint4(w[0], w[1], w[2], w[3]);
          rnorm_out[dr] = f16_from_f64_nonneg(sqrt(g2));
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// TurboQuant keys (blockIdx.y = 0, with the residual sketch) and values
// (blockIdx.y = 1) in one launch; each wave takes 16-token tiles.
template <typename InT>
__global__ void __launch_bounds__(256) turbo_append_kernel(const InT* __restrict__ k, const InT* __restrict__ v,
                                                           RotArg rot,
                                                           const float* __restrict__ proj,
                                                           const float* __restrict__ levels,
                                                           const float* __restrict__ thresh, uint8_t* kc,
                                                           uint8_t* sketch, uint16_t* knorm, uint16_t* krnorm,
                                                           uint8_t* vc, uint16_t* vnorm, size_t rows, int n,
                                                           int cap, AppendPos pos) {
  __shared__ __align__(16) uint16_t R_lds[128 * kSPad];
  __shared__ __align__(16) uint16_t S_lds[128 * kSPad];
  __shared__ double scratch[4][16 * 129];  // per wave: x tile (as double), then the residual
  __shared__ uint8_t idx_lds[4][16 * 128];
  if (blockIdx.y == 0)
    turbo_body<InT, true>(k, rot, proj, levels, thresh, kc, sketch, knorm, krnorm, rows, n, cap, pos, R_lds,
                          S_lds, scratch, idx_lds);
  else
    turbo_body<InT, false>(v, rot, nullptr, levels, thresh, vc, nullptr, vnorm, nullptr, rows, n, cap, pos,
                           R_lds, S_lds, scratch, idx_lds);
}

// Small appends (a few tiles, e.g. one token per sequence): the same
// arithmetic spread for latency rather than staged for throughput.  One
// workgroup of 8 waves per 16-token tile (blockIdx.y = 0 keys, 1 values); wave
// w computes output rows 16 w .. 16 w + 15 of R x (and of S r), reading just
// those rows of R (S) from global memory.  Every product element is summed in
// the same order as in turbo_body, so the codes and signs are the same.
template <typename InT>
__global__ void __launch_bounds__(512) turbo_append_small_kernel(
    const InT* __restrict__ k, const InT* __restrict__ v, RotArg ra,
    const float* __restrict__ proj, const float* __restrict__ levels, const float* __restrict__ thresh,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ sketch, uint16_t* __restrict__ knorm,
    uint16_t* __restrict__ krnorm, uint8_t* __restrict__ vc, uint16_t* __restrict__ vnorm, size_t rows, int n,
    int cap, AppendPos pos) {
  __shared__ double xs[16 * 129];  // x tile as double
  __shared__ double rs[16 * 129];  // keys: the residual
  __shared__ __align__(16) uint16_t rows_lds[8][2][16 * kSPad];  // per wave: its rows of R, then of S (bf16)
  __shared__ double g2part[8][16];  // keys: per-wave partial gamma^2 per token
  __shared__ int starts[kMaxRaggedSeqs];
  fill_starts(pos, starts);
  const bool keys = blockIdx.y == 0;
  const InT* x = keys ? k : v;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const size_t base = (size_t)blockIdx.x * 16;
  // this wave's 16 rows of R (and S, keys only): 8 KB contiguous each, read
  // with full-line loads (lane l, load j: float4 64 j + l of the rows) and kept
  // in LDS as bf16 (both matrices are bf16-valued)
  const bool dense = ra.kind == KV_ROT_DENSE;
  float4 mr[2][8];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (m == 0 ? dense : keys) {  // (a structured rotation has no matrix: ra.rot may be NULL)
      const float4* src = reinterpret_cast<const float4*>((m == 0 ? ra.rot : proj) + 16 * w * 128);
#pragma unroll
      for (int j = 0; j < 8; ++j) mr[m][j] = src[64 * j + lane];
    }
  }
  // x tile: thread t takes token t / 32, channels 4 (t % 32) .. + 3, zero past the last row
  {
    const int tk = tid >> 5, c0 = 4 * (tid & 31);
    const bool ok = base + tk < rows;
    const float4 xv = load4_as_f32(x + (base + (ok ? tk : 0)) * 128 + c0);
    // a structured rotation: channel c at position rot_perm(c)
    const int p0 = dense ? c0 : rot_perm(c0, ra.kind), p1 = dense ? c0 + 1 : rot_perm(c0 + 1, ra.kind);
    const int p2 = dense ? c0 + 2 : rot_perm(c0 + 2, ra.kind), p3 = dense ? c0 + 3 : rot_perm(c0 + 3, ra.kind);
    xs[tk * 129 + p0] = ok ? (double)xv.x : 0.0;
    xs[tk * 129 + p1] = ok ? (double)xv.y : 0.0;
    xs[tk * 129 + p2] = ok ? (double)xv.z : 0.0;
    xs[tk * 129 + p3] = ok ? (double)xv.w : 0.0;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (m == 0 ? dense : keys) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = 64 * j + lane, r = f >> 5, c4 = 4 * (f & 31);
        uint2 h;
        h.x = (__float_as_uint(mr[m][j].x) >> 16) | (__float_as_uint(mr[m][j].y) & 0xFFFF0000u);
        h.y = (__float_as_uint(mr[m][j].z) >> 16) | (__float_as_uint(mr[m][j].w) & 0xFFFF0000u);
        *reinterpret_cast<uint2*>(&rows_lds[w][m][r * kSPad + c4]) = h;
      }
    }
  }
  __syncthreads();
  // norms (every wave, same order as turbo_body): lane `col` sums its token over
  // the quarter kq, then the quarters are added
  double ss = 0.0;
  for (int c = kq * 32; c < kq * 32 + 32; ++c) ss = fma(xs[col * 129 + c], xs[col * 129 + c], ss);
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const double nrm = sqrt(ss);
  f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
  if (dense) {
    const uint16_t* Rw = &rows_lds[w][0][col * kSPad + kq];
#pragma unroll
    for (int ks = 0; ks < 32; ++ks)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xs[col * 129 + ks * 4 + kq], (double)bf16_to_f32(Rw[4 * ks]),
                                                 acc, 0, 0, 0);
  } else {
    // the butterfly over all 16 tokens in place once every wave has read its
    // norms, then y = mag (H x') for this wave's rows in the product's order
    __syncthreads();
    for (int h = 1; h < 128; h <<= 1) {
      hadamard_stage(xs, 16, 129, h, tid, 512);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = (double)ra.mag * xs[(kq + 4 * i) * 129 + 16 * w + col];
  }
  const double t0 = thresh[0], t1 = thresh[1], t2 = thresh[2];
  const double lv0 = levels[0], lv1 = levels[1], lv2 = levels[2], lv3 = levels[3];
  // element i of acc is y[token kq + 4 i][row 16 w + col]; the 2-bit codes of
  // rows 16 w .. 16 w + 15 form word w of each token's code row (row 16 w + b
  // in bits 2 b), gathered across the 16 lanes of a quarter
  uint8_t* codes = keys ? kc : vc;
  double rr[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = kq + 4 * i;
    const double tn = __shfl(nrm, tok);
    const double u = tn > 0.0 ? __ddiv_rn(acc[i], tn) : 0.0;
    const int id = (u >= t0) + (u >= t1) + (u >= t2);
    uint32_t word = (uint32_t)id << (2 * col);
    word |= __shfl_xor(word, 1);
    word |= __shfl_xor(word, 2);
    word |= __shfl_xor(word, 4);
    word |= __shfl_xor(word, 8);
    if (col == 0 && base + tok < rows) {
      const size_t dr = dst_row_tab(base + tok, n, cap, pos, starts);
      if (dr != kNoRow) *reinterpret_cast<uint32_t*>(codes + dr * 32 + 4 * w) = word;
    }
    if (keys) {
      const double lv = id == 0 ? lv0 : id == 1 ? lv1 : id == 2 ? lv2 : lv3;
      const double r = u - lv;
      rs[tok * 129 + 16 * w + col] = r;
      rr[i] = r * r;
    }
  }
  if (keys) {
    // this wave's 16 columns of gamma^2 per token
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double t = rr[i];
      t += __shfl_xor(t, 1);
      t += __shfl_xor(t, 2);
      t += __shfl_xor(t, 4);
      t += __shfl_xor(t, 8);
      if (col == 0) g2part[w][kq + 4 * i] = t;
    }
  }
  if (w == 0 && lane < 16 && base + lane < rows) {
    const size_t dr = dst_row_tab(base + lane, n, cap, pos, starts);
    if (dr != kNoRow) (keys ? knorm : vnorm)[dr] = f16_from_f64_nonneg(nrm);
  }
  if (!keys) return;
  __syncthreads();
  // S r for sketch rows 16 w .. 16 w + 15
  f64x4 sacc = f64x4{0.0, 0.0, 0.0, 0.0};
  const uint16_t* Sw = &rows_lds[w][1][col * kSPad + kq];
#pragma unroll
  for (int ks = 0; ks < 32; ++ks)
    sacc = __builtin_amdgcn_mfma_f64_16x16x4f64(rs[col * 129 + ks * 4 + kq], (double)bf16_to_f32(Sw[4 * ks]), sacc,
                                                0, 0, 0);
  // token t's bits for these rows: lanes 16 (t % 4) .. + 15 of ballot t / 4, bit
  // col = row 16 w + col, i.e. bytes 2 w and 2 w + 1 of its sketch
  uint32_t my_bits = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned long long bal = __ballot(sacc[i] >= 0.0);
    if ((lane >> 2) == i) my_bits = (uint32_t)(bal >> (16 * (lane & 3))) & 0xFFFFu;
  }
  if (lane < 16 && base + lane < rows) {
    const size_t dr = dst_row_tab(base + lane, n, cap, pos, starts);
    if (dr != kNoRow) *reinterpret_cast<uint16_t*>(sketch + dr * 16 + 2 * w) = (uint16_t)my_bits;
    if (w == 0 && dr != kNoRow) {
      double g2 = 0.0;
      for (int ww = 0; ww < 8; ++ww) g2 += g2part[ww][lane];
      krnorm[dr] = f16_from_f64_nonneg(sqrt(g2));
    }
  }
}

// bf16 copies of appended tokens for a mixed-precision cache.  Append token tt
// (of n) of sequence-head bh lands at position t = start_of(bh) + tt; it goes to
// slot t of the sink when t < S, and to slot t mod W of the recent ring when it
// is one of the append's last W tokens.  Virtual index v < Sn = min(n, S) is
// sink candidate tt = v; v >= Sn is ring token tt = n - Wn + (v - Sn), Wn =
// min(n, W).  Eight channels per thread; fp32 inputs round to nearest even.
template <typename InT>
__global__ void __launch_bounds__(256) window_copy_kernel(const InT* __restrict__ k, const InT* __restrict__ v,
                                                          int d, uint16_t* __restrict__ sk, uint16_t* __restrict__ sv,
                                                          uint16_t* __restrict__ rk, uint16_t* __restrict__ rv,
                                                          int S, int W, int bh_count, int n, AppendPos pos) {
  __shared__ int starts[kMaxRaggedSeqs];
  fill_starts(pos, starts);
  const int per_row = d / 8, Sn = min(n, S), Wn = min(n, W), nv = Sn + Wn;
  const size_t half = (size_t)bh_count * nv * per_row;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < 2 * half; i += (size_t)gridDim.x * 256) {
    const bool is_v = i >= half;
    const size_t j = is_v ? i - half : i;
    const int c8 = (int)(j % per_row) * 8;
    const int vi = (int)((j / per_row) % nv);
    const size_t bh = j / ((size_t)per_row * nv);
    const bool sink = vi < Sn;
    const int tt = sink ? vi : n - Wn + (vi - Sn);
    const int t = start_tab(pos, starts, bh) + tt;
    if (sink && t >= S) continue;  // past the sink
    const InT* src = (is_v ? v : k) + (bh * n + tt) * d + c8;
    uint32_t w[4];
    if constexpr (std::is_same<InT, uint16_t>::value) {
      const uint4 r = *reinterpret_cast<const uint4*>(src);
      w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
    } else {
      const float4 x0 = *reinterpret_cast<const float4*>(src), x1 = *reinterpret_cast<const float4*>(src + 4);
      const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo = __float_as_uint(f[2 * e]), hi = __float_as_uint(f[2 * e + 1]);
        lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
        hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
        w[e] = lo | (hi << 16);
      }
    }
    uint16_t* dst = sink ? (is_v ? sv : sk) + (bh * S + t) * d + c8 : (is_v ? rv : rk) + (bh * W + t % W) * d + c8;
    *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
  }
}

int blocks_for(size_t threads) { return (int)((threads + 255) / 256); }

// Workgroups of the QJL append: one resident round (each stages S once).
#ifndef KVQ_QJL_APPEND_BLOCKS
#define KVQ_QJL_APPEND_BLOCKS (256 * KVQ_QJL_APPEND_WAVES_PER_EU)
#endif

// Appends of at most this many rows take the latency-bound TurboQuant kernel.
constexpr size_t kTurboSmallRows = 2048;

int persistent_blocks(size_t rows) {
  size_t tiles = (rows + 63) / 64;
  return (int)std::min<size_t>(tiles, 2048);
}

template <typename InT>
int append_typed(const kv_cache* c, const InT* k, const InT* v, const AppendPos& pos, int n, hipStream_t st) {
  const kv_layout& L = c->layout;
  const int d = L.head_dim, cap = L.capacity;
  const int bh = L.batch * L.num_kv_heads;
  const size_t rows = (size_t)bh * n;
  auto* kc = static_cast<uint8_t*>(c->buf[KV_BUF_K_CODES]);
  auto* ks = static_cast<uint16_t*>(c->buf[KV_BUF_K_SCALE]);
  auto* vc = static_cast<uint8_t*>(c->buf[KV_BUF_V_CODES]);
  auto* vs = static_cast<uint16_t*>(c->buf[KV_BUF_V_SCALE]);
  switch (L.format) {
    case KV_FMT_FP4:
      fp4_append_kernel<InT><<<dim3(blocks_for(rows * (d / 16)), 2), 256, 0, st>>>(k, v, d, kc, ks, vc, vs, rows,
                                                                                  n, cap, pos);
      break;
    case KV_FMT_LATENT_FP4: {
      const size_t work = std::max(rows * (d / 16), rows * (size_t)L.rope_dim);
      latent_append_kernel<InT><<<dim3(blocks_for(work), 2), 256, 0, st>>>(
          k, d, L.rope_dim, kc, ks, static_cast<uint16_t*>(c->buf[KV_BUF_ROPE]), rows, n, cap, pos);
      break;
    }
    case KV_FMT_KIVI2: {
      bool aligned = n % 32 == 0 && pos.start % 32 == 0;
      for (int b = 0; pos.ragged && b < L.batch; ++b) aligned = aligned && pos.s[b] % 32 == 0;
      if (!aligned) {
        for (int phase = 0; phase < 2; ++phase)  // code from the old staging, then replace it
          kivi_append_any_kernel<InT><<<dim3(bh * (n / 32 + 2)), 256, 0, st>>>(
              k, v, d, kc, static_cast<float*>(c->buf[KV_BUF_K_SCALE]), static_cast<float*>(c->buf[KV_BUF_K_ZERO]),
              vc, static_cast<float*>(c->buf[KV_BUF_V_SCALE]), static_cast<float*>(c->buf[KV_BUF_V_ZERO]),
              static_cast<float*>(c->buf[KV_BUF_K_STAGE]), n, cap, pos, phase);
        break;
      }
      kivi_append_kernel<InT><<<dim3(bh * (n / 32)), 256, 0, st>>>(
          k, v, d, kc, static_cast<float*>(c->buf[KV_BUF_K_SCALE]), static_cast<float*>(c->buf[KV_BUF_K_ZERO]),
          vc, static_cast<float*>(c->buf[KV_BUF_V_SCALE]), static_cast<float*>(c->buf[KV_BUF_V_ZERO]),
          static_cast<float*>(c->buf[KV_BUF_K_STAGE]), bh, n, cap, pos);
      break;
    }
    case KV_FMT_QJL1_FP4V: {
      const int blocks = (int)std::min<size_t>((rows + 63) / 64, KVQ_QJL_APPEND_BLOCKS);
      qjl_append_kernel<InT><<<blocks, 256, 0, st>>>(
          k, v, c->proj, static_cast<uint8_t*>(c->buf[KV_BUF_K_SKETCH]), static_cast<uint16_t*>(c->buf[KV_BUF_K_NORM]),
          vc, vs, rows, n, cap, pos);
      break;
    }
    case KV_FMT_TURBO:
      if (rows <= kTurboSmallRows) {
        turbo_append_small_kernel<InT><<<dim3((unsigned)((rows + 15) / 16), 2), 512, 0, st>>>(
            k, v, rot_arg(c), c->proj, c->lm_levels, c->lm_thresh, kc, static_cast<uint8_t*>(c->buf[KV_BUF_K_SKETCH]),
            static_cast<uint16_t*>(c->buf[KV_BUF_K_NORM]), static_cast<uint16_t*>(c->buf[KV_BUF_K_RNORM]), vc,
            static_cast<uint16_t*>(c->buf[KV_BUF_V_NORM]), rows, n, cap, pos);
        break;
      }
      turbo_append_kernel<InT><<<dim3(persistent_blocks(rows), 2), 256, 0, st>>>(
          k, v, rot_arg(c), c->proj, c->lm_levels, c->lm_thresh, kc, static_cast<uint8_t*>(c->buf[KV_BUF_K_SKETCH]),
          static_cast<uint16_t*>(c->buf[KV_BUF_K_NORM]), static_cast<uint16_t*>(c->buf[KV_BUF_K_RNORM]), vc,
          static_cast<uint16_t*>(c->buf[KV_BUF_V_NORM]), rows, n, cap, pos);
      break;
    default:
      return KV_EUNSUPPORTED;
  }
  // mixed precision: bf16 copies of the sink tokens and of the append's last
  // recent_tokens tokens (older ring slots are overwritten by later appends)
  if (L.sink_tokens || L.recent_tokens) {
    const size_t items = 2 * (size_t)bh * (std::min(n, L.sink_tokens) + std::min(n, L.recent_tokens)) * (d / 8);
    window_copy_kernel<InT><<<blocks_for(items), 256, 0, st>>>(
        k, v, d, static_cast<uint16_t*>(c->buf[KV_BUF_SINK_K]), static_cast<uint16_t*>(c->buf[KV_BUF_SINK_V]),
        static_cast<uint16_t*>(c->buf[KV_BUF_RECENT_K]), static_cast<uint16_t*>(c->buf[KV_BUF_RECENT_V]),
        L.sink_tokens, L.recent_tokens, bh, n, pos);
  }
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}

}  // namespace

int launch_append(const kv_cache* c, const void* k, const void* v, int in_dtype, int start, const int32_t* starts,
                  int n_new, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const kv_layout& L = c->layout;
  const bool latent = L.format == KV_FMT_LATENT_FP4;
  const int heads = latent ? 1 : L.num_kv_heads;
  const size_t in_row = (size_t)L.head_dim + (latent ? L.rope_dim : 0);
  const size_t in_seq_bytes = (size_t)heads * n_new * in_row * (in_dtype == KV_DT_F32 ? 4 : 2);
  // per-sequence starts travel by value, kMaxRaggedSeqs sequences per launch;
  // a launch over sequences [b0, b0 + nb) sees them as a cache of nb sequences
  const int chunk = starts ? kMaxRaggedSeqs : L.batch;
  for (int b0 = 0; b0 < L.batch; b0 += chunk) {
    const int nb = std::min(chunk, L.batch - b0);
    kv_cache sub = *c;
    sub.layout.batch = nb;
    // a paged pool is shared by every sequence: only the per-sequence buffers
    // (windows, staging) and the block table move
    const bool paged = L.page_tokens > 0;
    for (int i = 0; i < KV_BUF_COUNT; ++i)
      if (c->buf[i] && !(paged && i < KV_BUF_SINK_K))
        sub.buf[i] = static_cast<char*>(c->buf[i]) + (size_t)b0 * (kv_buffer_bytes(&L, i) / L.batch);
    if (paged) sub.block_table = c->block_table + (size_t)b0 * (L.capacity / L.page_tokens);
    AppendPos pos{};
    pos.start = start;
    pos.ragged = starts ? 1 : 0;
    pos.heads = heads;
    pos.pm = page_map(&sub);
    for (int b = 0; starts && b < nb; ++b) pos.s[b] = starts[b0 + b];
    const char* kb = static_cast<const char*>(k) + (size_t)b0 * in_seq_bytes;
    const char* vb = v ? static_cast<const char*>(v) + (size_t)b0 * in_seq_bytes : nullptr;
    const int rc = in_dtype == KV_DT_F32
                       ? append_typed<float>(&sub, reinterpret_cast<const float*>(kb),
                                             reinterpret_cast<const float*>(vb), pos, n_new, st)
                       : append_typed<uint16_t>(&sub, reinterpret_cast<const uint16_t*>(kb),
                                                reinterpret_cast<const uint16_t*>(vb), pos, n_new, st);
    if (rc != KV_OK) return rc;
  }
  return KV_OK;
}

}  // namespace kvq
