// Device-side helpers for the libkvq kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

// ---------------------------------------------------------------- token rows

constexpr size_t kNoRow = ~size_t(0);

// Pool page of sequence b's position t, or -1 when its table entry names no
// page of the pool (such a page is never read or written).
__device__ __forceinline__ int page_of(const PageMap& m, int b, int t) {
  if (!m.table) return b;
  const int p = m.table[(size_t)b * m.per_seq + (t >> m.shift)];
  return (unsigned)p < (unsigned)m.num_pages ? p : -1;
}

// page_of for a wave-uniform (b, t) of a paged map, read through the scalar
// cache (the table is read-only in every kernel, so it may be read as constant
// memory): waiting for it does not wait for the wave's vector loads in flight,
// which the decode kernels keep across the lookup of their next tile.
typedef __attribute__((address_space(4))) const int32_t const_i32;
// The raw entry (not yet checked against the pool, so that the read can stay in
// flight until the page is used) ...
__device__ __forceinline__ int page_entry_uniform(const PageMap& m, int b, int t) {
  const int32_t* p = m.table + (size_t)b * m.per_seq + (t >> m.shift);
  return *reinterpret_cast<const_i32*>(reinterpret_cast<uintptr_t>(p));
}
// ... and the checked page, or -1.
__device__ __forceinline__ int page_checked(const PageMap& m, int entry) {
  return (unsigned)entry < (unsigned)m.num_pages ? entry : -1;
}
__device__ __forceinline__ int page_of_uniform(const PageMap& m, int b, int t) {
  return page_checked(m, page_entry_uniform(m, b, t));
}

// Token row of (sequence b, head h of H, position t) in a per-token buffer, or
// kNoRow.  KIVI key metadata rows are token row / 32 (pages hold whole groups).
__device__ __forceinline__ size_t token_row(const PageMap& m, int H, int b, int h, int t) {
  if (!m.table) return ((size_t)b * H + h) * m.tokens + t;
  const int p = page_of(m, b, t);
  if (p < 0) return kNoRow;
  return ((size_t)p * H + h) * m.tokens + (t & (m.tokens - 1));
}

// ---------------------------------------------------------------- 16-bit floats

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Nearest bf16 of a finite double, ties to even; returns the bit pattern.
__device__ __forceinline__ uint16_t bf16_from_f64(double x) {
  if (x == 0.0) return (uint16_t)(__double_as_longlong(x) >> 48);  // keeps -0
  double a = fabs(x);
  float f;
  if (a < 0x1p-126) {
    f = (float)(rint(a * 0x1p133) * 0x1p-133);
  } else {
    unsigned long long u = (unsigned long long)__double_as_longlong(a);
    unsigned long long lsb = (u >> 45) & 1ull;
    u += (1ull << 44) - 1ull + lsb;
    u &= ~((1ull << 45) - 1ull);
    f = (float)__longlong_as_double((long long)u);
  }
  uint16_t bits = (uint16_t)(__float_as_uint(f) >> 16);
  return x < 0 ? (uint16_t)(bits | 0x8000u) : bits;
}

// Nearest fp16 of a non-negative finite double (a norm), ties to even; bit pattern.
__device__ __forceinline__ uint16_t f16_from_f64_nonneg(double a) {
  if (a == 0.0) return 0;
  if (a < 0x1p-14) {  // subnormal: spacing 2^-24
    double q = rint(a * 0x1p24);
    return (uint16_t)q;  // q <= 1024; 1024 is the smallest normal's pattern 0x0400
  }
  unsigned long long u = (unsigned long long)__double_as_longlong(a);
  unsigned long long lsb = (u >> 42) & 1ull;
  u += (1ull << 41) - 1ull + lsb;
  u &= ~((1ull << 42) - 1ull);
  double r = __longlong_as_double((long long)u);
  if (r > 65504.0) return 0x7C00;  // +inf
  int e = (int)((u >> 52) & 0x7FF) - 1023;           // 2^e <= r < 2^(e+1), e >= -14
  unsigned frac = (unsigned)((u >> 42) & 0x3FF);
  return (uint16_t)(((e + 15) << 10) | frac);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- E2M1

// E2M1 magnitudes by code 0..7.
__device__ __forceinline__ float e2m1_mag(uint32_t i) {
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6
  const float t[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  return t[i & 7];
}

__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  float m = e2m1_mag(nib);
  return (nib & 8) ? -m : m;
}

// Nibble of x with scale s > 0: nearest value to |x|/s, exact ties to the even
// code, saturating at 6, sign bit from x.  The midpoints times s are exact in
// fp32 (at most 11 significant bits), so every comparison is exact.
__device__ __forceinline__ uint32_t e2m1_encode(float x, float s) {
  const float ax = fabsf(x);
  uint32_t idx = 0;
  idx += (ax > 0.25f * s);
  idx += (ax >= 0.75f * s);  // tie between codes 1 and 2 goes up (to even 2)
  idx += (ax > 1.25f * s);
  idx += (ax >= 1.75f * s);
  idx += (ax > 2.5f * s);
  idx += (ax >= 3.5f * s);
  idx += (ax > 5.0f * s);
  return idx | (__float_as_uint(x) >> 31 << 3);
}

// ---------------------------------------------------------------- input loads

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ---------------------------------------------------------------- cross-row lane exchange

// max of x over lanes l and l ^ 16 (l ^ 32), in registers: v_permlane16_swap
// (v_permlane32_swap) of x with itself leaves the two lanes' values in the two
// halves of the result, in either order.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------- structured rotation

// The structured rotation R = mag H P (page "TurboQuant vs OSCAR vs EpiCache",
// section "quantization frontiers", the OSCAR paragraph: a Hadamard transform
// behind a bit-reversal permutation): (R x)[i] = mag sum_k (-1)^popcount(i & k)
// x[rev(k)], and (R^T y)[j] = mag (H y)[rev(j)], rev the reversal of the seven
// index bits of a 128-channel row (the identity for KV_ROT_HADAMARD).
__device__ __forceinline__ int rot_perm(int k, int kind) {
  return kind == KV_ROT_HADAMARD_BITREV ? (int)(__builtin_bitreverse32((uint32_t)k) >> 25) : k;
}

// Stage h (1, 2, 4, ..., 64) of the in-place Walsh-Hadamard butterfly over
// `rows` rows of 128 values at x + r * pitch: butterfly p (of rows * 64) pairs
// positions i and i + h, i the p % 64-th index whose bit h is clear, taken by
// the calling thread for p = first, first + step, ...  After the seven stages
// row r holds H times what it held (Sylvester order, unnormalised).  The caller
// orders the stages (a barrier between them).
template <typename T>
__device__ __forceinline__ void hadamard_stage(T* x, int rows, int pitch, int h, int first, int step) {
  for (int p = first; p < rows * 64; p += step) {
    const int b = p & 63;
    const int i = ((b & ~(h - 1)) << 1) | (b & (h - 1));
    T* v = x + (size_t)(p >> 6) * pitch;
    const T a = v[i], c = v[i + h];
    v[i] = a + c;
    v[i + h] = a - c;
  }
}

}  // namespace kvq
