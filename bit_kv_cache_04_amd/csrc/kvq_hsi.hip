// Hierarchical sparse indexing (page "How DeepSeek-V4.1-Flash cut KV-cache
// storage by 4x via CSA2", HSI section): the candidate pool of the full-mode
// layer (block maxima over `block` positions, the top blocks) and the top-k of a
// reindex-mode layer over that pool.  Scores are inputs (the indexer is a model
// component).  A radix select finds the k-th largest key in four 8-bit passes,
// then one pass in index order keeps every larger key and the earliest of the
// equal ones, so the output comes out in ascending order.  One workgroup
// selects for one sequence, or, for pools over sequences longer than
// kSelLdsKeys blocks, many workgroups do (global histograms, per-chunk counts
// and bases, ordered emits per chunk).
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelLdsKeys = 16384;  // key sets up to this size are staged in LDS
constexpr int kPer = 8;             // consecutive keys a thread takes per step
static_assert(kSelLdsKeys >= kSelThreads * kPer, "a step's keys fit the staging array");

// Order-preserving key of a finite fp32 score: a larger score has a larger key,
// and -0 reads as +0 (equal scores, equal keys).  Every key is nonzero.
__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one int per thread over the workgroup, and the total.
__device__ __forceinline__ int wg_exclusive_scan(int v, int& total) {
  __shared__ int wsum[kSelWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = wsum[w];
    before += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();  // wsum is reused by the next scan
  total = tot;
  return before + x - v;
}

// The k-th largest of the n keys key_at(i) (1 <= k <= n) and how many of the
// keys equal to it are among the k largest.
template <class KeyAt>
__device__ void radix_threshold(const KeyAt& key_at, int n, int k, uint32_t& thr, int& take_eq) {
  __shared__ int hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    // kPer keys per thread and step, read coalesced (key base + j * threads +
    // thread) and in flight together (a histogram needs no order)
    for (int base = 0; base < n; base += kSelThreads * kPer) {
      uint32_t u[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = base + j * kSelThreads + threadIdx.x;
        u[j] = i < n ? key_at(i) : 0u;
      }
      // the keys mostly share a few bins (scores crowd, and same-address LDS
      // atomics serialise): one atomic per run of equal bins
      int run_bin = -1, run_cnt = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = base + j * kSelThreads + threadIdx.x;
        const int bin = i < n && (u[j] & mask) == prefix ? (int)((u[j] >> shift) & 255u) : -1;
        if (bin != run_bin) {
          if (run_cnt) atomicAdd(&hist[run_bin], run_cnt);
          run_bin = bin;
          run_cnt = 0;
        }
        run_cnt += bin >= 0;
      }
      if (run_cnt) atomicAdd(&hist[run_bin], run_cnt);
    }
    __syncthreads();
    // bins from the top: thread i holds bin 255 - i; the bin where the running
    // count reaches krem holds the k-th largest
    const int v = threadIdx.x < 256 ? hist[255 - threadIdx.x] : 0;
    int tot;
    const int before = wg_exclusive_scan(v, tot);
    if (threadIdx.x < 256 && before < krem && before + v >= krem) {
      s_prefix = prefix | ((uint32_t)(255 - threadIdx.x) << shift);
      s_krem = krem - before;
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 255u << shift;
    __syncthreads();  // hist and the shared results are reused by the next pass
  }
  thr = prefix;
  take_eq = krem;
}

// One pass in index order: item i is kept if its key exceeds thr, or equals it
// and fewer than take_eq equal keys come before it.  emit(i, off) receives the
// kept items in order with off the running sum of weight() over the kept items
// before i.  Each thread takes kPer consecutive items per step; with `chunk`
// (LDS room for kSelThreads * kPer keys) a step's keys are first read coalesced
// into it.  Returns the total weight kept.
template <class KeyAt, class Weight, class Emit>
__device__ int emit_selected(const KeyAt& key_at, const Weight& weight, const Emit& emit, int n, uint32_t thr,
                             int take_eq, uint32_t* chunk = nullptr, int run_eq = 0, int run_out = 0) {
  for (int base = 0; base < n; base += kSelThreads * kPer) {
    const int i0 = base + threadIdx.x * kPer;
    if (chunk) {
      uint32_t x[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = base + j * kSelThreads + threadIdx.x;
        x[j] = i < n ? key_at(i) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) chunk[j * kSelThreads + threadIdx.x] = x[j];
      __syncthreads();  // (the scans below keep the next step's writes after these reads)
    }
    uint32_t u[kPer];
    int c_eq = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      u[j] = chunk ? chunk[threadIdx.x * kPer + j] : i0 + j < n ? key_at(i0 + j) : 0u;  // 0: below every key
      c_eq += u[j] == thr;
    }
    int tot_eq, tot_w;
    int eq_rank = run_eq + wg_exclusive_scan(c_eq, tot_eq);
    bool keep[kPer];
    int c_w = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool eq = u[j] == thr;
      keep[j] = u[j] > thr || (eq && eq_rank < take_eq);
      eq_rank += eq;
      c_w += keep[j] ? weight(i0 + j) : 0;
    }
    int off = run_out + wg_exclusive_scan(c_w, tot_w);
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (keep[j]) {
        emit(i0 + j, off);
        off += weight(i0 + j);
      }
    run_eq += tot_eq;
    run_out += tot_w;
  }
  return run_out;
}

// Key of the largest score of each block of `blk` positions below L: thread j of
// sequence b (blockIdx.y) takes block j.
__global__ void __launch_bounds__(256) hsi_block_max_kernel(const float* __restrict__ scores, int stride,
                                                            const int32_t* __restrict__ seq_lens, int blk,
                                                            int nb_stride, uint32_t* __restrict__ keys) {
  const int b = blockIdx.y;
  const int L = min(max(seq_lens[b], 0), stride);
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j * blk >= L) return;
  const float* s = scores + (size_t)b * stride + (size_t)j * blk;
  const int n = min(blk, L - j * blk);
  float m = s[0];
  for (int i = 1; i < n; ++i) m = fmaxf(m, s[i]);
  keys[(size_t)b * nb_stride + j] = score_key(m);
}

// Candidate pool of sequence b (blockIdx.x): the positions of its top_blocks
// blocks with the largest keys (all when it has fewer), ascending.
__global__ void __launch_bounds__(kSelThreads) hsi_pool_kernel(const uint32_t* __restrict__ keys, int nb_stride,
                                                               const int32_t* __restrict__ seq_lens, int stride,
                                                               int blk, int top_blocks, int32_t* __restrict__ pool,
                                                               int pool_cap, int32_t* __restrict__ pool_n) {
  const int b = blockIdx.x;
  const int L = min(max(seq_lens[b], 0), stride);
  const int nb = (L + blk - 1) / blk;
  __shared__ uint32_t lk[kSelLdsKeys];
  const uint32_t* kb = keys + (size_t)b * nb_stride;
  int32_t* out = pool + (size_t)b * pool_cap;
  const bool staged = nb <= kSelLdsKeys;
  if (staged) {
    for (int base = 0; base < nb; base += kSelThreads * kPer) {
      uint32_t x[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) x[j] = base + j * kSelThreads + threadIdx.x < nb ? kb[base + j * kSelThreads + threadIdx.x] : 0u;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (base + j * kSelThreads + threadIdx.x < nb) lk[base + j * kSelThreads + threadIdx.x] = x[j];
    }
    __syncthreads();
  }
  auto key_at = [&](int j) { return staged ? lk[j] : kb[j]; };
  uint32_t thr = 0;  // every key exceeds 0: all blocks kept
  int take = 0;
  if (top_blocks < nb) radix_threshold(key_at, nb, top_blocks, thr, take);
  const int total = emit_selected(
      key_at, [&](int j) { return min(blk, L - j * blk); },
      [&](int j, int off) {
        const int c = min(blk, L - j * blk);
        for (int r = 0; r < c; ++r) out[off + r] = j * blk + r;
      },
      nb, thr, take, staged ? nullptr : lk);
  if (threadIdx.x == 0) pool_n[b] = total;
}

// Top-k of sequence b's pool entries by score (all when fewer), as positions in
// pool order (ascending).
__global__ void __launch_bounds__(kSelThreads) hsi_select_kernel(const float* __restrict__ pool_scores,
                                                                 const int32_t* __restrict__ pool,
                                                                 const int32_t* __restrict__ pool_n, int pool_cap,
                                                                 int top_k, int32_t* __restrict__ sel,
                                                                 int32_t* __restrict__ sel_n) {
  __shared__ uint32_t lk[kSelLdsKeys];
  const int b = blockIdx.x;
  const int n = min(max(pool_n[b], 0), pool_cap);
  const float* sc = pool_scores + (size_t)b * pool_cap;
  const int32_t* pb = pool + (size_t)b * pool_cap;
  int32_t* out = sel + (size_t)b * top_k;
  const bool staged = n <= kSelLdsKeys;
  if (staged) {
    for (int base = 0; base < n; base += kSelThreads * kPer) {
      float x[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) x[j] = base + j * kSelThreads + threadIdx.x < n ? sc[base + j * kSelThreads + threadIdx.x] : 0.f;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (base + j * kSelThreads + threadIdx.x < n) lk[base + j * kSelThreads + threadIdx.x] = score_key(x[j]);
    }
    __syncthreads();
  }
  auto key_at = [&](int i) { return staged ? lk[i] : score_key(sc[i]); };
  uint32_t thr = 0;
  int take = 0;
  if (top_k < n) radix_threshold(key_at, n, top_k, thr, take);
  const int total = emit_selected(
      key_at, [](int) { return 1; }, [&](int i, int off) { out[off] = pb[i]; }, n, thr, take);
  if (threadIdx.x == 0) sel_n[b] = total;
}

// ---------------------------------------------------------------- many workgroups per sequence
//
// For long sequences (more than kSelLdsKeys blocks) the pool is selected by
// kChunk-key chunks, one workgroup each, in kernels that follow each other on
// the stream: four histogram passes into a global histogram, each closed by a
// one-workgroup pick of the bin; then per-chunk counts, a scan over chunks and
// an ordered emit per chunk.  State per sequence (in the workspace):
//   st[0] prefix, st[1] keys still to take, st[2] 1 when every block is kept.
constexpr int kChunk = kSelThreads * kPer;  // keys per workgroup

__device__ __forceinline__ int blocks_of(const int32_t* seq_lens, int b, int stride, int blk) {
  return (min(max(seq_lens[b], 0), stride) + blk - 1) / blk;
}

__global__ void __launch_bounds__(256) hsi_multi_init_kernel(const int32_t* __restrict__ seq_lens, int stride,
                                                             int blk, int top_blocks, int* __restrict__ ghist,
                                                             int* __restrict__ state) {
  const int b = blockIdx.x;
  ghist[(size_t)b * 256 + threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    const int nb = blocks_of(seq_lens, b, stride, blk);
    state[4 * b] = 0;
    state[4 * b + 1] = min(top_blocks, nb);
    state[4 * b + 2] = top_blocks >= nb ? 1 : 0;
  }
}

// Histogram pass: chunk blockIdx.x of sequence blockIdx.y, keys matching the
// prefix so far in their top 8 * pass bits.
__global__ void __launch_bounds__(kSelThreads) hsi_multi_hist_kernel(const uint32_t* __restrict__ keys, int nb_stride,
                                                                     const int32_t* __restrict__ seq_lens, int stride,
                                                                     int blk, int pass, int* __restrict__ ghist,
                                                                     const int* __restrict__ state) {
  __shared__ int hist[256];
  const int b = blockIdx.y;
  if (state[4 * b + 2]) return;  // every block kept
  const int nb = blocks_of(seq_lens, b, stride, blk);
  const int base = blockIdx.x * kChunk;
  if (base >= nb) return;
  const uint32_t prefix = (uint32_t)state[4 * b];
  const int shift = 24 - 8 * pass;
  const uint32_t mask = pass == 0 ? 0u : ~0u << (32 - 8 * pass);
  if (threadIdx.x < 256) hist[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t* kb = keys + (size_t)b * nb_stride;
  uint32_t u[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = base + j * kSelThreads + threadIdx.x;
    u[j] = i < nb ? kb[i] : 0u;
  }
  int run_bin = -1, run_cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = base + j * kSelThreads + threadIdx.x;
    const int bin = i < nb && (u[j] & mask) == prefix ? (int)((u[j] >> shift) & 255u) : -1;
    if (bin != run_bin) {
      if (run_cnt) atomicAdd(&hist[run_bin], run_cnt);
      run_bin = bin;
      run_cnt = 0;
    }
    run_cnt += bin >= 0;
  }
  if (run_cnt) atomicAdd(&hist[run_bin], run_cnt);
  __syncthreads();
  if (threadIdx.x < 256 && hist[threadIdx.x]) atomicAdd(&ghist[(size_t)b * 256 + threadIdx.x], hist[threadIdx.x]);
}

// Close a pass: the bin holding the k-th largest key extends the prefix; the
// histogram is cleared for the next pass.
__global__ void __launch_bounds__(256) hsi_multi_pick_kernel(int pass, int* __restrict__ ghist,
                                                             int* __restrict__ state) {
  __shared__ int wt[4];
  const int b = blockIdx.x;
  if (state[4 * b + 2]) return;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int krem = state[4 * b + 1];  // read by every thread before the barrier below
  const uint32_t prefix = (uint32_t)state[4 * b];
  const int x = ghist[(size_t)b * 256 + 255 - t];  // thread t holds bin 255 - t
  ghist[(size_t)b * 256 + 255 - t] = 0;
  int v = x;  // inclusive running count from the top bin
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wt[wv] = v;
  __syncthreads();
  for (int w = 0; w < wv; ++w) v += wt[w];
  const int before = v - x;
  if (before < krem && v >= krem) {  // exactly one bin: it holds the krem-th largest key
    state[4 * b] = (int)(prefix | ((uint32_t)(255 - t) << (24 - 8 * pass)));
    state[4 * b + 1] = krem - before;
  }
}

// Per-chunk counts under the final threshold: equal keys, the weight of larger
// keys, and whether the sequence's last (clipped) block is an equal key here.
__global__ void __launch_bounds__(kSelThreads) hsi_multi_count_kernel(const uint32_t* __restrict__ keys, int nb_stride,
                                                                      const int32_t* __restrict__ seq_lens, int stride,
                                                                      int blk, const int* __restrict__ state,
                                                                      int* __restrict__ counts, int nchunks) {
  const int b = blockIdx.y;
  const int L = min(max(seq_lens[b], 0), stride);
  const int nb = (L + blk - 1) / blk;
  const int base = blockIdx.x * kChunk;
  const bool all = state[4 * b + 2] != 0;
  const uint32_t thr = all ? 0u : (uint32_t)state[4 * b];
  const uint32_t* kb = keys + (size_t)b * nb_stride;
  int c_eq = 0, c_w = 0, last_eq = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = base + j * kSelThreads + threadIdx.x;
    if (i < nb) {
      const uint32_t u = kb[i];
      if (u > thr) c_w += min(blk, L - i * blk);
      if (u == thr) {
        ++c_eq;
        if (i == nb - 1) last_eq = 1;
      }
    }
  }
  int t_eq, t_w, t_last;
  wg_exclusive_scan(c_eq, t_eq);
  wg_exclusive_scan(c_w, t_w);
  wg_exclusive_scan(last_eq, t_last);
  if (threadIdx.x == 0) {
    int* c = counts + ((size_t)b * nchunks + blockIdx.x) * 4;
    c[0] = t_eq;
    c[1] = t_w;
    c[2] = t_last;
  }
}

// Running bases of every chunk: equal keys before it, output positions before it.
__global__ void __launch_bounds__(256) hsi_multi_scan_kernel(const int32_t* __restrict__ seq_lens, int stride,
                                                             int blk, const int* __restrict__ state,
                                                             int* __restrict__ counts, int nchunks,
                                                             int32_t* __restrict__ pool_n) {
  const int b = blockIdx.x;
  if (threadIdx.x != 0) return;
  const int L = min(max(seq_lens[b], 0), stride);
  const int nb = (L + blk - 1) / blk;
  const int take = state[4 * b + 2] ? 0 : state[4 * b + 1];
  const int w_last = nb ? L - (nb - 1) * blk : 0;
  int eq_base = 0, out_base = 0;
  for (int c = 0; c < nchunks; ++c) {
    int* e = counts + ((size_t)b * nchunks + c) * 4;
    const int n_eq = e[0], w_gt = e[1], last_eq = e[2];
    const int kept = min(max(take - eq_base, 0), n_eq);
    const int w_eq = kept * blk - (last_eq && kept == n_eq && kept > 0 ? blk - w_last : 0);
    e[0] = eq_base;
    e[1] = out_base;
    eq_base += n_eq;
    out_base += w_gt + w_eq;
  }
  pool_n[b] = out_base;
}

// Ordered emit of one chunk from its bases.
__global__ void __launch_bounds__(kSelThreads) hsi_multi_emit_kernel(const uint32_t* __restrict__ keys, int nb_stride,
                                                                     const int32_t* __restrict__ seq_lens, int stride,
                                                                     int blk, const int* __restrict__ state,
                                                                     const int* __restrict__ counts, int nchunks,
                                                                     int32_t* __restrict__ pool, int pool_cap) {
  __shared__ uint32_t lk[kChunk];
  const int b = blockIdx.y;
  const int L = min(max(seq_lens[b], 0), stride);
  const int nb = (L + blk - 1) / blk;
  const int base = blockIdx.x * kChunk;
  if (base >= nb) return;
  const bool all = state[4 * b + 2] != 0;
  const uint32_t thr = all ? 0u : (uint32_t)state[4 * b];
  const int take = all ? 0 : state[4 * b + 1];
  const int* e = counts + ((size_t)b * nchunks + blockIdx.x) * 4;
  const uint32_t* kb = keys + (size_t)b * nb_stride + base;
  int32_t* out = pool + (size_t)b * pool_cap;
  const int n = min(kChunk, nb - base);
  emit_selected(
      [&](int i) { return kb[i]; }, [&](int i) { return min(blk, L - (base + i) * blk); },
      [&](int i, int off) {
        const int j = base + i, c = min(blk, L - j * blk);
        for (int r = 0; r < c; ++r) out[off + r] = j * blk + r;
      },
      n, thr, take, lk, e[0], e[1]);
}

}  // namespace

namespace {
// workspace: keys [B][nbs], then (long sequences) histograms [B][256], state
// [B][4] and chunk counts [B][nchunks][4], all 32-bit
int chunks_of(int stride, int blk) { return ((stride + blk - 1) / blk + kChunk - 1) / kChunk; }
bool multi_of(int stride, int blk) { return (stride + blk - 1) / blk > kSelLdsKeys; }
}  // namespace

size_t hsi_candidates_workspace(int batch, int stride, int blk) {
  size_t words = (size_t)batch * ((stride + blk - 1) / blk);
  if (multi_of(stride, blk)) words += (size_t)batch * (256 + 4 + 4 * (size_t)chunks_of(stride, blk));
  return words * sizeof(uint32_t);
}

int launch_hsi_candidates(const float* scores, int batch, int stride, const int32_t* seq_lens, int blk,
                          int top_blocks, int32_t* pool, int32_t* pool_n, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int nbs = (stride + blk - 1) / blk;
  uint32_t* keys = static_cast<uint32_t*>(ws);
  hsi_block_max_kernel<<<dim3((nbs + 255) / 256, batch), 256, 0, st>>>(scores, stride, seq_lens, blk, nbs, keys);
  if (!multi_of(stride, blk)) {
    hsi_pool_kernel<<<batch, kSelThreads, 0, st>>>(keys, nbs, seq_lens, stride, blk, top_blocks, pool,
                                                   top_blocks * blk, pool_n);
  } else {
    const int nch = chunks_of(stride, blk);
    int* ghist = reinterpret_cast<int*>(keys + (size_t)batch * nbs);
    int* state = ghist + (size_t)batch * 256;
    int* counts = state + (size_t)batch * 4;
    const dim3 grid(nch, batch);
    hsi_multi_init_kernel<<<batch, 256, 0, st>>>(seq_lens, stride, blk, top_blocks, ghist, state);
    for (int pass = 0; pass < 4; ++pass) {
      hsi_multi_hist_kernel<<<grid, kSelThreads, 0, st>>>(keys, nbs, seq_lens, stride, blk, pass, ghist, state);
      hsi_multi_pick_kernel<<<batch, 256, 0, st>>>(pass, ghist, state);
    }
    hsi_multi_count_kernel<<<grid, kSelThreads, 0, st>>>(keys, nbs, seq_lens, stride, blk, state, counts, nch);
    hsi_multi_scan_kernel<<<batch, 256, 0, st>>>(seq_lens, stride, blk, state, counts, nch, pool_n);
    hsi_multi_emit_kernel<<<grid, kSelThreads, 0, st>>>(keys, nbs, seq_lens, stride, blk, state, counts, nch, pool,
                                                        top_blocks * blk);
  }
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}

int launch_hsi_select(const float* pool_scores, const int32_t* pool, const int32_t* pool_n, int batch, int pool_cap,
                      int top_k, int32_t* sel, int32_t* sel_n, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hsi_select_kernel<<<batch, kSelThreads, 0, st>>>(pool_scores, pool, pool_n, pool_cap, top_k, sel, sel_n);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_EDEVICE;
}

}  // namespace kvq
