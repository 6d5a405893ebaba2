// Host-only parts of libkvq: layout validation, buffer sizes, bytes per token,
// split planning, workspace layout and the method's constants (Lloyd-Max
// codebook, Haar rotation, QJL matrix).  No HIP calls in this file, so every
// function here can run on a machine without a GPU.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "kvq_internal.h"

namespace kvq {

int check_layout(const kv_layout* L) {
  if (!L) return KV_EINVAL;
  if (L->batch < 1 || L->num_kv_heads < 1 || L->head_dim < 1 || L->capacity < 1 ||
      L->rope_dim < 0 || L->group < 0 || L->qjl_m < 0 || L->lm_bits < 0 || L->sink_tokens < 0 ||
      L->recent_tokens < 0 || L->sink_tokens > L->capacity || L->recent_tokens > L->capacity)
    return KV_EINVAL;
  // paged storage: whole KIVI groups and decode tiles per page
  if (L->page_tokens < 0 || L->num_pages < 0) return KV_EINVAL;
  if (L->page_tokens == 0 && L->num_pages != 0) return KV_EINVAL;
  if (L->page_tokens > 0 && (L->page_tokens < 32 || (L->page_tokens & (L->page_tokens - 1)) ||
                             L->capacity % L->page_tokens || L->num_pages < 1))
    return KV_EINVAL;
  // structured rotations: TurboQuant only
  if (L->rotation < KV_ROT_DENSE || L->rotation > KV_ROT_HADAMARD) return KV_EINVAL;
  if (L->rotation != KV_ROT_DENSE && L->format != KV_FMT_TURBO) return KV_EINVAL;
  // bf16 sink / recent windows: every per-head format (the latent cache has none)
  if ((L->sink_tokens || L->recent_tokens) && (L->format == KV_FMT_LATENT_FP4 || L->format == KV_FMT_BF16))
    return KV_EUNSUPPORTED;
  switch (L->format) {
    case KV_FMT_KIVI2:
      if (L->head_dim != 64 && L->head_dim != 128) return KV_EUNSUPPORTED;
      if (L->group != kKiviGroup || L->rope_dim || L->qjl_m || L->lm_bits) return KV_EUNSUPPORTED;
      if (L->capacity % kKiviGroup) return KV_EINVAL;
      return KV_OK;
    case KV_FMT_FP4:
      if (L->head_dim != 64 && L->head_dim != 128) return KV_EUNSUPPORTED;
      if (L->group != kFp4Group || L->rope_dim || L->qjl_m || L->lm_bits) return KV_EUNSUPPORTED;
      return KV_OK;
    case KV_FMT_TURBO:
      if (L->head_dim != 128 || L->qjl_m != kQjlM || L->lm_bits != kLmBits) return KV_EUNSUPPORTED;
      if (L->group || L->rope_dim) return KV_EUNSUPPORTED;
      return KV_OK;
    case KV_FMT_QJL1_FP4V:
      if (L->head_dim != 128 || L->qjl_m != kQjlM || L->group != kFp4Group) return KV_EUNSUPPORTED;
      if (L->rope_dim || L->lm_bits) return KV_EUNSUPPORTED;
      return KV_OK;
    case KV_FMT_LATENT_FP4:
      if (L->num_kv_heads != 1 || L->head_dim != 512 || L->rope_dim != 64) return KV_EUNSUPPORTED;
      if (L->group != kFp4Group || L->qjl_m || L->lm_bits) return KV_EUNSUPPORTED;
      return KV_OK;
    case KV_FMT_BF16:
      return KV_EUNSUPPORTED;  // sizes only; no kernels store or read it
    default:
      return KV_EINVAL;
  }
}

int check_cache(const kv_cache* c) {
  if (!c) return KV_EINVAL;
  int st = check_layout(&c->layout);
  if (st != KV_OK) return st;
  for (int b = 0; b < KV_BUF_COUNT; ++b)
    if (kv_buffer_bytes(&c->layout, b) && !c->buf[b]) return KV_EINVAL;
  int f = c->layout.format;
  if (f == KV_FMT_TURBO && ((!c->rot && c->layout.rotation == KV_ROT_DENSE) || !c->proj || !c->lm_levels ||
                            !c->lm_thresh))
    return KV_EINVAL;
  if (f == KV_FMT_QJL1_FP4V && !c->proj) return KV_EINVAL;
  if (c->layout.page_tokens > 0 && !c->block_table) return KV_EINVAL;
  // the append kernels stage R and S with 16-byte loads
  if ((reinterpret_cast<uintptr_t>(c->rot) | reinterpret_cast<uintptr_t>(c->proj)) & 15) return KV_EINVAL;
  return KV_OK;
}

int query_width(const kv_layout* L) { return L->head_dim + L->rope_dim; }

int prepared_query_width(const kv_layout* L) {
  if (L->format == KV_FMT_TURBO) return L->head_dim + L->qjl_m;
  if (L->format == KV_FMT_QJL1_FP4V) return L->qjl_m;
  return L->head_dim + L->rope_dim;
}

int value_width(const kv_layout* L) { return L->head_dim; }

bool turbo_fast_path_ok(const kv_layout& L, int num_q_heads, int nq) {
  (void)num_q_heads;  // any group: (query, head) pairs, 16 per launch
  (void)nq;
  return L.format == KV_FMT_TURBO && L.head_dim == 128 && L.qjl_m == 128 && L.lm_bits == 2 &&
         (size_t)L.capacity * 32 < (size_t(1) << 31);
}

bool latent_fast_path_ok(const kv_layout& L, int num_q_heads, int nq, int q_dtype) {
  (void)nq;  // several queries: one launch per query
  return L.format == KV_FMT_LATENT_FP4 && L.head_dim == 512 && L.rope_dim == 64 && q_dtype == KV_DT_BF16 &&
         (num_q_heads == 32 || num_q_heads == 64 || num_q_heads == 128) &&
         (size_t)L.capacity * 256 < (size_t(1) << 31);
}

bool kivi_fast_path_ok(const kv_layout& L) {
  return L.format == KV_FMT_KIVI2 && (L.head_dim == 64 || L.head_dim == 128) && L.page_tokens == 0 && L.sink_tokens == 0 &&
         L.recent_tokens == 0 && (size_t)L.capacity * 32 < (size_t(1) << 31);
}

int mfma_columns(int n) {
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : n <= 16 ? 16 : 32;
}

bool mfma_fast_path_ok(const kv_layout& L, int num_q_heads, int nq, int q_dtype) {
  const int G = num_q_heads / L.num_kv_heads;
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
  if (L.head_dim != 128) return false;
  // several queries: every (query, head) pair a column of its own, 16 columns per
  // launch (FP4 keys: 32 in two blocks)
  if (nq > 1)
    return (L.format == KV_FMT_FP4 && q_dtype == KV_DT_BF16) || (L.format == KV_FMT_QJL1_FP4V && L.qjl_m == 128);
  if (!g_ok) return false;
  if (L.format == KV_FMT_FP4) return q_dtype == KV_DT_BF16;
  if (L.format == KV_FMT_QJL1_FP4V) return L.qjl_m == 128;
  return false;
}

SplitPlan plan_splits(const kv_layout* L, int num_q_heads, int nq, int q_dtype, int max_seq_len, int requested,
                      bool general, int max_splits) {
  // Workgroups cover their split in steps of `tile` tokens; aim for enough
  // workgroups to keep a 256-CU part busy several times over, but no split
  // shorter than a few steps.
  const int G = num_q_heads / L->num_kv_heads;
  const bool fast = !general && (mfma_fast_path_ok(*L, num_q_heads, nq, q_dtype) ||
                                 turbo_fast_path_ok(*L, num_q_heads, nq) || kivi_fast_path_ok(*L));
  const bool latent = !general && latent_fast_path_ok(*L, num_q_heads, nq, q_dtype);
  const int tile = fast ? 128 : 64;
  // the latent kernel keeps one workgroup per compute unit resident and every
  // split writes Hq x 514 partial floats: one round of workgroups, a few long
  // splits per sequence (4 at batch 64; 8 measured no faster in the kernel and
  // doubles the partials the merge reads).  The streaming matrix-core kernels
  // keep three workgroups per compute unit resident; FP4 and TurboQuant
  // measured fastest at about 1,024 workgroups (each one's start and finish
  // leave its compute unit's share of the stream idle), QJL keys at 2,048.
  const long target = latent ? 256 : fast && L->format != KV_FMT_QJL1_FP4V ? 1024 : 2048;
  long units = (long)L->batch * L->num_kv_heads;
  if (!fast && !latent && nq * G > 16) units *= (nq * G + 15) / 16;  // the generic kernel's head blocks
  int splits = requested;
  if (splits <= 0) {
    long want = (target + units - 1) / units;
    long maxs = (max_seq_len + tile - 1) / tile;  // at least one tile per split
    splits = (int)std::max(1L, std::min(want, maxs));
  }
  if (splits > max_splits) splits = max_splits;
  if (splits > max_seq_len) splits = max_seq_len;
  if (splits < 1) splits = 1;
  int per = (max_seq_len + splits - 1) / splits;
  per = (per + tile - 1) / tile * tile;
  splits = (max_seq_len + per - 1) / per;
  return SplitPlan{splits, per};
}

DecodeWorkspace decode_workspace(const kv_layout* L, int num_q_heads, int splits) {
  // Counters first, at a fixed offset: they must stay zero between calls, and a
  // later call with another split count must find them where it left them.
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  DecodeWorkspace w;
  size_t rows = (size_t)L->batch * num_q_heads;
  w.cnt_off = 0;
  w.qprep_off = align((size_t)L->batch * L->num_kv_heads * sizeof(unsigned));
  w.qpiece_off = w.qprep_off + align(rows * prepared_query_width(L) * sizeof(float));
  const size_t piece_bytes = L->format == KV_FMT_TURBO ? kTurboPieceBytes
                            : L->format == KV_FMT_QJL1_FP4V ? kQjlPieceBytes : 0;
  w.part_off = w.qpiece_off + align(rows * piece_bytes);
  w.total = w.part_off + align(rows * (size_t)splits * (value_width(L) + 2) * sizeof(float));
  return w;
}

}  // namespace kvq

using namespace kvq;

extern "C" size_t kv_buffer_bytes(const kv_layout* L, int32_t which) {
  if (check_layout(L) != KV_OK || which < 0 || which >= KV_BUF_COUNT) return 0;
  const size_t B = L->batch, H = L->num_kv_heads, T = L->capacity, d = L->head_dim;
  // per-token buffers: B x H x capacity rows, or the pool's pages x H x page_tokens
  const size_t bht = L->page_tokens > 0 ? (size_t)L->num_pages * H * L->page_tokens : B * H * T;
  if (which == KV_BUF_SINK_K || which == KV_BUF_SINK_V) return B * H * (size_t)L->sink_tokens * d * 2;
  if (which == KV_BUF_RECENT_K || which == KV_BUF_RECENT_V) return B * H * (size_t)L->recent_tokens * d * 2;
  if (which == KV_BUF_K_STAGE) return L->format == KV_FMT_KIVI2 ? B * H * (4 + (size_t)kKiviGroup * d) * 4 : 0;
  switch (L->format) {
    case KV_FMT_KIVI2:
      switch (which) {
        case KV_BUF_K_CODES: case KV_BUF_V_CODES: return bht * d / 4;
        case KV_BUF_K_SCALE: case KV_BUF_K_ZERO: return bht / kKiviGroup * d * 4;
        case KV_BUF_V_SCALE: case KV_BUF_V_ZERO: return bht * (d / kKiviGroup) * 4;
        default: return 0;
      }
    case KV_FMT_FP4:
      switch (which) {
        case KV_BUF_K_CODES: case KV_BUF_V_CODES: return bht * d / 2;
        case KV_BUF_K_SCALE: case KV_BUF_V_SCALE: return bht * (d / kFp4Group) * 2;
        default: return 0;
      }
    case KV_FMT_TURBO:
      switch (which) {
        case KV_BUF_K_CODES: case KV_BUF_V_CODES: return bht * d / 4;
        case KV_BUF_K_SKETCH: return bht * L->qjl_m / 8;
        case KV_BUF_K_NORM: case KV_BUF_K_RNORM: case KV_BUF_V_NORM: return bht * 2;
        default: return 0;
      }
    case KV_FMT_QJL1_FP4V:
      switch (which) {
        case KV_BUF_K_SKETCH: return bht * L->qjl_m / 8;
        case KV_BUF_K_NORM: return bht * 2;
        case KV_BUF_V_CODES: return bht * d / 2;
        case KV_BUF_V_SCALE: return bht * (d / kFp4Group) * 2;
        default: return 0;
      }
    case KV_FMT_LATENT_FP4:
      switch (which) {
        case KV_BUF_K_CODES: return bht * d / 2;
        case KV_BUF_K_SCALE: return bht * (d / kFp4Group) * 2;
        case KV_BUF_ROPE: return bht * L->rope_dim * 2;
        default: return 0;
      }
    default:
      return 0;
  }
}

extern "C" size_t kv_bytes_per_token(const kv_layout* L, int32_t num_layers) {
  if (!L || num_layers < 1) return 0;
  if (L->format == KV_FMT_BF16) {
    if (L->num_kv_heads < 1 || L->head_dim < 1) return 0;
    return (size_t)num_layers * L->num_kv_heads * L->head_dim * 2 /*K,V*/ * 2 /*bytes*/;
  }
  if (check_layout(L) != KV_OK) return 0;
  // Sum the per-token share of every buffer: each buffer holds B*H*capacity
  // token slots (B*capacity for the latent; a paged pool num_pages*H*page_tokens),
  // so divide by that.
  size_t slots = L->page_tokens > 0 ? (size_t)L->num_pages * L->num_kv_heads * L->page_tokens
                                    : (size_t)L->batch * L->num_kv_heads * L->capacity;
  size_t total = 0;
  for (int b = 0; b < KV_BUF_COUNT; ++b)
    if (b < KV_BUF_SINK_K) total += kv_buffer_bytes(L, b);  // not the per-sequence windows and staging
  return (size_t)num_layers * L->num_kv_heads * (total / slots);
}

extern "C" const char* kv_status_string(int status) {
  switch (status) {
    case KV_OK: return "ok";
    case KV_EINVAL: return "invalid argument";
    case KV_ECAPACITY: return "tokens beyond cache capacity";
    case KV_EUNSUPPORTED: return "unsupported layout or dtype";
    case KV_EWORKSPACE: return "workspace missing or too small";
    case KV_EDEVICE: return "kernel launch failed";
    default: return "unknown status";
  }
}

// ---------------------------------------------------------------- constants

namespace {

// Round a finite double to the nearest bf16 value (ties to even), as a float.
float bf16_round(double x) {
  if (x == 0.0 || !std::isfinite(x)) return (float)x;
  double a = std::fabs(x);
  double r;
  if (a < 0x1p-126) {
    r = std::nearbyint(a * 0x1p133) * 0x1p-133;  // bf16 subnormal spacing 2^-133
  } else {
    uint64_t u;
    std::memcpy(&u, &a, 8);
    const int drop = 52 - 7;  // keep 7 fraction bits
    uint64_t lsb = (u >> drop) & 1;
    u += ((uint64_t)1 << (drop - 1)) - 1 + lsb;
    u &= ~(((uint64_t)1 << drop) - 1);
    std::memcpy(&r, &u, 8);
  }
  float f = (float)r;  // exact: at most 8 significant bits (or inf past the range)
  return x < 0 ? -f : f;
}

double std_normal_pdf(double z) { return std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI); }
double std_normal_cdf(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }

}  // namespace

namespace kvq {
float hadamard_magnitude(int d) { return bf16_round(1.0 / std::sqrt((double)d)); }
}  // namespace kvq

extern "C" int kv_lloyd_max_gaussian(int32_t bits, int32_t dim, float* levels, float* thresholds) {
  if (bits < 1 || bits > 4 || dim < 1 || !levels || !thresholds) return KV_EINVAL;
  const int n = 1 << bits;
  std::vector<double> c(n), t(n - 1), nc(n);
  for (int i = 0; i < n; ++i) c[i] = -2.0 + 4.0 * i / (n - 1);
  for (int it = 0; it < 100000; ++it) {
    for (int i = 0; i + 1 < n; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
    double delta = 0.0;
    for (int i = 0; i < n; ++i) {
      // mean of N(0,1) over (lo, hi): (pdf(lo) - pdf(hi)) / (cdf(hi) - cdf(lo))
      double plo = i == 0 ? 0.0 : std_normal_pdf(t[i - 1]);
      double phi = i == n - 1 ? 0.0 : std_normal_pdf(t[i]);
      double clo = i == 0 ? 0.0 : std_normal_cdf(t[i - 1]);
      double chi = i == n - 1 ? 1.0 : std_normal_cdf(t[i]);
      nc[i] = (plo - phi) / (chi - clo);
      delta = std::max(delta, std::fabs(nc[i] - c[i]));
    }
    // the source is symmetric, so is the fixed point: keep the iterate exactly
    // antisymmetric (c[n-1-i] = -c[i]) so that the middle threshold is exactly 0
    for (int i = 0; i < n / 2; ++i) {
      const double m = 0.5 * (nc[n - 1 - i] - nc[i]);
      nc[i] = -m;
      nc[n - 1 - i] = m;
    }
    c.swap(nc);
    if (delta <= 1e-15) break;
  }
  const double sigma = 1.0 / std::sqrt((double)dim);
  for (int i = 0; i < n; ++i) levels[i] = (float)(c[i] * sigma);
  for (int i = 0; i + 1 < n; ++i) thresholds[i] = (float)(0.5 * (c[i] + c[i + 1]) * sigma);
  return KV_OK;
}

extern "C" int kv_make_rotation(const double* gauss, int32_t d, float* rot) {
  if (!gauss || !rot || d < 1 || d > 1024) return KV_EINVAL;
  // Householder QR of A = gauss: A = Q R.  W holds A column-major while reflectors
  // are applied; reflector k is stored in V[k][k..d).
  std::vector<double> W((size_t)d * d), V((size_t)d * d, 0.0), Q((size_t)d * d, 0.0);
  auto w = [&](int i, int j) -> double& { return W[(size_t)j * d + i]; };
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) w(i, j) = gauss[(size_t)i * d + j];
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += w(i, k) * w(i, k);
    nrm = std::sqrt(nrm);
    if (!(nrm > 0.0)) return KV_EINVAL;
    double alpha = w(k, k) > 0 ? -nrm : nrm;
    double* v = &V[(size_t)k * d];
    double vn = 0.0;
    for (int i = k; i < d; ++i) {
      v[i] = w(i, k) - (i == k ? alpha : 0.0);
      vn += v[i] * v[i];
    }
    vn = std::sqrt(vn);
    if (vn > 0.0)
      for (int i = k; i < d; ++i) v[i] /= vn;
    for (int j = k; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * w(i, j);
      for (int i = k; i < d; ++i) w(i, j) -= 2.0 * v[i] * s;
    }
    rdiag[k] = w(k, k);
  }
  // Q = H_0 H_1 ... H_{d-1}: apply the reflectors to the identity, last first.
  for (int i = 0; i < d; ++i) Q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &V[(size_t)k * d];
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * Q[(size_t)i * d + j];
      for (int i = k; i < d; ++i) Q[(size_t)i * d + j] -= 2.0 * v[i] * s;
    }
  }
  // Unique factorisation with diag(R) > 0: flip column j of Q where R_jj < 0.
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      double q = Q[(size_t)i * d + j] * (rdiag[j] < 0 ? -1.0 : 1.0);
      rot[(size_t)i * d + j] = bf16_round(q);
    }
  return KV_OK;
}

extern "C" int kv_make_hadamard_rotation(int32_t d, int32_t bit_reverse, float* rot) {
  if (!rot || d < 1 || d > 1024 || (d & (d - 1))) return KV_EINVAL;
  int nbits = 0;
  while ((1 << nbits) < d) ++nbits;
  // Entry (i, j) multiplies x[j]; with the permutation first, x[j] meets Walsh
  // column rev(j), and H[i][k] = (-1)^popcount(i & k).  Every entry is +-1/sqrt(d),
  // one bf16 value up to sign.
  const float mag = bf16_round(1.0 / std::sqrt((double)d));
  for (int j = 0; j < d; ++j) {
    int col = j;
    if (bit_reverse) {
      col = 0;
      for (int b = 0; b < nbits; ++b) col |= ((j >> b) & 1) << (nbits - 1 - b);
    }
    for (int i = 0; i < d; ++i)
      rot[(size_t)i * d + j] = (__builtin_popcount((unsigned)(i & col)) & 1) ? -mag : mag;
  }
  return KV_OK;
}

extern "C" int kv_make_projection(const double* gauss, int32_t m, int32_t d, float* proj) {
  if (!gauss || !proj || m < 1 || d < 1) return KV_EINVAL;
  for (size_t i = 0; i < (size_t)m * d; ++i) proj[i] = bf16_round(gauss[i]);
  return KV_OK;
}
