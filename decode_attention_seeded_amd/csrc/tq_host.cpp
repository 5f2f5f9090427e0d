// Host-only part of libtq.so: argument validation, the Lloyd-Max codebook,
// the rotation signs, fractional-bit rule, cache sizes and launch plans.
// Nothing here touches the GPU.

#include <cmath>
#include <cstring>
#include <mutex>

#include "tq_internal.h"

namespace tq {

namespace {

// P(Z >= x) and the standard normal density.
double upper_tail(double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x / std::sqrt(2.0)); }
double density(double x) {
  return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

// Lloyd iteration for the N(0,1) quantizer with 2^bits levels. The
// positive half is iterated (cells [a_k, a_{k+1}) with a_0 = 0, a_m = inf,
// centroid = E[Z | cell]) and mirrored, which keeps the codebook exactly
// antisymmetric with a zero middle threshold.
Codebook build_codebook(int bits) {
  Codebook cb;
  cb.bits = bits;
  const int m = 1 << (bits - 1);
  double pos[kMaxLevels / 2];
  // start: evenly spaced on (0, 3]
  for (int k = 0; k < m; ++k) pos[k] = 3.0 * (k + 0.5) / m;
  for (int it = 0; it < 1000000; ++it) {
    double edge[kMaxLevels / 2 + 1];
    edge[0] = 0.0;
    for (int k = 1; k < m; ++k) edge[k] = 0.5 * (pos[k - 1] + pos[k]);
    edge[m] = INFINITY;
    double change = 0.0;
    for (int k = 0; k < m; ++k) {
      const double mass = upper_tail(edge[k]) - upper_tail(edge[k + 1]);
      const double mean = (density(edge[k]) - density(edge[k + 1])) / mass;
      change = std::fmax(change, std::fabs(mean - pos[k]));
      pos[k] = mean;
    }
    if (change < 1e-16) break;
  }
  const int L = 2 * m;
  for (int k = 0; k < m; ++k) {
    cb.c[m + k] = pos[k];
    cb.c[m - 1 - k] = -pos[k];
  }
  for (int k = 1; k < L; ++k) cb.t[k - 1] = 0.5 * (cb.c[k - 1] + cb.c[k]);
  cb.t[m - 1] = 0.0;
  return cb;
}

// Lloyd iteration for the exact marginal of z = sqrt(d) u, u one coordinate
// of a uniformly random unit vector in R^d: density proportional to
// (1 - z^2/d)^((d-3)/2) on |z| < sqrt(d). Cell mass by Simpson's rule in
// theta (z = sqrt(d) sin(theta), integrand sqrt(d) cos^(d-2)(theta)); the
// first moment in closed form, d/(d-1) [(1 - a^2/d)^((d-1)/2) - (1 -
// b^2/d)^((d-1)/2)]. Positive half iterated, then mirrored, as above.
Codebook build_sphere_codebook(int bits, int d) {
  const Codebook g = build_codebook(bits);
  Codebook cb;
  cb.bits = bits;
  const int m = 1 << (bits - 1);
  const double rd = std::sqrt(double(d));
  auto base = [&](double z) { return std::fmax(0.0, 1.0 - z * z / d); };
  auto mass = [&](double a, double b) {
    const double ta = std::asin(std::fmin(1.0, a / rd)), tb = std::asin(std::fmin(1.0, b / rd));
    const int n = 4096;                       // even
    const double h = (tb - ta) / n;
    double acc = 0.0;
    for (int i = 0; i <= n; ++i) {
      const double w = (i == 0 || i == n) ? 1.0 : (i & 1) ? 4.0 : 2.0;
      acc += w * std::pow(std::cos(ta + i * h), d - 2);
    }
    return rd * acc * h / 3.0;
  };
  auto first = [&](double a, double b) {
    const double e = 0.5 * (d - 1);
    return d / double(d - 1) * (std::pow(base(a), e) - std::pow(base(b), e));
  };
  double pos[kMaxLevels / 2];
  for (int k = 0; k < m; ++k) pos[k] = std::fmin(g.c[m + k], 0.9 * rd);
  for (int it = 0; it < 100000; ++it) {
    double edge[kMaxLevels / 2 + 1];
    edge[0] = 0.0;
    for (int k = 1; k < m; ++k) edge[k] = 0.5 * (pos[k - 1] + pos[k]);
    edge[m] = rd;
    double change = 0.0;
    for (int k = 0; k < m; ++k) {
      const double mean = first(edge[k], edge[k + 1]) / mass(edge[k], edge[k + 1]);
      change = std::fmax(change, std::fabs(mean - pos[k]));
      pos[k] = mean;
    }
    if (change < 1e-14) break;
  }
  const int L = 2 * m;
  for (int k = 0; k < m; ++k) {
    cb.c[m + k] = pos[k];
    cb.c[m - 1 - k] = -pos[k];
  }
  for (int k = 1; k < L; ++k) cb.t[k - 1] = 0.5 * (cb.c[k - 1] + cb.c[k]);
  cb.t[m - 1] = 0.0;
  return cb;
}

// Nearest-even rounding of a positive double to binary16, returned as a
// double (normal range only; the centroids here are in [0.1, 3]).
double round_f16(double x) {
  int e;
  const double m = std::frexp(x, &e);          // x = m * 2^e, m in [0.5, 1)
  const double scaled = std::ldexp(m, 11);     // 11 significant bits
  return std::ldexp(std::nearbyint(scaled), e - 11);
}

// Scale alpha in [1, 2) (steps of 2^-20) minimizing the largest relative
// fp16 rounding error of alpha * c over the positive centroids.
void fit_alpha(Codebook& cb) {
  const int m = 1 << (cb.bits - 1);
  double best = 1e9, best_a = 1.0;
  for (int i = 0; i < (1 << 20); ++i) {
    const double a = 1.0 + std::ldexp(double(i), -20);
    double worst = 0.0;
    for (int k = 0; k < m && worst < best; ++k) {
      const double v = a * cb.c[m + k];
      worst = std::fmax(worst, std::fabs(round_f16(v) - v) / v);
    }
    if (worst < best) {
      best = worst;
      best_a = a;
    }
  }
  cb.alpha = best_a;
  cb.alpha_err = best;
}

std::once_flag g_once[5];
Codebook g_cb[5];
std::mutex g_sphere_mu;
Codebook g_sphere[5][2];                 // [bits][d == 256]
bool g_sphere_ok[5][2];

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

const Codebook& codebook(int bits) {
  std::call_once(g_once[bits], [bits] {
    g_cb[bits] = build_codebook(bits);
    fit_alpha(g_cb[bits]);
  });
  return g_cb[bits];
}

const Codebook& codebook(int bits, int kind, int d) {
  if (kind != TQ_CODEBOOK_SPHERE) return codebook(bits);
  const int j = d == 256 ? 1 : 0;
  std::lock_guard<std::mutex> lock(g_sphere_mu);
  if (!g_sphere_ok[bits][j]) {
    g_sphere[bits][j] = build_sphere_codebook(bits, d);
    fit_alpha(g_sphere[bits][j]);
    g_sphere_ok[bits][j] = true;
  }
  return g_sphere[bits][j];
}

bool codebook_fits_code_lookup(const tq_config* cfg, int bits) {
  if (bits != 3 && bits != 4) return true;
  const Codebook& cb = codebook(bits, cfg->codebook, cfg->d);
  const int L = 1 << bits;
  const double w = 1.0 / kCodeLutScale, lim = (kCodeLutOff - 1) * w;
  for (int k = 0; k < L - 1; ++k) {
    if (!(std::fabs(cb.t[k]) < lim)) return false;
    if (k > 0 && !(cb.t[k] - cb.t[k - 1] > w)) return false;
  }
  return true;
}

int check_config(const tq_config* cfg) {
  if (!cfg) return TQ_ERR_ARG;
  if (!valid_d(cfg->d) || !valid_bits(cfg->bits_k) || !valid_bits(cfg->bits_v))
    return TQ_ERR_UNSUPPORTED;
  if (cfg->norm_dtype != TQ_F16 && cfg->norm_dtype != TQ_F32) return TQ_ERR_UNSUPPORTED;
  if (cfg->qjl != 0 && cfg->qjl != 1) return TQ_ERR_ARG;
  if (cfg->codebook != TQ_CODEBOOK_GAUSS && cfg->codebook != TQ_CODEBOOK_SPHERE)
    return TQ_ERR_UNSUPPORTED;
  // every supported codebook fits; a codebook that did not would get wrong codes
  if (!codebook_fits_code_lookup(cfg, cfg->bits_k) || !codebook_fits_code_lookup(cfg, cfg->bits_v))
    return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

int check_cache(const tq_config* cfg, const tq_cache* c) {
  if (!c) return TQ_ERR_ARG;
  if (c->B < 0 || c->Hkv < 1 || c->capacity < 0) return TQ_ERR_ARG;
  if (!c->kc || !c->vc || !c->kn || !c->vn) return TQ_ERR_ARG;
  if (cfg->qjl && (!c->kq || !c->kr)) return TQ_ERR_ARG;
  if (!aligned16(c->kc) || !aligned16(c->vc) || !aligned16(c->kn) || !aligned16(c->vn))
    return TQ_ERR_ALIGN;
  if (cfg->qjl && (!aligned16(c->kq) || !aligned16(c->kr))) return TQ_ERR_ALIGN;
  return TQ_OK;
}

static int decode_tile(int d) { return d == 128 ? 256 : 512; }

// Default split count: about `target` workgroups over the chip (256 CUs).
// The matrix-core kernel holds a whole compute unit per workgroup, so it aims at one
// round of 256 workgroups; the narrow kernels at ~8 workgroups per CU.
static int finish_plan(int64_t n_ctx, int splits, int64_t units, int tile, int64_t target,
                       DecodePlan* p) {
  const int64_t tiles = (n_ctx + tile - 1) / tile;
  int64_t s;
  if (splits > 0) {
    s = splits;
  } else {
    if (units < 1) units = 1;
    s = (target + units - 1) / units;
  }
  if (s > tiles) s = tiles;
  if (s > kMaxSplitCount) s = kMaxSplitCount;
  if (s < 1) s = 1;
  const int64_t tiles_per_split = (tiles + s - 1) / s;
  p->tps = tiles_per_split * tile;
  p->splits = int((n_ctx + p->tps - 1) / p->tps);
  p->tile = tile;
  return TQ_OK;
}

int plan_decode(int d, int bits_v, int qjl, int B, int Hq, int Hkv, int64_t n_ctx, int splits,
                DecodePlan* p) {
  if (!valid_d(d)) return TQ_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || splits < 0) return TQ_ERR_ARG;
  if (n_ctx < 1) return TQ_ERR_ARG;
  *p = DecodePlan();
  p->G = Hq / Hkv;
  p->gk = (p->G % 4 == 0) ? 4 : (p->G % 2 == 0) ? 2 : 1;
  p->chunks = p->G / p->gk;
  p->mx = use_mx(d, bits_v, qjl) ? 1 : 0;
  const int64_t units = int64_t(B) * Hkv * p->chunks;
  if (p->mx)
    finish_plan(n_ctx, splits, units, 64 * mx_waves(d), 256, p);
  else
    finish_plan(n_ctx, splits, units, decode_tile(d), 2048, p);
  const size_t heads = size_t(B) * Hq;
  if (units > kMaxDecodeRows) return TQ_ERR_ARG;
  // arrival counters first, at a fixed offset and size, so that they never
  // move or overlap another section when one workspace serves calls of
  // different shapes
  size_t off = 0;
  p->off_cnt = off; off = align256(off + size_t(kMaxDecodeRows) * sizeof(uint32_t));
  p->off_qp = off;  off = align256(off + heads * d * sizeof(float));
  p->off_qq = off;  if (qjl) off = align256(off + heads * d * sizeof(float));
  p->off_ml = off;  off = align256(off + heads * p->splits * 2 * sizeof(float));
  p->off_acc = off; off = align256(off + heads * p->splits * size_t(d) * sizeof(float));
  p->total = off;
  return TQ_OK;
}

int plan_dense(int d, int B, int Hq, int Hkv, int64_t n_ctx, int splits, DecodePlan* p) {
  // the dense baseline runs the same split-K skeleton with bf16 rows
  return plan_decode(d, 16, 0, B, Hq, Hkv, n_ctx, splits, p);
}

}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_strerror(int s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_ARG: return "TQ_ERR_ARG: invalid argument";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED: unsupported d, bit width or dtype";
    case TQ_ERR_ALIGN: return "TQ_ERR_ALIGN: device pointer not 16-byte aligned";
    case TQ_ERR_CAPACITY: return "TQ_ERR_CAPACITY: token range exceeds cache capacity";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE: workspace too small";
    case TQ_ERR_NO_DEVICE: return "TQ_ERR_NO_DEVICE: no HIP device";
    case TQ_ERR_HIP: return "TQ_ERR_HIP: HIP runtime error";
    default: return "unknown tq_status";
  }
}

int tq_bits_split(double kv_bits, int force_turboquant, int* enabled, int* bits_k,
                  int* bits_v) {
  if (!enabled || !bits_k || !bits_v || !std::isfinite(kv_bits)) return TQ_ERR_ARG;
  const double nearest = std::nearbyint(kv_bits);
  const bool integral = std::fabs(kv_bits - nearest) <= 1e-6;
  if (integral && !force_turboquant) {
    *enabled = 0;
    return TQ_OK;
  }
  int bk, bv;
  if (integral) {
    bk = bv = int(nearest);
  } else {
    bk = int(std::floor(kv_bits));
    bv = int(std::ceil(kv_bits));
  }
  *enabled = 1;
  if (!valid_bits(bk) || !valid_bits(bv)) return TQ_ERR_UNSUPPORTED;
  *bits_k = bk;
  *bits_v = bv;
  return TQ_OK;
}

int tq_codebook(int bits, double* centroids, double* thresholds) {
  if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
  const Codebook& cb = codebook(bits);
  const int L = 1 << bits;
  if (centroids) std::memcpy(centroids, cb.c, sizeof(double) * L);
  if (thresholds) std::memcpy(thresholds, cb.t, sizeof(double) * (L - 1));
  return TQ_OK;
}

int tq_codebook_ex(int bits, int kind, int d, double* centroids, double* thresholds) {
  if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
  if (kind != TQ_CODEBOOK_GAUSS && kind != TQ_CODEBOOK_SPHERE) return TQ_ERR_UNSUPPORTED;
  if (kind == TQ_CODEBOOK_SPHERE && !valid_d(d)) return TQ_ERR_UNSUPPORTED;
  const Codebook& cb = codebook(bits, kind, d);
  const int L = 1 << bits;
  if (centroids) std::memcpy(centroids, cb.c, sizeof(double) * L);
  if (thresholds) std::memcpy(thresholds, cb.t, sizeof(double) * (L - 1));
  return TQ_OK;
}

int tq_signs(uint64_t seed, int d, int8_t* out) {
  if (!out || d < 1) return TQ_ERR_ARG;
  for (int i = 0; i < d; ++i) out[i] = (splitmix64_at(seed, uint64_t(i)) >> 63) ? -1 : 1;
  return TQ_OK;
}

int64_t tq_cache_bytes(const tq_config* cfg, int B, int Hkv, int64_t capacity,
                       int64_t* plane_bytes) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (B < 0 || Hkv < 1 || capacity < 0) return TQ_ERR_ARG;
  const int64_t rows = int64_t(B) * Hkv * capacity;
  int64_t p[6] = {
      rows * cfg->d * cfg->bits_k / 8, rows * cfg->d * cfg->bits_v / 8,
      rows * norm_bytes(cfg),          rows * norm_bytes(cfg),
      cfg->qjl ? rows * cfg->d / 8 : 0, cfg->qjl ? rows * 2 : 0};
  int64_t total = 0;
  for (int i = 0; i < 6; ++i) {
    if (plane_bytes) plane_bytes[i] = p[i];
    total += p[i];
  }
  return total;
}

int tq_num_splits(const tq_config* cfg, int B, int Hq, int Hkv, int64_t n_ctx, int splits) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  DecodePlan p;
  st = plan_decode(cfg->d, cfg->bits_v, cfg->qjl, B, Hq, Hkv, n_ctx, splits, &p);
  return st != TQ_OK ? st : p.splits;
}

int64_t tq_workspace_bytes(const tq_config* cfg, int B, int Hq, int Hkv, int64_t n_ctx,
                           int splits) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  DecodePlan p;
  st = plan_decode(cfg->d, cfg->bits_v, cfg->qjl, B, Hq, Hkv, n_ctx, splits, &p);
  return st != TQ_OK ? st : int64_t(p.total);
}

int64_t tq_dense_workspace_bytes(int B, int Hq, int Hkv, int d, int64_t n_ctx, int splits) {
  DecodePlan p;
  int st = plan_dense(d, B, Hq, Hkv, n_ctx, splits, &p);
  return st != TQ_OK ? st : int64_t(p.total);
}

}  // extern "C"
