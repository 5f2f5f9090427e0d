// Internal helpers shared by the host part (tq_host.cpp) and the kernel
// launchers (tq_kernels.hip) of libtq.so. Not part of the public ABI.
#pragma once

#include <cstdint>
#include <cstdlib>
#include <cstddef>

#include "tq.h"

namespace tq {

constexpr int kMaxLevels = 16;  // 2^4
constexpr int kMaxSplitCount = 4096;  // split-K partials per query head
constexpr int kMaxDecodeRows = 65535; // decode workgroup rows (B * Hkv * head groups)

// Codebook tables in the precisions the kernels consume.
struct Codebook {
  int bits = 0;
  double c[kMaxLevels];      // ascending centroids
  double t[kMaxLevels - 1];  // thresholds
  // Scale in [1, 2) that puts every alpha * c_k as close as possible to an
  // fp16 value (decode tables hold fp16 alpha * c; 1/alpha is applied in
  // fp32 with the row norm), and the residual max relative error.
  double alpha = 1.0;
  double alpha_err = 0.0;
};

// Lloyd-Max codebook for N(0,1), cached per bit width (thread-safe).
const Codebook& codebook(int bits);
// The codebook a config selects: N(0,1) (TQ_CODEBOOK_GAUSS) or the exact
// finite-d marginal (TQ_CODEBOOK_SPHERE, d 128 or 256); cached, thread-safe.
const Codebook& codebook(int bits, int kind, int d);

// SplitMix64 output i (0-based) of the stream started at state `seed`.
inline uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline bool valid_d(int d) { return d == 128 || d == 256; }
inline bool valid_bits(int b) { return b >= 2 && b <= 4; }
inline bool valid_in_dtype(int t) { return t == TQ_F32 || t == TQ_BF16 || t == TQ_F16; }

// Validates a tq_config (shape/format fields only).
int check_config(const tq_config* cfg);
// Validates a cache against a config (pointers, alignment, shape).
int check_cache(const tq_config* cfg, const tq_cache* cache);

inline int norm_bytes(const tq_config* cfg) { return cfg->norm_dtype == TQ_F16 ? 2 : 4; }

// Decode launch geometry.
//   gk:     query heads handled by one workgroup (1, 2 or 4)
//   chunks: G / gk workgroup groups per KV head
//   tile:   tokens per tile (= threads per workgroup)
//   splits: split-K count; every split holds >= 1 token
//   tps:    tokens per split (multiple of tile)
struct DecodePlan {
  int G = 0, gk = 0, chunks = 0, tile = 0, splits = 0;
  int mx = 0;        // 1: the matrix-core kernel, 0: the workgroup-tile kernel
  int64_t tps = 0;
  // workspace section offsets (bytes); off_cnt: the matrix-core kernel's
  // arrival counters (kMaxDecodeRows words at offset 0, zero between calls)
  size_t off_qp = 0, off_qq = 0, off_ml = 0, off_acc = 0, off_cnt = 0, total = 0;
};

// Geometry of the bulk encode's code lookup for 3- and 4-bit codes: buckets
// of width 1 / kCodeLutScale in z, kCodeLutOff of them below z = 0 and as
// many above, the two end buckets open towards -inf and +inf. A codebook
// fits it when its thresholds are more than one bucket apart (at most one
// inside any bucket) and all lie inside the inner buckets.
constexpr int kCodeLutScale = 4;
constexpr int kCodeLutOff = 16;
constexpr int kCodeLutBuckets = 2 * kCodeLutOff;
bool codebook_fits_code_lookup(const tq_config* cfg, int bits);

// Waves per workgroup of the matrix-core decode kernel (one workgroup holds a
// compute unit; a workgroup round covers 64 tokens per wave), and whether a
// format runs it (d 128 or 256, 2- to 4-bit values, with or without QJL).
// Setting TQ_DECODE_VALU=1 in the environment sends every format to the
// VALU kernel instead (a diagnostic switch, read on every plan).
constexpr int mx_waves(int d) { return 8 + 0 * d; }
inline bool use_mx(int d, int bits_v, int qjl) {
  (void)qjl;
  const char* v = std::getenv("TQ_DECODE_VALU");
  if (v && v[0] == '1') return false;
  return (d == 128 || d == 256) && bits_v >= 2 && bits_v <= 4;
}

// Fills a plan; returns TQ_OK or a negative status.
int plan_decode(int d, int bits_v, int qjl, int B, int Hq, int Hkv, int64_t n_ctx,
                int splits, DecodePlan* plan);
int plan_dense(int d, int B, int Hq, int Hkv, int64_t n_ctx, int splits,
               DecodePlan* plan);

}  // namespace tq
