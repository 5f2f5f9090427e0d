// Public entry points of libtq.so: host-side validation, launch planning and
// kernel launches. Every argument is checked before the first HIP call.

#include <cmath>
#include <mutex>

#include "tq_internal.h"
#include "tq_kernels.h"
#include "tq_prefill.h"

namespace tq {

using DecodeLauncher = int (*)(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d128_k2(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d128_k3(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d128_k4(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d128_k16(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d256_k2(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d256_k3(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d256_k4(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);
int launch_decode_d256_k16(int, int, int, int, const DecodeArgs&, dim3, hipStream_t);

int launch_prefill_d128(int, int, int, const PrefillArgs&, dim3, hipStream_t);
int launch_prefill_d256(int, int, int, const PrefillArgs&, dim3, hipStream_t);

using EncodeLauncher = int (*)(int, bool, const EncodeArgs&, hipStream_t);
int launch_encode_d128_k2(int, bool, const EncodeArgs&, hipStream_t);
int launch_encode_d128_k3(int, bool, const EncodeArgs&, hipStream_t);
int launch_encode_d128_k4(int, bool, const EncodeArgs&, hipStream_t);
int launch_encode_d256_k2(int, bool, const EncodeArgs&, hipStream_t);
int launch_encode_d256_k3(int, bool, const EncodeArgs&, hipStream_t);
int launch_encode_d256_k4(int, bool, const EncodeArgs&, hipStream_t);

namespace {

DecodeLauncher decode_launcher(int d, int bk) {
  if (d == 128) {
    switch (bk) {
      case 2: return launch_decode_d128_k2;
      case 3: return launch_decode_d128_k3;
      case 4: return launch_decode_d128_k4;
      case 16: return launch_decode_d128_k16;
    }
  } else if (d == 256) {
    switch (bk) {
      case 2: return launch_decode_d256_k2;
      case 3: return launch_decode_d256_k3;
      case 4: return launch_decode_d256_k4;
      case 16: return launch_decode_d256_k16;
    }
  }
  return nullptr;
}

EncodeLauncher encode_launcher(int d, int bk) {
  switch (bk) {
    case 2: return d == 128 ? launch_encode_d128_k2 : launch_encode_d256_k2;
    case 3: return d == 128 ? launch_encode_d128_k3 : launch_encode_d256_k3;
    case 4: return d == 128 ? launch_encode_d128_k4 : launch_encode_d256_k4;
  }
  return nullptr;
}

int device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return TQ_ERR_NO_DEVICE;
  return TQ_OK;
}

int last_launch() { return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

unsigned row_grid(int64_t rows) {
  const int64_t g = (rows + 15) / 16;
  return unsigned(g < 16384 ? g : 16384);
}

// Bit i set when rotation sign i (SplitMix64 stream `seed`) is negative.
void sign_bitmap(uint64_t seed, int d, uint32_t (&w)[8]) {
  for (int k = 0; k < 8; ++k) w[k] = 0;
  for (int i = 0; i < d; ++i)
    if (splitmix64_at(seed, uint64_t(i)) >> 63) w[i >> 5] |= 1u << (i & 31);
}

// t_{L/2} .. t_{L-2}: the positive thresholds of the antisymmetric codebook.
void fill_positive_thresholds(const tq_config* cfg, int bits, double* tpos) {
  const Codebook& cb = codebook(bits, cfg->codebook, cfg->d);
  const int H = 1 << (bits - 1);
  for (int j = 0; j < 7; ++j) tpos[j] = j < H - 1 ? cb.t[H + j] : INFINITY;
}

void fill_codebook_f64(const tq_config* cfg, int bits, double* thr, double* cen) {
  const Codebook& cb = codebook(bits, cfg->codebook, cfg->d);
  const int L = 1 << bits;
  for (int k = 0; k < 15; ++k) thr[k] = k < L - 1 ? cb.t[k] : INFINITY;
  for (int k = 0; k < 16; ++k) cen[k] = k < L ? cb.c[k] : 0.0;
}

// alpha * centroids for the fp16 decode tables; returns alpha.
double fill_codebook_f32(const tq_config* cfg, int bits, float* cen) {
  const Codebook& cb = codebook(bits, cfg->codebook, cfg->d);
  const int L = 1 << bits;
  for (int k = 0; k < 16; ++k) cen[k] = k < L ? float(cb.alpha * cb.c[k]) : 0.f;
  return cb.alpha;
}

int launch_qprep(int d, const QPrepArgs& a, hipStream_t st) {
  const unsigned grid = unsigned((a.heads + 15) / 16);
  if (d == 128)
    hipLaunchKernelGGL(k_qprep<128>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_qprep<256>, dim3(grid), dim3(256), 0, st, a);
  return last_launch();
}

int launch_merge(int d, const MergeArgs& a, hipStream_t st) {
  const dim3 grid(unsigned(a.heads), unsigned(d / 32));
  if (d == 128)
    hipLaunchKernelGGL(k_merge<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_merge<256>, grid, dim3(256), 0, st, a);
  return last_launch();
}

// Kernel arguments of the encode of rows [offset, offset + n_new) of every
// (batch, KV head) from k, v: [B*Hkv][n_new][d] of in_dtype.
void fill_encode_args(const tq_config* cfg, const void* k, const void* v, int in_dtype,
                      int64_t offset, int64_t n_new, const tq_cache* cache, EncodeArgs* a) {
  a->x[0] = k;
  a->x[1] = v;
  a->codes[0] = static_cast<uint8_t*>(cache->kc);
  a->codes[1] = static_cast<uint8_t*>(cache->vc);
  a->norms[0] = cache->kn;
  a->norms[1] = cache->vn;
  a->qbits = static_cast<uint8_t*>(cache->kq);
  a->rnorm = static_cast<uint16_t*>(cache->kr);
  a->n_new = n_new;
  a->offset = offset;
  a->capacity = cache->capacity;
  a->BH = cache->B * cache->Hkv;
  a->in_dtype = in_dtype;
  a->norm_f16 = cfg->norm_dtype == TQ_F16;
  sign_bitmap(cfg->seed, cfg->d, a->sbits);
  sign_bitmap(cfg->qjl_seed, cfg->d, a->qsbits);
  fill_positive_thresholds(cfg, cfg->bits_k, a->tpos[0]);
  fill_positive_thresholds(cfg, cfg->bits_v, a->tpos[1]);
  double thr_unused[15];
  fill_codebook_f64(cfg, cfg->bits_k, thr_unused, a->cen_k);
}

// Shared tail of the packed and dense decode paths: q preparation, split-K
// kernel, merge.
int run_decode(int d, int bk, int bv, int qjl, const DecodePlan& p, DecodeArgs da,
               QPrepArgs qa, int B, int Hq, int Hkv, void* ws, float* out, uint64_t seed,
               hipStream_t st) {
  char* w = static_cast<char*>(ws);
  qa.qp = reinterpret_cast<float*>(w + p.off_qp);
  qa.qq = qjl ? reinterpret_cast<float*>(w + p.off_qq) : nullptr;
  da.qp = qa.qp;
  da.qq = qa.qq;
  da.ml = reinterpret_cast<float*>(w + p.off_ml);
  da.acc = reinterpret_cast<float*>(w + p.off_acc);
  da.cnt = reinterpret_cast<uint32_t*>(w + p.off_cnt);
  da.out = out;
  da.tps = p.tps;
  da.Hkv = Hkv;
  da.Hq = Hq;
  da.G = p.G;
  da.chunks = p.chunks;
  da.S = p.splits;
  da.seed = seed;
  da.q_raw = qa.q;
  da.q_dtype = qa.q_dtype;
  da.qmult = qa.mult;
  int st1 = TQ_OK;
  // the matrix-core kernel rotates its own query rows
  if (!p.mx) st1 = launch_qprep(d, qa, st);
  if (st1 != TQ_OK) return st1;
  DecodeLauncher fn = decode_launcher(d, bk);
  if (!fn) return TQ_ERR_UNSUPPORTED;
  dim3 grid(unsigned(p.splits), unsigned(int64_t(B) * Hkv * p.chunks));
  st1 = fn(bv, p.gk, qjl, p.mx, da, grid, st);
  if (st1 != TQ_OK) return st1;
  // the matrix-core kernel merges its own splits (last workgroup per row)
  if (p.mx) return TQ_OK;
  MergeArgs ma;
  ma.ml = da.ml;
  ma.acc = da.acc;
  ma.out = out;
  ma.heads = int64_t(B) * Hq;
  ma.S = p.splits;
  return launch_merge(d, ma, st);
}

// Decode attention over the first n_ctx tokens; with `app`, token n_ctx - 1
// is first encoded from app's rows (fused into the decode launch when the
// matrix-core kernel runs, else one encode launch before it).
int attend(const tq_config* cfg, const void* q, int q_dtype, int B, int Hq,
           const tq_cache* cache, int64_t n_ctx, float scale, int splits, float* out, void* ws,
           size_t ws_bytes, hipStream_t stream, const EncodeArgs* app, bool chunk = false) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  st = check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!valid_in_dtype(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (B != cache->B || Hq < 1 || Hq % cache->Hkv != 0 || splits < 0) return TQ_ERR_ARG;
  if (!std::isfinite(scale)) return TQ_ERR_ARG;
  if (n_ctx < 1) return TQ_ERR_ARG;
  if (n_ctx > cache->capacity) return TQ_ERR_CAPACITY;
  if (B == 0) return TQ_OK;
  if (!q || !out || !ws) return TQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return TQ_ERR_ALIGN;
  DecodePlan p;
  st = plan_decode(cfg->d, cfg->bits_v, cfg->qjl, B, Hq, cache->Hkv, n_ctx, splits, &p);
  if (st != TQ_OK) return st;
  if (ws_bytes < p.total) return TQ_ERR_WORKSPACE;
  st = device_ready();
  if (st != TQ_OK) return st;
  if (app && (!p.mx || cfg->qjl)) {
    EncodeLauncher efn = encode_launcher(cfg->d, cfg->bits_k);
    if (!efn) return TQ_ERR_UNSUPPORTED;
    st = efn(cfg->bits_v, cfg->qjl != 0, *app, stream);
    if (st != TQ_OK) return st;
    app = nullptr;
  }

  const float tau = scale == 0.f ? 1.0f / std::sqrt(float(cfg->d)) : scale;
  QPrepArgs qa{};
  qa.q = q;
  qa.heads = int64_t(B) * Hq;
  qa.q_dtype = q_dtype;
  qa.rotate = 1;
  qa.pairs = 1;
  qa.qjl = cfg->qjl;
  qa.mult = tau * dev::kLog2e;
  qa.seed = cfg->seed;
  qa.qjl_seed = cfg->qjl_seed;
  sign_bitmap(cfg->seed, cfg->d, qa.sbits);
  sign_bitmap(cfg->qjl_seed, cfg->d, qa.qsbits);

  DecodeArgs da{};
  da.kc = static_cast<const uint8_t*>(cache->kc);
  da.vc = static_cast<const uint8_t*>(cache->vc);
  da.kn = cache->kn;
  da.vn = cache->vn;
  da.kq = static_cast<const uint32_t*>(cache->kq);
  da.kr = static_cast<const uint16_t*>(cache->kr);
  da.capacity = cache->capacity;
  da.n_ctx = n_ctx;
  da.norm_f16 = cfg->norm_dtype == TQ_F16;
  da.inv_sqrt_d = float(1.0 / std::sqrt(double(cfg->d)));
  da.qjl_c = float(std::sqrt(M_PI / (2.0 * cfg->d)));
  da.qjl_seed = cfg->qjl_seed;
  for (int k = 0; k < 8; ++k) {
    da.sbits[k] = qa.sbits[k];
    da.qsbits[k] = qa.qsbits[k];
  }
  const double ak = fill_codebook_f32(cfg, cfg->bits_k, da.cbk);
  const double av = fill_codebook_f32(cfg, cfg->bits_v, da.cbv);
  da.kscale = float(1.0 / (std::sqrt(double(cfg->d)) * ak));
  da.vscale = float(1.0 / (std::sqrt(double(cfg->d)) * av));
  if (app) {
    da.append = 1;
    da.enc = *app;
    if (chunk) {
      // every split decodes a share of the old tokens (a multiple of 64)
      // and of the appended ones, whose rows it encodes first
      da.append = 2;
      da.n_old = n_ctx - app->n_new;
      const int64_t S = p.splits;
      da.tpo = ((da.n_old + S - 1) / S + 63) / 64 * 64;
      da.tpn = (app->n_new + S - 1) / S;
    }
  }
  return run_decode(cfg->d, cfg->bits_k, cfg->bits_v, cfg->qjl, p, da, qa, B, Hq, cache->Hkv,
                    ws, out, cfg->seed, stream);
}

}  // namespace
}  // namespace tq

// ---------------------------------------------------------------------------
// Allocation-free decode: the split partials and the arrival counters live in
// this file-scope device array instead of a caller workspace. Each GPU the
// library runs on holds its own copy until the process ends; it starts zeroed
// and every decode leaves its counters at zero again. Host code must use the
// per-device address from hipGetSymbolAddress, never the array's name.
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace tq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_ERR_NO_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return TQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TQ_OK;
}

}  // namespace
// ---------------------------------------------------------------------------
// Streaming-read probe: every 16-byte chunk of the buffer is loaded once
// with nontemporal (streaming) loads, four chunks in flight per lane,
// XOR-folded; one word per wave is written.
// ---------------------------------------------------------------------------

constexpr int kProbeBlocks = 16384;

__global__ void __launch_bounds__(256) k_read_probe(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u* q = reinterpret_cast<const v4u*>(p);
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    v4u a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = __builtin_nontemporal_load(q + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
  }
  for (; i < n16; i += stride) {
    const v4u a = __builtin_nontemporal_load(q + i);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x ^= __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

}  // namespace tq

using namespace tq;

extern "C" {

int tq_rht(const void* x, int x_dtype, float* y, int64_t rows, int d, uint64_t seed,
           int inverse, hipStream_t stream) {
  if (rows < 0) return TQ_ERR_ARG;
  if (!valid_d(d) || !valid_in_dtype(x_dtype)) return TQ_ERR_UNSUPPORTED;
  if (inverse != 0 && inverse != 1) return TQ_ERR_ARG;
  if (rows == 0) return TQ_OK;
  if (!x || !y) return TQ_ERR_ARG;
  if (!aligned16(x) || !aligned16(y)) return TQ_ERR_ALIGN;
  int st = device_ready();
  if (st != TQ_OK) return st;
  RhtArgs a{x, y, rows, x_dtype, inverse, seed};
  if (d == 128)
    hipLaunchKernelGGL(k_rht<128>, dim3(row_grid(rows)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_rht<256>, dim3(row_grid(rows)), dim3(256), 0, stream, a);
  return last_launch();
}

int tq_encode_kv(const tq_config* cfg, const void* k, const void* v, int in_dtype,
                 int64_t offset, int64_t n_new, const tq_cache* cache, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  st = check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!valid_in_dtype(in_dtype)) return TQ_ERR_UNSUPPORTED;
  if (offset < 0 || n_new < 0) return TQ_ERR_ARG;
  if (offset + n_new > cache->capacity) return TQ_ERR_CAPACITY;
  const int64_t rows = int64_t(cache->B) * cache->Hkv * n_new;
  if (rows == 0) return TQ_OK;
  if (!k || !v) return TQ_ERR_ARG;
  if (!aligned16(k) || !aligned16(v)) return TQ_ERR_ALIGN;
  st = device_ready();
  if (st != TQ_OK) return st;

  EncodeArgs a{};
  fill_encode_args(cfg, k, v, in_dtype, offset, n_new, cache, &a);
  EncodeLauncher fn = encode_launcher(cfg->d, cfg->bits_k);
  if (!fn) return TQ_ERR_UNSUPPORTED;
  return fn(cfg->bits_v, cfg->qjl != 0, a, stream);
}

int tq_qjl_sketch(const float* r, int64_t rows, int d, uint64_t qjl_seed, uint32_t* bits,
                  uint16_t* rnorm_f16, hipStream_t stream) {
  if (rows < 0) return TQ_ERR_ARG;
  if (!valid_d(d)) return TQ_ERR_UNSUPPORTED;
  if (rows == 0) return TQ_OK;
  if (!r || !bits || !rnorm_f16) return TQ_ERR_ARG;
  if (!aligned16(r) || !aligned16(bits) || !aligned16(rnorm_f16)) return TQ_ERR_ALIGN;
  int st = device_ready();
  if (st != TQ_OK) return st;
  QjlArgs a{r, bits, rnorm_f16, rows, qjl_seed};
  if (d == 128)
    hipLaunchKernelGGL(k_qjl<128>, dim3(row_grid(rows)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_qjl<256>, dim3(row_grid(rows)), dim3(256), 0, stream, a);
  return last_launch();
}

int tq_attend_decode(const tq_config* cfg, const void* q, int q_dtype, int B, int Hq,
                     const tq_cache* cache, int64_t n_ctx, float scale, int splits, float* out,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  return attend(cfg, q, q_dtype, B, Hq, cache, n_ctx, scale, splits, out, ws, ws_bytes, stream,
                nullptr);
}

int tq_attend_decode_noalloc(const tq_config* cfg, const void* q, int q_dtype, int B, int Hq,
                             const tq_cache* cache, int64_t n_ctx, float scale, int splits,
                             float* out, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  st = check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (B != cache->B || Hq < 1 || Hq % cache->Hkv != 0 || splits < 0 || n_ctx < 1)
    return TQ_ERR_ARG;
  if (n_ctx > cache->capacity) return TQ_ERR_CAPACITY;
  if (B == 0) return TQ_OK;
  DecodePlan p;
  st = plan_decode(cfg->d, cfg->bits_v, cfg->qjl, B, Hq, cache->Hkv, n_ctx, splits, &p);
  if (st != TQ_OK) return st;
  if (p.total > kScratchBytes) return TQ_ERR_WORKSPACE;
  st = device_ready();
  if (st != TQ_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != TQ_OK) return st;
  return attend(cfg, q, q_dtype, B, Hq, cache, n_ctx, scale, splits, out, ws, kScratchBytes,
                stream, nullptr);
}

int tq_append_attend_decode(const tq_config* cfg, const void* k_new, const void* v_new,
                            int in_dtype, const void* q, int q_dtype, int B, int Hq,
                            const tq_cache* cache, int64_t n_ctx, float scale, int splits,
                            float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  st = check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!valid_in_dtype(in_dtype)) return TQ_ERR_UNSUPPORTED;
  if (n_ctx < 1) return TQ_ERR_ARG;
  if (n_ctx > cache->capacity) return TQ_ERR_CAPACITY;
  if (B != cache->B) return TQ_ERR_ARG;
  if (B == 0) return TQ_OK;
  if (!k_new || !v_new) return TQ_ERR_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return TQ_ERR_ALIGN;
  EncodeArgs e{};
  fill_encode_args(cfg, k_new, v_new, in_dtype, n_ctx - 1, 1, cache, &e);
  return attend(cfg, q, q_dtype, B, Hq, cache, n_ctx, scale, splits, out, ws, ws_bytes, stream,
                &e);
}

int tq_append_chunk_attend_decode(const tq_config* cfg, const void* k_new, const void* v_new,
                                  int in_dtype, int64_t n_new, const void* q, int q_dtype, int B,
                                  int Hq, const tq_cache* cache, int64_t n_ctx, float scale,
                                  int splits, float* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  st = check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!valid_in_dtype(in_dtype)) return TQ_ERR_UNSUPPORTED;
  if (n_ctx < 1 || n_new < 1 || n_new > n_ctx) return TQ_ERR_ARG;
  if (n_ctx > cache->capacity) return TQ_ERR_CAPACITY;
  if (B != cache->B) return TQ_ERR_ARG;
  if (B == 0) return TQ_OK;
  if (!k_new || !v_new) return TQ_ERR_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return TQ_ERR_ALIGN;
  EncodeArgs e{};
  fill_encode_args(cfg, k_new, v_new, in_dtype, n_ctx - n_new, n_new, cache, &e);
  return attend(cfg, q, q_dtype, B, Hq, cache, n_ctx, scale, splits, out, ws, ws_bytes, stream,
                &e, true);
}

int tq_dense_decode_bf16(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                         int d, int64_t n_ctx, float scale, int splits, float* out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (!valid_d(d)) return TQ_ERR_UNSUPPORTED;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || splits < 0 || n_ctx < 1)
    return TQ_ERR_ARG;
  if (!std::isfinite(scale)) return TQ_ERR_ARG;
  if (B == 0) return TQ_OK;
  if (!q || !k || !v || !out || !ws) return TQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws))
    return TQ_ERR_ALIGN;
  DecodePlan p;
  int st = plan_dense(d, B, Hq, Hkv, n_ctx, splits, &p);
  if (st != TQ_OK) return st;
  if (ws_bytes < p.total) return TQ_ERR_WORKSPACE;
  st = device_ready();
  if (st != TQ_OK) return st;

  const float tau = scale == 0.f ? 1.0f / std::sqrt(float(d)) : scale;
  QPrepArgs qa{};
  qa.q = q;
  qa.heads = int64_t(B) * Hq;
  qa.q_dtype = TQ_BF16;
  qa.rotate = 0;
  qa.qjl = 0;
  qa.mult = tau * dev::kLog2e;

  DecodeArgs da{};
  da.kc = static_cast<const uint8_t*>(k);
  da.vc = static_cast<const uint8_t*>(v);
  da.capacity = n_ctx;
  da.n_ctx = n_ctx;
  return run_decode(d, 16, 16, 0, p, da, qa, B, Hq, Hkv, ws, out, 0, stream);
}

int tq_attend_prefill(const tq_config* cfg, const void* q, int q_dtype, int B, int Hq,
                      int64_t n_q, const tq_cache* cache, int64_t n_ctx, float scale, float* out,
                      hipStream_t stream) {
  int st = check_config(cfg);
  if (st != TQ_OK) return st;
  st = check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!valid_in_dtype(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (B != cache->B || Hq < 1 || Hq % cache->Hkv != 0) return TQ_ERR_ARG;
  if (!std::isfinite(scale)) return TQ_ERR_ARG;
  if (n_q < 1 || n_ctx < n_q) return TQ_ERR_ARG;
  if (n_ctx > cache->capacity) return TQ_ERR_CAPACITY;
  if (n_ctx > INT32_MAX) return TQ_ERR_UNSUPPORTED;   // token positions are 32-bit
  const int G = Hq / cache->Hkv;
  const int64_t rows = pf_rows(cfg->d, cfg->qjl != 0);
  const int64_t tiles = (n_q * G + rows - 1) / rows;
  if (tiles > (int64_t(1) << 31) - 1 || int64_t(B) * cache->Hkv > 65535) return TQ_ERR_ARG;
  if (B == 0) return TQ_OK;
  if (!q || !out) return TQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(out)) return TQ_ERR_ALIGN;
  st = device_ready();
  if (st != TQ_OK) return st;

  const float tau = scale == 0.f ? 1.0f / std::sqrt(float(cfg->d)) : scale;
  PrefillArgs a{};
  a.kc = static_cast<const uint8_t*>(cache->kc);
  a.vc = static_cast<const uint8_t*>(cache->vc);
  a.kn = cache->kn;
  a.vn = cache->vn;
  a.q = q;
  a.out = out;
  a.capacity = cache->capacity;
  a.n_ctx = n_ctx;
  a.n_q = n_q;
  a.Hkv = cache->Hkv;
  a.Hq = Hq;
  a.G = G;
  a.q_dtype = q_dtype;
  a.norm_f16 = cfg->norm_dtype == TQ_F16;
  const double ak = fill_codebook_f32(cfg, cfg->bits_k, a.cbk);
  const double av = fill_codebook_f32(cfg, cfg->bits_v, a.cbv);
  a.kscale = float(1.0 / (std::sqrt(double(cfg->d)) * ak));
  a.vscale = float(1.0 / (std::sqrt(double(cfg->d)) * av));
  a.qmult = tau * dev::kLog2e;
  sign_bitmap(cfg->seed, cfg->d, a.sbits);
  a.kq = static_cast<const uint32_t*>(cache->kq);
  a.kr = static_cast<const uint16_t*>(cache->kr);
  a.qjl_c = float(std::sqrt(M_PI / (2.0 * cfg->d)));
  sign_bitmap(cfg->qjl_seed, cfg->d, a.qsbits);
  const dim3 grid(unsigned(tiles), unsigned(int64_t(B) * cache->Hkv));
  return cfg->d == 128
             ? launch_prefill_d128(cfg->bits_k, cfg->bits_v, cfg->qjl, a, grid, stream)
             : launch_prefill_d256(cfg->bits_k, cfg->bits_v, cfg->qjl, a, grid, stream);
}

int64_t tq_read_probe_sink_words(int64_t bytes) {
  if (bytes < 0) return TQ_ERR_ARG;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + 255) / 256;
  return 4 * (blocks < kProbeBlocks ? blocks : kProbeBlocks);
}

int tq_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0) return TQ_ERR_ARG;
  if (bytes == 0) return TQ_OK;
  if (!src || !sink) return TQ_ERR_ARG;
  if (!aligned16(src)) return TQ_ERR_ALIGN;
  int st = device_ready();
  if (st != TQ_OK) return st;
  const unsigned blocks = unsigned(tq_read_probe_sink_words(bytes) / 4);
  hipLaunchKernelGGL(k_read_probe, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return last_launch();
}

}  // extern "C"
