/*
 * tq.h - TurboQuant KV-cache decode path for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libtq.so. Plain pointers and sizes only.
 *
 * The method (see the pages "TurboQuant Performance Benefits: Memory
 * Reduction and Speed Optimization in MLX-VLM", "How to Use TurboQuant with
 * the MLX-VLM Python API: A Complete Guide" and the mlx-turboquant README):
 *   - K and V rows are rotated by a seeded randomized Hadamard transform
 *     R = H_d diag(s) / sqrt(d) (sign flip, then a normalized Walsh-Hadamard
 *     transform in Sylvester order; s from SplitMix64 seeded with `seed`,
 *     s_i = -1 when the top bit of the i-th output is set);
 *   - each row is normalized (one norm per row, stored rounded to the norm
 *     dtype) and every coordinate of z = sqrt(d) R x / ||x|| is quantized
 *     against the N(0,1) Lloyd-Max codebook: code = #{k : z >= t_k};
 *   - codes are bit-packed: code i of a row sits at bits [b*i, b*i + b) of the
 *     row's little-endian byte string;
 *   - decode attention runs on the packed codes: the query is rotated into
 *     the same frame, scores come from codebook lookups, the softmax is
 *     online, values are dequantized and accumulated in the same pass;
 *   - optionally a 1-bit QJL sketch of the key residual r = R k - k_hat
 *     (sign bits of R_2 r, R_2 built like R from `qjl_seed`, plus ||r|| in
 *     fp16) corrects the score by sqrt(pi/(2d)) ||r|| <R_2 R q, sign(R_2 r)>.
 *
 * Conventions shared by every entry point:
 *   - Device buffers are allocated and owned by the caller. The library never
 *     allocates, frees or synchronizes; every call only enqueues work on
 *     `stream` (0 = the null stream) and returns.
 *   - Every argument is validated on the host before any HIP call. A failed
 *     validation returns a negative tq_status and touches no memory.
 *   - Device pointers must be 16-byte aligned (TQ_ERR_ALIGN otherwise).
 *   - Functions are stateless and may be called from several host threads.
 *   - No C++ exception crosses this interface.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = -1,          /* null pointer, negative size, inconsistent shape  */
  TQ_ERR_UNSUPPORTED = -2,  /* d not in {128,256}, bits not in {2,3,4}, dtype   */
  TQ_ERR_ALIGN = -3,        /* a device pointer is not 16-byte aligned          */
  TQ_ERR_CAPACITY = -4,     /* offset + n_new > capacity, or n_ctx > capacity   */
  TQ_ERR_WORKSPACE = -5,    /* workspace smaller than tq_workspace_bytes()      */
  TQ_ERR_NO_DEVICE = -6,    /* no HIP device visible                           */
  TQ_ERR_HIP = -7           /* a HIP launch or runtime call failed              */
} tq_status;

/* Element types of inputs (q, k, v, x) and of the per-row norms. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;
typedef enum { TQ_CODEBOOK_GAUSS = 0, TQ_CODEBOOK_SPHERE = 1 } tq_codebook_kind;

/* Static description of one quantized cache format. */
typedef struct {
  int d;              /* head dimension: 128 or 256                           */
  int bits_k;         /* key code width: 2, 3 or 4                            */
  int bits_v;         /* value code width: 2, 3 or 4                          */
  int norm_dtype;     /* TQ_F16 or TQ_F32: storage of the per-row norms       */
  int qjl;            /* 1: keys also carry the 1-bit QJL residual sketch     */
  uint64_t seed;      /* SplitMix64 seed of the rotation signs s              */
  uint64_t qjl_seed;  /* SplitMix64 seed of the QJL rotation R_2              */
  int codebook;       /* TQ_CODEBOOK_GAUSS (0): Lloyd-Max for N(0,1);
                         TQ_CODEBOOK_SPHERE (1): Lloyd-Max for the exact
                         finite-d marginal of sqrt(d) * a coordinate of a
                         uniform unit vector, density proportional to
                         (1 - z^2/d)^((d-3)/2): the exact law whose shape
                         the README's introduction calls near-Gaussian   */
} tq_config;

/*
 * Caller-owned device planes of a packed cache with B batch entries, Hkv KV
 * heads and room for `capacity` tokens. Row (b, h, t) is record
 * (b * Hkv + h) * capacity + t of every plane:
 *   kc : d*bits_k/8 bytes per record (packed key codes)
 *   vc : d*bits_v/8 bytes per record (packed value codes)
 *   kn : key norm   (2 bytes if norm_dtype == TQ_F16, else 4)
 *   vn : value norm (same dtype as kn)
 *   kq : d/8 bytes per record, QJL sign bits; as little-endian uint32 words,
 *        coordinate 32m + j is bit j of word m; bit = 1 where (R_2 r)_i < 0
 *        (only when qjl, else may be NULL)
 *   kr : fp16 ||r|| per record (only when qjl, else may be NULL)
 * tq_cache_bytes() gives each plane's size.
 */
typedef struct {
  void* kc;
  void* vc;
  void* kn;
  void* vn;
  void* kq;
  void* kr;
  int B;
  int Hkv;
  int64_t capacity;
} tq_cache;

/*
 * Fractional bit widths (performance page, "Fractional-Bit Precision
 * Support"; API page, "How TurboQuant Activation Works").
 * *enabled = 0 when TurboQuant is not selected: kv_bits is not finite-and-
 * fractional and force_turboquant is 0 (the uniform fallback, not provided
 * here); bits_k / bits_v are then left untouched. Otherwise *enabled = 1 and
 * bits_k = floor(kv_bits), bits_v = ceil(kv_bits) for a fractional width
 * (3.5 -> 3/4), or both = kv_bits for an integer width. A width within 1e-6
 * of an integer counts as that integer.
 * Returns TQ_OK, TQ_ERR_ARG (null output pointer, non-finite kv_bits) or
 * TQ_ERR_UNSUPPORTED (a resulting width outside 2..4). Host only.
 */
int tq_bits_split(double kv_bits, int force_turboquant, int* enabled,
                  int* bits_k, int* bits_v);

/*
 * N(0,1) Lloyd-Max codebook for `bits` in 1..4 (performance page, "What Is
 * TurboQuant?": MSE code-book; README: Lloyd-Max LUT). Writes 2^bits
 * ascending centroids and 2^bits - 1 thresholds t_k = (c_{k-1} + c_k) / 2
 * (host arrays, either may be NULL). Computed in double on the host.
 */
int tq_codebook(int bits, double* centroids, double* thresholds);

/* The codebook a tq_config's `codebook` field selects, in the layout of
 * tq_codebook: kind TQ_CODEBOOK_GAUSS (d ignored) or TQ_CODEBOOK_SPHERE
 * (d 128 or 256). TQ_ERR_UNSUPPORTED for other bits, kinds or d. Each
 * codebook is computed on the host at its first use (a finite-d one takes
 * up to about a second) and cached for the life of the process. */
int tq_codebook_ex(int bits, int kind, int d, double* centroids, double* thresholds);

/* The +-1 rotation signs for (seed, d) as int8 (host array of d): the random
 * diagonal of the deterministic rotation (API page, "What is TurboQuant?":
 * a seeded random rotation before the codebook; README: randomized
 * Hadamard). Host only. TQ_ERR_ARG for a NULL out or d < 1. */
int tq_signs(uint64_t seed, int d, int8_t* out);

/*
 * Bytes of each plane of a cache (capacity tokens) written to
 * plane_bytes[6] in the order kc, vc, kn, vn, kq, kr (may be NULL): the
 * packed codes at bits_k and bits_v per coordinate plus one norm per row
 * (performance page, "Aggressive Compression Ratios"), and with QJL one
 * sign bit per key coordinate plus a residual norm (README, "The 1-bit QJL
 * residual": +1 bit per channel). Returns the total, or a negative
 * tq_status.
 */
int64_t tq_cache_bytes(const tq_config* cfg, int B, int Hkv, int64_t capacity,
                       int64_t* plane_bytes);

/*
 * Rotate rows: y = R x (inverse = 0) or y = R^T x (inverse = 1).
 * x: [rows][d] of x_dtype (device); y: [rows][d] fp32 (device), may alias x
 * only when x_dtype == TQ_F32. d in {128, 256}. rows == 0 is a no-op.
 * (API page: _rht_forward / _rht_inverse; README: randomized Hadamard.)
 */
int tq_rht(const void* x, int x_dtype, float* y, int64_t rows, int d,
           uint64_t seed, int inverse, hipStream_t stream);

/*
 * Encode n_new tokens of K and V into the cache at token positions
 * [offset, offset + n_new) of every (b, h) row (performance page, "What Is
 * TurboQuant?"; README, "The 1-bit QJL residual").
 * k, v: [B][Hkv][n_new][d] contiguous, in_dtype TQ_F32/TQ_BF16/TQ_F16.
 * Writes kc, vc, kn, vn (and kq, kr when cfg->qjl) of those positions only.
 * Converting a dense cache is offset = 0, n_new = length; a decode-time
 * append is offset = length, n_new = 1. n_new == 0 is a no-op.
 * Codes are computed in double precision, so they equal the exact
 * definition except where z lies exactly on a threshold.
 */
int tq_encode_kv(const tq_config* cfg, const void* k, const void* v,
                 int in_dtype, int64_t offset, int64_t n_new,
                 const tq_cache* cache, hipStream_t stream);

/*
 * Standalone QJL sketch of residual rows (README, "The 1-bit QJL residual").
 * r: [rows][d] fp32 (device). Writes bits: [rows][d/32] uint32 words
 * (coordinate 32m + j at bit j of word m; 1 where (R_2 r)_i < 0) and
 * rnorm_f16: [rows] fp16 bit patterns of ||r||. d in {128, 256}.
 * tq_encode_kv with qjl = 1 produces the same bits as encoding without QJL,
 * forming r = R k - k_hat_rot, and calling this.
 */
int tq_qjl_sketch(const float* r, int64_t rows, int d, uint64_t qjl_seed,
                  uint32_t* bits, uint16_t* rnorm_f16, hipStream_t stream);

/*
 * Split count tq_attend_decode uses for these sizes (splits = 0 means the
 * library's choice). Returns >= 1, or a negative tq_status.
 */
int tq_num_splits(const tq_config* cfg, int B, int Hq, int Hkv, int64_t n_ctx,
                  int splits);

/* Workspace bytes tq_attend_decode needs; negative tq_status on bad args
 * (TQ_ERR_ARG also when B * Hkv * head groups exceeds 65535).
 * The workspace starts with 65535 arrival counters (256 KB, one per
 * (batch, KV head, head group) row of the decode grid): on the matrix-core
 * kernel (d 128 or 256) the last workgroup of each row to finish merges the
 * row's split partials, which follow the counters. The counters must read
 * zero when a call starts: zero the buffer once before its first use. Every
 * call leaves them at zero again, so the same buffer serves later calls of
 * any shape that fits. Two calls that share a workspace must not run at the
 * same time. */
int64_t tq_workspace_bytes(const tq_config* cfg, int B, int Hq, int Hkv,
                           int64_t n_ctx, int splits);

/*
 * One decode step of attention over the first n_ctx tokens of the cache
 * (performance page, "Custom Metal Kernel Implementation": scores on packed
 * codes fused with value aggregation; README, "How it plugs in": the query
 * is rotated and the QJL correction added).
 *   q:   [B][Hq][d] of q_dtype (device). Hq must be a multiple of cache->Hkv;
 *        query head h reads KV head h / (Hq / Hkv).
 *   out: [B][Hq][d] fp32 (device):
 *        out = softmax_j(scale * <q, k_hat_j> [+ QJL term]) . v_hat_j
 *        with k_hat / v_hat the dequantized rows in the original frame.
 *   scale: 0 selects 1/sqrt(d).
 *   splits: 0 lets the library choose (see tq_num_splits).
 *   ws:  device workspace of at least tq_workspace_bytes() bytes, zero before
 *        its first use (see tq_workspace_bytes).
 * n_ctx must be in [1, capacity]. The result does not depend on host
 * threads or on timing: partials are merged in a fixed order.
 * Precision and range: products run on fp16 operands with fp32
 * accumulation. The rotated query and the softmax weights times the value
 * norms are scaled by powers of two (undone in fp32) that keep them inside
 * fp16's normal range for any finite input, so large or tiny values and
 * queries neither overflow nor flush to zero. The query is rounded to fp16
 * (relative 2^-11 per element), so a score's error grows with |q| |k|: the
 * output's max row-relative error against fp64 is about 5e-4 for
 * unit-variance q and k (scores spanning a few log2 units) and about 2e-3
 * when q is 10x larger.
 * Kernels: d 128 and 256 run on the matrix cores; other head dims, or every
 * format when the environment variable TQ_DECODE_VALU is "1" when the call
 * is planned, run on a vector-ALU kernel with the same results contract.
 */
int tq_attend_decode(const tq_config* cfg, const void* q, int q_dtype, int B,
                     int Hq, const tq_cache* cache, int64_t n_ctx, float scale,
                     int splits, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as tq_attend_decode, with the same arguments minus the workspace.
 * The split partials and arrival counters live in a static 8 MiB device
 * buffer inside the library, one per GPU, held until the process ends; the
 * library allocates and frees nothing. Returns TQ_ERR_WORKSPACE, before any
 * HIP call, when the call needs more than 8 MiB (tq_workspace_bytes() of the
 * same arguments), e.g. B * Hq * splits * (d + 2) * 4 bytes beyond ~7.7 MiB.
 * Every call on one GPU shares that buffer: calls that overlap in time on the
 * same GPU (two streams, two host threads) race and must not be issued.
 */
int tq_attend_decode_noalloc(const tq_config* cfg, const void* q, int q_dtype, int B,
                             int Hq, const tq_cache* cache, int64_t n_ctx, float scale,
                             int splits, float* out, hipStream_t stream);

/*
 * One generation step: append the newest token, then attend (README, "How it
 * plugs in": the cache stores the new rotated key and value, then the
 * patched scaled_dot_product_attention runs on the rotated query; API page,
 * "Implementation Details: Cache Substitution"). Same result, cache bytes
 * and output, as
 *   tq_encode_kv(cfg, k_new, v_new, in_dtype, n_ctx - 1, 1, cache, stream);
 *   tq_attend_decode(cfg, q, q_dtype, B, Hq, cache, n_ctx, ...);
 *   k_new, v_new: [B][Hkv][1][d] of in_dtype (device), 16-byte aligned: the
 *                 rows of token n_ctx - 1.
 * The other arguments, the workspace and the errors are those of
 * tq_attend_decode; all arguments are checked before any work is queued.
 * For formats with 2- or 4-bit values and no QJL this is one launch: the
 * workgroup that owns the last split encodes the token before its first
 * tile. The other formats queue the encode and the decode back to back.
 */
int tq_append_attend_decode(const tq_config* cfg, const void* k_new,
                            const void* v_new, int in_dtype, const void* q,
                            int q_dtype, int B, int Hq, const tq_cache* cache,
                            int64_t n_ctx, float scale, int splits, float* out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One step that appends a chunk of n_new tokens and attends (README, "How
 * it plugs in": the cache stores the new rotated keys and values, then
 * attention runs on the rotated query; API page, "Implementation Details:
 * Cache Substitution"). Same result (up to the order of the sums) and the
 * same cache bytes as
 *   tq_encode_kv(cfg, k_new, v_new, in_dtype, n_ctx - n_new, n_new, cache, stream);
 *   tq_attend_decode(cfg, q, q_dtype, B, Hq, cache, n_ctx, ...);
 *   k_new, v_new: [B][Hkv][n_new][d] of in_dtype (device), 16-byte aligned:
 *                 the rows of tokens n_ctx - n_new .. n_ctx - 1.
 * 1 <= n_new <= n_ctx (else TQ_ERR_ARG); the other arguments, the workspace
 * and the errors are those of tq_attend_decode; all arguments are checked
 * before any work is queued. On the matrix-core decode without QJL this is
 * one launch: every split decodes a share of the older tokens and a share
 * of the new ones, and its workgroup encodes its new rows first. Other
 * formats queue the encode and the decode back to back.
 */
int tq_append_chunk_attend_decode(const tq_config* cfg, const void* k_new,
                                  const void* v_new, int in_dtype, int64_t n_new,
                                  const void* q, int q_dtype, int B, int Hq,
                                  const tq_cache* cache, int64_t n_ctx, float scale,
                                  int splits, float* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * Causal multi-query attention of a prefill chunk over the packed cache
 * (the time-to-first-token path the README times in "Throughput, latency &
 * memory"; the API page's patched attention, "Implementation Details: Cache
 * Substitution", rotates the queries into the cache's frame).
 * The chunk's n_q tokens must already be in the cache (tq_encode_kv at
 * offset n_ctx - n_q); query i of the chunk sits at position
 * n_ctx - n_q + i and attends to cache tokens 0 .. that position:
 *   out[b][h][i] = sum_{j <= n_ctx-n_q+i} softmax_j(scale <q[b][h][i], k_hat_j>)
 *                  v_hat_j,   KV head of h = h / (Hq / Hkv)
 *   q   : [B][Hq][n_q][d] of q_dtype (device, 16-byte aligned)
 *   out : [B][Hq][n_q][d] fp32 (device, caller-owned, 16-byte aligned)
 *   scale: 0 selects 1/sqrt(d). No workspace.
 * With cfg->qjl the QJL term of tq_attend_decode is added to every score.
 * Errors (before any work is queued): TQ_ERR_ARG (1 <= n_q <= n_ctx
 * violated, Hq not a multiple of Hkv, B != cache B, null pointers),
 * TQ_ERR_CAPACITY (n_ctx > capacity), TQ_ERR_ALIGN, TQ_ERR_UNSUPPORTED
 * (d, bit widths, codebook or q dtype, or n_ctx above 2^31 - 1: the kernel
 * holds token positions in 32 bits).
 */
int tq_attend_prefill(const tq_config* cfg, const void* q, int q_dtype, int B, int Hq,
                      int64_t n_q, const tq_cache* cache, int64_t n_ctx, float scale,
                      float* out, hipStream_t stream);

/*
 * Dense bf16 decode attention for comparison on the same GPU (not part of
 * the method): out = softmax(scale q K^T) V over k, v: [B][Hkv][n_ctx][d]
 * bf16, q: [B][Hq][d] bf16, out fp32. Same workspace rules
 * (tq_dense_workspace_bytes).
 */
int64_t tq_dense_workspace_bytes(int B, int Hq, int Hkv, int d, int64_t n_ctx,
                                 int splits);
int tq_dense_decode_bf16(const void* q, const void* k, const void* v, int B,
                         int Hq, int Hkv, int d, int64_t n_ctx, float scale,
                         int splits, float* out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Streaming-read probe for bandwidth measurement (not part of the method):
 * reads `bytes` bytes at `src` once with 16-byte nontemporal loads and writes the XOR of
 * every 32-bit word a wave read to sink[w], one word per wave of the launch
 * (the XOR of all of sink[0 .. tq_read_probe_sink_words(bytes)) is the XOR of
 * every word of the buffer). src: device, 16-byte aligned, bytes a multiple
 * of 16; sink: device, caller-owned. Returns TQ_ERR_ARG / TQ_ERR_ALIGN
 * before queueing anything when these do not hold.
 */
int64_t tq_read_probe_sink_words(int64_t bytes);
int tq_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * Group-affine variant (mlx-turboquant README: "Quantize the KV cache" with
 * kv_group_size = 64; "How it plugs in": the cache is mlx-lm's group-affine
 * quantized cache with the keys rotated and the query rotated at attention
 * time; "Memory footprint over long context": the same bytes per token as
 * the 4-bit codebook cache). Per token and KV head: d codes of b bits
 * (LSB-first bitstream, as the codebook cache) and, per group of 64
 * coordinates, an fp16 scale and an fp16 bias. Keys are rotated by R (seed)
 * first, values are stored in their own frame. Encoding a group y: bias =
 * fp16(min y), scale = fp16((max y - min y) / (2^b - 1)), code =
 * round-half-even((y - bias) / scale) clamped to [0, 2^b - 1] (0 when scale
 * is 0), all in double precision; dequantized value scale * code + bias.
 */
typedef struct {
  int d;              /* head dimension: 128 or 256                           */
  int bits_k;         /* key code width: 2, 3 or 4                            */
  int bits_v;         /* value code width: 2, 3 or 4                          */
  int group;          /* coordinates per scale and bias: must be 64           */
  uint64_t seed;      /* SplitMix64 seed of the key rotation signs            */
} tq_affine_config;

/* Device planes (caller-owned, 16-byte aligned), rows [B][Hkv][capacity]:
 * kc, vc: d*bits/8 bytes per row; ks, kb, vs, vb: d/64 fp16 per row. */
typedef struct {
  void* kc;
  void* vc;
  void* ks;
  void* kb;
  void* vs;
  void* vb;
  int B;
  int Hkv;
  int64_t capacity;
} tq_affine_cache;

/* Total bytes of the six planes; plane_bytes[6] (kc, vc, ks, kb, vs, vb) may
 * be NULL. Negative tq_status on bad arguments. Host only. */
int64_t tq_affine_cache_bytes(const tq_affine_config* cfg, int B, int Hkv,
                              int64_t capacity, int64_t* plane_bytes);

/* Encode n_new tokens of K and V into rows [offset, offset + n_new) of every
 * (b, h); k, v: [B][Hkv][n_new][d] of in_dtype, 16-byte aligned. Same
 * argument rules and errors as tq_encode_kv. */
int tq_affine_encode_kv(const tq_affine_config* cfg, const void* k, const void* v,
                        int in_dtype, int64_t offset, int64_t n_new,
                        const tq_affine_cache* cache, hipStream_t stream);

/* Split count and workspace bytes of tq_affine_attend_decode. */
int tq_affine_num_splits(const tq_affine_config* cfg, int B, int Hq, int Hkv,
                         int64_t n_ctx, int splits);
int64_t tq_affine_workspace_bytes(const tq_affine_config* cfg, int B, int Hq,
                                  int Hkv, int64_t n_ctx, int splits);

/* Decode attention over the first n_ctx tokens of an affine cache:
 * out[b][h] = sum_j softmax_j(scale * <R q, y_hat_j>) v_hat_j, fp32, with
 * y_hat the dequantized rotated keys and v_hat the dequantized values.
 * Arguments, workspace and errors as tq_attend_decode. 4-bit keys and values
 * at d 128 run on the matrix cores (fp16 operands, fp32 accumulation; codes
 * exact); other formats, or every format when TQ_DECODE_VALU is "1", on a
 * vector-ALU kernel. */
int tq_affine_attend_decode(const tq_affine_config* cfg, const void* q, int q_dtype,
                            int B, int Hq, const tq_affine_cache* cache,
                            int64_t n_ctx, float scale, int splits, float* out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Human-readable name of a tq_status. Never NULL. */
const char* tq_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
