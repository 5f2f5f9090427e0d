// Kernel templates of libtq.so (gfx950, wave64). Instantiated by the
// tq_inst_*.hip translation units and launched from tq_api.hip.
#pragma once

#include "tq_device.h"

namespace tq {

// ---------------------------------------------------------------------------
// Arguments
// ---------------------------------------------------------------------------

struct RhtArgs {
  const void* x;
  float* y;
  int64_t rows;
  int x_dtype;
  int inverse;
  uint64_t seed;
};

// Encode of one token range of K and V into the packed cache (one launch,
// blockIdx.z selects the tensor).
struct EncodeArgs {
  const void* x[2];       // K rows, V rows: [B*Hkv][n_new][D]
  uint8_t* codes[2];      // packed code planes
  void* norms[2];         // fp16 or fp32 norm planes
  uint8_t* qbits;         // QJL sign plane (keys with QJL only)
  uint16_t* rnorm;        // QJL residual-norm plane
  int64_t n_new, offset, capacity;
  int BH;                 // B * Hkv
  int in_dtype;
  int norm_f16;
  uint32_t sbits[8];      // rotation signs, bit i set when sign i is negative
  uint32_t qsbits[8];     // QJL rotation signs, same layout
  double tpos[2][7];      // thresholds t_{L/2} .. t_{L-2} of K and V (t_{L/2-1} = 0)
  double cen_k[16];       // key centroids, ascending (QJL residual)
};

struct QjlArgs {
  const float* r;
  uint32_t* bits;
  uint16_t* rnorm;
  int64_t rows;
  uint64_t qjl_seed;
};

struct QPrepArgs {
  const void* q;          // [B*Hq][D]
  float* qp;              // [B*Hq][D]: scale*log2(e) * R q   (or unrotated)
  float* qq;              // [B*Hq][D]: R_2 qp (QJL only)
  int64_t heads;
  int q_dtype;
  int rotate;             // 0: dense baseline, no rotation
  int pairs;              // 1: write qp as fp16 pairs (packed decode)
  int qjl;
  float mult;             // scale * log2(e)
  uint64_t seed, qjl_seed;
  uint32_t sbits[8];      // rotation signs, bit i set when sign i is negative
  uint32_t qsbits[8];     // QJL rotation signs, same layout
};

struct DecodeArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const void* kn;
  const void* vn;
  const uint32_t* kq;
  const uint16_t* kr;
  const float* qp;
  const float* qq;
  float* ml;              // [B*Hq][S][2]  (max in log2 units, sum)
  float* acc;             // [B*Hq][S][D]
  int64_t capacity, n_ctx, tps;
  int Hkv, Hq, G, chunks, S;
  int norm_f16;
  float inv_sqrt_d;
  float kscale;           // 1 / (sqrt(d) * alpha_k): fp32 part of the key scale
  float vscale;           // 1 / (sqrt(d) * alpha_v)
  float qjl_c;            // sqrt(pi / (2 d))
  uint64_t qjl_seed;      // QJL rotation seed (kernels that rotate the query)
  float cbk[16];          // alpha_k * key centroids (exact in fp16 to ~1e-4)
  float cbv[16];          // alpha_v * value centroids
  uint64_t seed;          // rotation seed: partials are rotated back (R^T)
  const void* q_raw;      // [B*Hq][D] queries, for kernels that rotate them themselves
  int q_dtype;
  float qmult;            // scale * log2(e)
  uint32_t sbits[8];      // rotation signs, bit i set when sign i is negative
  uint32_t qsbits[8];     // QJL rotation signs, same layout
  int append;             // 1: the last split first encodes token n_ctx - 1 (enc);
                          // 2: every split first encodes its share of the
                          //    enc.n_new appended tokens (below)
  EncodeArgs enc;         // the appended K/V rows and the cache planes
  // append == 2: split s reads old tokens [s tpo, s tpo + tpo) (tpo a multiple
  // of 64) below n_old, then new tokens [n_old + s tpn, n_old + s tpn + tpn)
  int64_t n_old, tpo, tpn;
  uint32_t* cnt;          // [grid.y] arrival counters (zero between calls)
  float* out;             // [B*Hq][D] output of kernels that merge their splits
};

struct MergeArgs {
  const float* ml;
  const float* acc;
  float* out;
  int64_t heads;
  int S;
};

// ---------------------------------------------------------------------------
// tq_rht: 16 lanes per row, E = D/16 elements per lane, fp32.
// ---------------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(256) k_rht(RhtArgs a) {
  constexpr int E = D / 16;
  const int l16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const uint32_t smask = dev::sign_mask(a.seed, l16 * E, E);
  const float norm = 1.0f / sqrtf(float(D));
  for (int64_t row = int64_t(blockIdx.x) * 16 + grp; row < a.rows;
       row += int64_t(gridDim.x) * 16) {
    float v[E];
    dev::load_row_part<E>(a.x, a.x_dtype, row * D + l16 * E, v);
    if (!a.inverse) {
#pragma unroll
      for (int i = 0; i < E; ++i) if (smask >> i & 1) v[i] = -v[i];
    }
    dev::fwht16<E, float>(v, l16);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      v[i] *= norm;
      if (a.inverse && (smask >> i & 1)) v[i] = -v[i];
    }
    float4* dst = reinterpret_cast<float4*>(a.y + row * D + l16 * E);
#pragma unroll
    for (int k = 0; k < E / 4; ++k)
      dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// ---------------------------------------------------------------------------
// Encode: rotation, norm, quantization and packing of one K or V plane, a
// row on P = D/32 lanes with 32 coordinates each. The transform and the
// comparisons run in double: the Hadamard sums of bf16 inputs are then
// exact, so the codes equal the definition except for values lying exactly
// on a threshold.
// ---------------------------------------------------------------------------

// Dword k (k < 8) of 8 uniform dwords for a lane-dependent k: a select
// chain, so the index needs no private memory.
__device__ __forceinline__ uint32_t pick8(const uint32_t (&w)[8], int k) {
  uint32_t x = w[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) x = (k == j) ? w[j] : x;
  return x;
}

// x from lane (lane ^ M) of the same quad (M = 1 or 2), through DPP
// quad_perm on the two halves of the double.
template <int M>
__device__ __forceinline__ double quad_xor_f64(double x) {
  constexpr int CTRL = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t bits = uint64_t(__double_as_longlong(x));
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(bits)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(bits >> 32)), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}

template <int M>
__device__ __forceinline__ double lane_xor_f64(double x) {
  if constexpr (M <= 2) return quad_xor_f64<M>(x);
  else return __shfl_xor(x, M, 2 * M);
}

// Walsh-Hadamard transform (unnormalized, Sylvester order) of a row spread
// over P consecutive lanes, 32 coordinates each (coordinate = lane_in_row *
// 32 + i): five butterfly stages inside the lane, log2(P) across lanes. In a
// cross-lane stage the lower lane of a pair keeps x + y and the upper one
// x - y, so each lane computes partner + sg * own with sg[s] = +1 or -1.
template <int P>
__device__ __forceinline__ void fwht32xP(double (&v)[32], const double (&sg)[3]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        const double x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
    }
  }
  // eight coordinates at a time, so that at most 16 partner registers are
  // live on top of the row
  dev::static_for<0, (P == 8 ? 3 : 2)>([&](auto sc) {
    constexpr int st = decltype(sc)::value;
#pragma unroll
    for (int i0 = 0; i0 < 32; i0 += 8) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i) v[i] = fma(v[i], sg[st], lane_xor_f64<(1 << st)>(v[i]));
    }
  });
  __builtin_amdgcn_sched_barrier(0);
  // pin the results here: otherwise the last stage is sunk past the norm
  // branches to its uses and its 32 partner values stay live meanwhile
#pragma unroll
  for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(v[i]));
}

template <int P>
__device__ __forceinline__ double group_sum_f64(double x) {
  x += lane_xor_f64<1>(x);
  x += lane_xor_f64<2>(x);
  if constexpr (P == 8) x += lane_xor_f64<4>(x);
  return x;
}

// k_encode's strided row layout: with S = 5 - log2(P), lane lp of a row holds
// the coordinates whose bits [S, 5) equal lp, its register j the one with
// bits [0, S) = j mod 2^S and bits [5, 5 + log2 P) = j / 2^S. A lane then
// reads P segments of 2^S consecutive elements, and the butterflies on all
// bits but [S, 5) stay inside the lane.
template <int P>
__host__ __device__ constexpr int enc_seg_bits() {
  static_assert(P == 4 || P == 8, "rows of 128 or 256 coordinates");
  return P == 4 ? 3 : 2;
}
template <int P>
__host__ __device__ constexpr int strided_coord(int lp, int j) {
  return ((j >> enc_seg_bits<P>()) << 5) | (lp << enc_seg_bits<P>()) |
         (j & ((1 << enc_seg_bits<P>()) - 1));
}

// One lane's 32 input coordinates as raw 16-byte words: 4 for 16-bit inputs
// (IW = 2 bytes per element), 8 for fp32.
template <int IW>
struct RowWords {
  uint4 q[2 * IW];
};

// Per-lane constants of the encode kernel: the rotation signs of the lane's
// 32 coordinates (for 16-bit inputs as XOR masks on the packed element
// pairs: bit 15 and bit 31), and the cross-lane butterfly signs.
template <int IW>
struct EncodeLane {
  uint32_t smask;
  uint32_t pm[IW == 2 ? 16 : 1];
  uint32_t qmask;
  double sg[3];
  int lp;
};

template <int D, int IW>
__device__ __forceinline__ void load_words(const EncodeArgs& a, int z, int bh, int64_t t, int lp,
                                           RowWords<IW>& r) {
  const int64_t tc = t < a.n_new ? t : a.n_new - 1;   // rows past the end re-read the last one
  const int64_t row = int64_t(bh) * a.n_new + tc;
  const uint4* s = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.x[z]) +
                                                  (row * D + lp * 32) * IW);
#pragma unroll
  for (int k = 0; k < 2 * IW; ++k) r.q[k] = s[k];
}

// The lane's 32 input coordinates in k_encode's strided layout: P segments of
// 32 IW / P bytes (rows past the end re-read the last one).
template <int D, int IW>
__device__ __forceinline__ void load_words_strided(const EncodeArgs& a, int z, int bh, int64_t t,
                                                   int lp, RowWords<IW>& r) {
  constexpr int P = D / 32;
  constexpr int SEG = 32 * IW / P;
  const int64_t tc = t < a.n_new ? t : a.n_new - 1;
  const uint8_t* row =
      static_cast<const uint8_t*>(a.x[z]) + (int64_t(bh) * a.n_new + tc) * (D * IW);
#pragma unroll
  for (int g = 0; g < P; ++g) {
    const uint8_t* src = row + strided_coord<P>(lp, g << enc_seg_bits<P>()) * IW;
    if constexpr (SEG >= 16) {
#pragma unroll
      for (int k = 0; k < SEG / 16; ++k)
        r.q[g * (SEG / 16) + k] = reinterpret_cast<const uint4*>(src)[k];
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(src);
      if (g & 1) {
        r.q[g >> 1].z = w.x;
        r.q[g >> 1].w = w.y;
      } else {
        r.q[g >> 1].x = w.x;
        r.q[g >> 1].y = w.y;
      }
    }
  }
}

// Sign-flipped coordinates x_i * s_i as doubles, and sum of squares (DT:
// 0 fp32, 1 bf16, 2 fp16).
template <int DT, int IW = (DT == 0 ? 4 : 2)>
__device__ __forceinline__ double words_to_f64(const RowWords<IW>& r, const EncodeLane<IW>& el,
                                               double (&u)[32]) {
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 2 * IW; ++k) {
    const uint32_t w4[4] = {r.q[k].x, r.q[k].y, r.q[k].z, r.q[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (IW == 2) {
        const int e = 8 * k + 2 * j;
        const uint32_t w = w4[j] ^ el.pm[4 * k + j];
        float lo, hi;
        if constexpr (DT == 1) {
          lo = __uint_as_float(w << 16);
          hi = __uint_as_float(w & 0xFFFF0000u);
        } else {
          lo = dev::f16_to_f32(w & 0xFFFFu);
          hi = dev::f16_to_f32(w >> 16);
        }
        u[e] = lo;
        u[e + 1] = hi;
        ss = fma(u[e], u[e], ss);
        ss = fma(u[e + 1], u[e + 1], ss);
      } else {
        const int e = 4 * k + j;
        const uint32_t w = w4[j] ^ ((el.smask << (31 - e)) & 0x80000000u);
        u[e] = __uint_as_float(w);
        ss = fma(u[e], u[e], ss);
      }
    }
  }
  return ss;
}

// LDS cells (16 bytes: two doubles) of the transpose from the strided to the
// contiguous layout, for one wave's 64/P rows. It runs in two rounds, one
// per value of coordinate bit 1, each moving half of every row; chunk c of
// a round is coordinate >> 2, and (row r, chunk c) lives in cell
// r RS + (r >> 1) E1 + c + (c >> 3) p3. The padding keeps every write and
// read instruction free of bank conflicts (16-lane groups over 64 banks and
// 8-lane groups over 32) and makes each address a per-lane base plus a
// per-instruction constant (checked below).
template <int P>
struct XposeLayout;
template <>
struct XposeLayout<4> {
  static constexpr int RS = 41, E1 = 6, p3 = 2, cells = 695;
};
template <>
struct XposeLayout<8> {
  static constexpr int RS = 72, E1 = 0, p3 = 1, cells = 575;
};
template <int P>
__host__ __device__ constexpr int xpose_cell(int r, int c) {
  return r * XposeLayout<P>::RS + (r >> 1) * XposeLayout<P>::E1 + c + (c >> 3) * XposeLayout<P>::p3;
}
// chunk written from register pair j (strided) and read into pair k (contiguous)
template <int P>
__host__ __device__ constexpr int xpose_wchunk(int lp, int j) {
  return strided_coord<P>(lp, j) >> 2;
}
__host__ __device__ constexpr int xpose_rchunk(int lp, int k) { return (32 * lp + k) >> 2; }

template <int P>
constexpr bool xpose_layout_ok() {
  constexpr int R = 64 / P, C = 8 * P, N = XposeLayout<P>::cells;
  bool seen[N] = {};
  for (int r = 0; r < R; ++r)
    for (int c = 0; c < C; ++c) {
      const int x = xpose_cell<P>(r, c);
      if (x < 0 || x >= N || seen[x]) return false;
      seen[x] = true;
    }
  for (int r = 0; r < R; ++r)
    for (int lp = 0; lp < P; ++lp)
      for (int j = 0; j < 32; j += 2) {
        const int dw = xpose_cell<P>(r, xpose_wchunk<P>(lp, j)) - xpose_cell<P>(r, xpose_wchunk<P>(lp, 0));
        const int dr = xpose_cell<P>(r, xpose_rchunk(lp, j)) - xpose_cell<P>(r, xpose_rchunk(lp, 0));
        if (dw != xpose_cell<P>(0, xpose_wchunk<P>(0, j)) - xpose_cell<P>(0, xpose_wchunk<P>(0, 0)) ||
            dr != xpose_cell<P>(0, xpose_rchunk(0, j)) - xpose_cell<P>(0, xpose_rchunk(0, 0)))
          return false;
      }
  return true;
}
static_assert(xpose_layout_ok<4>() && xpose_layout_ok<8>(), "transpose layout");

// FWHT (unnormalized) of a row held in the strided layout, which it leaves in
// the contiguous one (register k of lane lp = coordinate 32 lp + k): the
// butterflies on the register bits, the transpose through the wave's LDS
// cells xb, whose first write and read cells are at byte offsets wb and rb
// for this lane, then the butterflies on bits [S, 5). The cells are private
// to the wave, whose LDS operations complete in order: a wave-scope fence
// only keeps the compiler from moving them.
template <int P>
__device__ __forceinline__ void fwht_strided(double (&v)[32], char* xb, int wb, int rb) {
  constexpr int S = enc_seg_bits<P>();
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        const double x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
    }
  }
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int j = 4 * m + 2 * hr;
      const int off = 16 * (xpose_cell<P>(0, xpose_wchunk<P>(0, j)) - xpose_cell<P>(0, xpose_wchunk<P>(0, 0)));
      *reinterpret_cast<double2*>(xb + wb + off) = make_double2(v[j], v[j + 1]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int k = 4 * m + 2 * hr;
      const int off = 16 * (xpose_cell<P>(0, xpose_rchunk(0, k)) - xpose_cell<P>(0, xpose_rchunk(0, 0)));
      const double2 t = *reinterpret_cast<const double2*>(xb + rb + off);
      v[k] = t.x;
      v[k + 1] = t.y;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int h = 1 << S; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        const double x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
    }
  }
}

// Code lookup of k_encode (3- and 4-bit codes): with S = kCodeLutScale and
// OFF = kCodeLutOff, bucket b covers z = u / n in [(b - OFF) / S,
// (b + 1 - OFF) / S), the first one extended down to -inf and the last one up
// to +inf; the host admits only codebooks whose thresholds are more than 1/S
// apart and inside the inner buckets. Entry b is the double S t + OFF of the
// one threshold t inside the bucket (2^60 when there is none), with its low
// BITS mantissa bits replaced by the number of thresholds at or below the
// bucket's lower edge. The code is that number plus (S z + OFF >= entry): the
// replaced bits move the threshold by less than 2^-46 in z, and the rounding
// of S z + OFF is below 2^-50, both far inside the decision band. The 32
// entries of a table lie in distinct LDS banks, so its reads never conflict.

// Packs the low BITS bits of each of 32 codes LSB-first into BITS dwords
// with one funnel shift per code (two for a code that straddles dwords):
// bits above BITS in a code are ignored.
template <int BITS>
__device__ __forceinline__ void pack_codes_funnel(const uint32_t (&code)[32], uint32_t (&w)[BITS]) {
#pragma unroll
  for (int k = 0; k < BITS; ++k) {
    const int hi = 32 * k + 32;
    const int i0 = 32 * k / BITS, i1 = (hi - 1) / BITS;
    uint32_t x = 0u;
#pragma unroll
    for (int i = i0; i <= i1; ++i)
      x = __builtin_amdgcn_alignbit(code[i], x, uint32_t(i == i1 ? hi - BITS * i : BITS));
    w[k] = x;
  }
}

// Codes of 32 rotated coordinates u through a code lookup table lut (3- and
// 4-bit codes, above): z = u / n enters scaled by rns = kCodeLutScale / n (0
// for a zero row, which gets z = 0, the middle code L/2; a row with an
// infinite or NaN element gets unspecified codes). The low BITS bits of
// each result are the code; the bits above are not.
__device__ __forceinline__ void lookup_codes(const double (&u)[32], double rns, const double* lut,
                                             uint32_t (&code)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double z = fma(u[i], rns, double(kCodeLutOff));
    const double e = lut[min(max(int(z), 0), kCodeLutBuckets - 1)];
    code[i] = uint32_t(__double_as_longlong(e)) + (z >= e ? 1u : 0u);
  }
}

// Codes of 32 rotated coordinates u of a row of norm n by comparison. The
// code of z = u / n is #{k : z >= t_k}; with the antisymmetric codebook
// (t_{L/2-1} = 0, t_k = -t_{L-2-k}) it is L/2 + #{j : |u| >= n t_{L/2+j}}
// for u >= 0 and L/2 - 1 - #{j : |u| >= n t_{L/2+j}} for u < 0 (exact ties
// aside), which needs neither a division nor the negative half of the
// thresholds. A zero row gets the middle code L/2.
template <int BITS, int TS>
__device__ __forceinline__ void direct_codes(const EncodeArgs& a, const double (&u)[32], double n,
                                             uint32_t (&code)[32]) {
  constexpr int H = 1 << (BITS - 1);
  double T[H - 1];
#pragma unroll
  for (int j = 0; j < H - 1; ++j) T[j] = n > 0.0 ? a.tpos[TS][j] * n : INFINITY;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double au = fabs(u[i]);
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < H - 1; ++j) c += (au >= T[j]) ? 1u : 0u;
    code[i] = u[i] >= 0.0 ? uint32_t(H) + c : uint32_t(H - 1) - c;
  }
}

// Stores one row of tensor TS (0 = K, 1 = V) held on P = D/32 lanes: its norm
// n, its codes (low BITS bits of code[i] for the lane's coordinate i, packed
// LSB-first), and with QJL the sign sketch of the residual of the rotated
// coordinates u. Lanes of rows past the end (valid = false) compute but store
// nothing.
template <int D, int BITS, bool QJL, int TS, int IW>
__device__ __forceinline__ void store_encoded_row(const EncodeArgs& a, int bh, int64_t t,
                                                  bool valid, const EncodeLane<IW>& el,
                                                  const double (&u)[32], double n,
                                                  const uint32_t (&code)[32],
                                                  const double* cen = nullptr) {
  constexpr int P = D / 32;
  constexpr int E = 32;
  constexpr int L = 1 << BITS;
  constexpr int REC = D * BITS / 8;          // bytes per packed row
  constexpr int LW = BITS;                    // dwords of the row per lane (32 codes)
  const int lp = el.lp;
  const int64_t rec = int64_t(bh) * a.capacity + a.offset + t;

  double nstored;
  if (a.norm_f16) {
    const uint16_t h = dev::f64_to_f16_bits(n);
    nstored = dev::f16_bits_to_f64(h);
    if (valid && lp == 0) static_cast<uint16_t*>(a.norms[TS])[rec] = h;
  } else {
    const float nf = float(n);
    nstored = nf;
    if (valid && lp == 0) static_cast<float*>(a.norms[TS])[rec] = nf;
  }

  uint32_t w[LW];
  pack_codes_funnel<BITS>(code, w);
  if (valid) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes[TS] + rec * REC + lp * (4 * LW));
#pragma unroll
    for (int k = 0; k < LW; ++k) dst[k] = w[k];
  }

  if constexpr (QJL) {
    // residual in the rotated frame: r = (u - n_stored * c[code]) / sqrt(d)
    const double inv_sqrt_d = 1.0 / sqrt(double(D));
    double r[E];
    double rr = 0.0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      // the key centroid of the code: from the LDS copy cen when given,
      // else through a select chain over the kernel arguments
      const uint32_t ck = code[i] & uint32_t(L - 1);
      double ci = 0.0;
      if (cen) {
        ci = cen[ck];
      } else {
#pragma unroll
        for (int k = 0; k < L; ++k) ci = (ck == uint32_t(k)) ? a.cen_k[k] : ci;
      }
      const double ri = (u[i] - nstored * ci) * inv_sqrt_d;
      rr += ri * ri;
      r[i] = (el.qmask >> i & 1) ? -ri : ri;
    }
    rr = group_sum_f64<P>(rr);
    fwht32xP<P>(r, el.sg);
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) bits |= (r[i] < 0.0 ? 1u : 0u) << i;
    if (valid) {
      reinterpret_cast<uint32_t*>(a.qbits + rec * (D / 8))[lp] = bits;
      if (lp == 0) a.rnorm[rec] = dev::f64_to_f16_bits(sqrt(rr));
    }
  }
}

// One row of the decode kernels' appends, in the contiguous layout, from its
// sign-flipped coordinates u and the lane's share ss of its sum of squares:
// FWHT, norm, codes by comparison, stores.
template <int D, int BITS, bool QJL, int TS, int IW>
__device__ __forceinline__ void encode_row(const EncodeArgs& a, int bh, int64_t t, bool valid,
                                           const EncodeLane<IW>& el, double (&u)[32], double ss) {
  const double n = sqrt(group_sum_f64<D / 32>(ss));
  fwht32xP<D / 32>(u, el.sg);
  uint32_t code[32];
  direct_codes<BITS, TS>(a, u, n, code);
  store_encoded_row<D, BITS, QJL, TS, IW>(a, bh, t, valid, el, u, n, code);
}

// The lane's constants. SP = P selects the sign masks of k_encode's strided
// layout of P lanes per row, SP = 0 those of the contiguous one; the QJL
// signs are always contiguous (the residual is rotated after the FWHT).
template <int IW, bool QJL, int SP = 0>
__device__ __forceinline__ EncodeLane<IW> make_encode_lane(const EncodeArgs& a, int lp) {
  EncodeLane<IW> el;
  el.lp = lp;
  if constexpr (SP > 0) {
    constexpr int S = enc_seg_bits<SP>();
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j)
      m |= (a.sbits[j >> S] >> ((lp << S) | (j & ((1 << S) - 1))) & 1u) << j;
    el.smask = m;
  } else {
    el.smask = pick8(a.sbits, lp);
  }
  el.qmask = QJL ? pick8(a.qsbits, lp) : 0u;
  if constexpr (IW == 2) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      el.pm[j] = ((el.smask >> (2 * j) & 1u) << 15) | ((el.smask >> (2 * j + 1) & 1u) << 31);
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) el.sg[s] = (lp >> s & 1) ? -1.0 : 1.0;
  return el;
}

// Encodes token 0 of the (single-token) append in `e` for row bh: lanes
// [0, D/32) the key, lanes [D/32, D/16) the value (no QJL).
template <int D, int BK, int BV, int DT>
__device__ __forceinline__ void encode_append_row(const EncodeArgs& e, int bh, int lane) {
  constexpr int IW = DT == 0 ? 4 : 2;
  constexpr int P = D / 32;
  const int z = lane / P;
  const EncodeLane<IW> el = make_encode_lane<IW, false>(e, lane % P);
  RowWords<IW> rw;
  load_words<D, IW>(e, z, bh, 0, el.lp, rw);
  double u[32];
  const double ss = words_to_f64<DT>(rw, el, u);
  if (z == 0)
    encode_row<D, BK, false, 0, IW>(e, bh, 0, true, el, u, ss);
  else
    encode_row<D, BV, false, 1, IW>(e, bh, 0, true, el, u, ss);
}

// Fills the code lookup tables (above) of the 3- and 4-bit tensors among K
// (BK bits) and V (BV bits), in that order, with threads tid = 0, nthr, ...
template <int BK, int BV>
__device__ __forceinline__ void fill_code_luts(const EncodeArgs& a, double (*lut)[kCodeLutBuckets],
                                               int tid, int nthr) {
  constexpr bool LK = BK == 3 || BK == 4, LV = BV == 3 || BV == 4;
  constexpr int OFF = kCodeLutOff, NB = kCodeLutBuckets;
  for (int i = tid; i < ((LK ? 1 : 0) + (LV ? 1 : 0)) * NB; i += nthr) {
    const int tab = i / NB, bkt = i % NB;
    const int ts = LK && tab == 0 ? 0 : 1;
    const int bits = ts == 0 ? BK : BV;
    const double lo = double(bkt - OFF) / kCodeLutScale, hi = double(bkt + 1 - OFF) / kCodeLutScale;
    uint32_t c0 = 0;
    double tb = 0x1p60;
    // the L - 1 thresholds: 0 and +-t_{L/2+j}
    for (int j = -1; j < (1 << (bits - 1)) - 1; ++j) {
      for (int sgn = 0; sgn < (j < 0 ? 1 : 2); ++sgn) {
        const double tj = j < 0 ? 0.0 : (sgn ? -a.tpos[ts][j] : a.tpos[ts][j]);
        if (tj <= lo) ++c0;
        else if (tj < hi) tb = kCodeLutScale * tj + OFF;
      }
    }
    const uint64_t mask = (uint64_t(1) << bits) - 1;
    lut[tab][bkt] =
        __longlong_as_double(int64_t((uint64_t(__double_as_longlong(tb)) & ~mask) | c0));
  }
}

// Encodes rows [t0, t0 + n) of the appended tokens in `e`, K and V, for row
// bh: work items of 64/P rows (one wave each, as in k_encode) taken in turn
// by the nwaves waves of the workgroup, in the contiguous layout (DPP
// cross-lane stages, codes by comparison: with few items per wave, a code
// table's fill, barrier and LDS latency would cost more than they save).
template <int D, int BK, int BV, int DT>
__device__ __forceinline__ void encode_chunk_rows(const EncodeArgs& e, int bh, int64_t t0,
                                                  int64_t n, int wave, int nwaves, int lane) {
  constexpr int IW = DT == 0 ? 4 : 2;
  constexpr int P = D / 32;
  constexpr int RPW = 64 / P;
  const int groups = int((n + RPW - 1) / RPW);
  if (groups <= 0) return;
  const EncodeLane<IW> el = make_encode_lane<IW, false>(e, lane & (P - 1));
  const int rl = lane / P;
  for (int it = wave; it < 2 * groups; it += nwaves) {
    const int z = it >= groups ? 1 : 0;
    const int64_t r = int64_t(it - z * groups) * RPW + rl;
    RowWords<IW> rw;
    load_words<D, IW>(e, z, bh, t0 + r, el.lp, rw);
    double u[32];
    const double ss = words_to_f64<DT>(rw, el, u);
    if (z == 0)
      encode_row<D, BK, false, 0, IW>(e, bh, t0 + r, r < n, el, u, ss);
    else
      encode_row<D, BV, false, 1, IW>(e, bh, t0 + r, r < n, el, u, ss);
  }
}

// Persistent encode of K and V: a work item is 64/P consecutive rows (one
// wave) of one (tensor, batch*KV head) pair, numbered
// (tensor * BH + bh) * groups + group. Each wave walks the items with the
// grid's wave count as stride and loads the next item's input while it
// encodes the current one. Rows are loaded in the strided layout and
// transposed through LDS in the middle of the FWHT; 3- and 4-bit codes come
// from the per-workgroup lookup tables.
template <int D, int BK, int BV, bool QJL, int DT>
__global__ void __launch_bounds__(256) k_encode(EncodeArgs a) {
  constexpr int IW = DT == 0 ? 4 : 2;        // input bytes per coordinate
  constexpr int P = D / 32;
  constexpr int RPW = 64 / P;                // rows per work item
  constexpr int WPB = 4;                     // waves per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const uint32_t groups = uint32_t((a.n_new + RPW - 1) / RPW);
  const uint32_t per_tensor = uint32_t(a.BH) * groups;
  const uint32_t items = 2 * per_tensor;
  const uint32_t nwave = gridDim.x * WPB;
  uint32_t item = blockIdx.x * WPB + uint32_t(wave);

  // code lookups of the 3- and 4-bit tensors (key, value), one per workgroup
  constexpr bool LK = BK == 3 || BK == 4, LV = BV == 3 || BV == 4;
  __shared__ double lut[(LK && LV) ? 2 : 1][kCodeLutBuckets];
  __shared__ double2 xpose[WPB][XposeLayout<P>::cells];
  // QJL: the key centroids for the residual, one LDS read per coordinate
  __shared__ double cen[QJL ? 16 : 1];
  if constexpr (LK || LV) fill_code_luts<BK, BV>(a, lut, threadIdx.x, blockDim.x);
  if constexpr (QJL) {
    if (threadIdx.x < 16) cen[threadIdx.x] = a.cen_k[threadIdx.x];
  }
  if constexpr (LK || LV || QJL) __syncthreads();
  if (item >= items) return;

  const int lp = lane & (P - 1), rl = lane / P;
  const EncodeLane<IW> el = make_encode_lane<IW, QJL, P>(a, lp);
  char* xb = reinterpret_cast<char*>(&xpose[wave][0]);
  const int wb = 16 * xpose_cell<P>(rl, xpose_wchunk<P>(lp, 0));
  const int rb = 16 * xpose_cell<P>(rl, xpose_rchunk(lp, 0));

  struct Where { int z, bh; int64_t t; };
  auto where = [&](uint32_t it) {
    Where w;
    w.z = it >= per_tensor ? 1 : 0;
    const uint32_t rem = it - (w.z ? per_tensor : 0u);
    w.bh = int(rem / groups);
    w.t = int64_t(rem - uint32_t(w.bh) * groups) * RPW + rl;
    return w;
  };
  auto fetch = [&](uint32_t it, RowWords<IW>& rw) {
    const uint32_t c = it < items ? it : items - 1;    // past the last item: reload it
    const Where w = where(c);
    load_words_strided<D, IW>(a, w.z, w.bh, w.t, lp, rw);
  };

  // one input buffer: it is converted to doubles before the next item's
  // loads are issued into it
  RowWords<IW> rw;
  fetch(item, rw);
  for (;;) {
    double u[32];
    const double ss = words_to_f64<DT>(rw, el, u);
    const Where w = where(item);
    item += nwave;
    fetch(item, rw);
    // the row norm and the lookup scale first: their latency overlaps the FWHT
    const double n = sqrt(group_sum_f64<P>(ss));
    const double rns = n > 0.0 ? double(kCodeLutScale) / n : 0.0;
    fwht_strided<P>(u, xb, wb, rb);
    const bool valid = w.t < a.n_new;
    uint32_t code[32];
    // with lookups for both tensors the codes are found before the branch,
    // in the same block as the FWHT, whose work then hides the LDS latency
    if constexpr (LK && LV) lookup_codes(u, rns, lut[w.z], code);
    if (w.z == 0) {
      if constexpr (LK && !LV) lookup_codes(u, rns, lut[0], code);
      if constexpr (!LK) direct_codes<BK, 0>(a, u, n, code);
      store_encoded_row<D, BK, QJL, 0, IW>(a, w.bh, w.t, valid, el, u, n, code,
                                           QJL ? cen : nullptr);
    } else {
      if constexpr (LV && !LK) lookup_codes(u, rns, lut[0], code);
      if constexpr (!LV) direct_codes<BV, 1>(a, u, n, code);
      store_encoded_row<D, BV, false, 1, IW>(a, w.bh, w.t, valid, el, u, n, code);
    }
    if (item >= items) break;
  }
}

// ---------------------------------------------------------------------------
// Standalone QJL sketch of fp32 residual rows.
// ---------------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(256) k_qjl(QjlArgs a) {
  constexpr int E = D / 16;
  const int l16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const uint32_t qmask = dev::sign_mask(a.qjl_seed, l16 * E, E);
  for (int64_t row = int64_t(blockIdx.x) * 16 + grp; row < a.rows;
       row += int64_t(gridDim.x) * 16) {
    float f[E];
    dev::load_row_part<E>(a.r, 0, row * D + l16 * E, f);
    double r[E];
    double rr = 0.0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const double x = f[i];
      rr += x * x;
      r[i] = (qmask >> i & 1) ? -x : x;
    }
    rr = dev::group16_sum(rr);
    dev::fwht16<E, double>(r, l16);
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < E; ++i) bits |= (r[i] < 0.0 ? 1u : 0u) << i;
    dev::store_bytes(reinterpret_cast<uint8_t*>(a.bits) + row * (D / 8) + l16 * (E / 8),
                     bits, E / 8);
    if (l16 == 0) a.rnorm[row] = dev::f64_to_f16_bits(sqrt(rr));
  }
}

// ---------------------------------------------------------------------------
// Query preparation: qp = mult * R q (mult = scale * log2 e), and for QJL
// qq = R_2 qp. The dense baseline only scales.
// ---------------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(256) k_qprep(QPrepArgs a) {
  constexpr int E = D / 16;
  const int l16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t row = int64_t(blockIdx.x) * 16 + grp;
  if (row >= a.heads) return;   // whole 16-lane groups exit together
  float v[E];
  dev::load_row_part<E>(a.q, a.q_dtype, row * D + l16 * E, v);
  if (a.rotate) {
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
#pragma unroll
    for (int i = 0; i < E; ++i) if (smask >> i & 1) v[i] = -v[i];
    dev::fwht16<E, float>(v, l16);
  }
  const float mult = a.rotate ? a.mult / sqrtf(float(D)) : a.mult;
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] *= mult;
  if (a.pairs) {
    // fp16 pairs (v_2m, v_2m+1), D/2 dwords per head, scaled by a power of
    // two 2^-e that puts the head's largest element near 2^10 (no fp16
    // overflow or subnormals); e follows the pairs of all heads as one int
    // per head (read by the decode kernel, which undoes it in fp32)
    float vmax = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) vmax = fmaxf(vmax, fabsf(v[i]));
    vmax = dev::group_max16(vmax);
    const int qe = vmax > 0.f ? ilogbf(vmax) - 10 : 0;
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint32_t*>(a.qp) + row * (D / 2) +
                                          l16 * (E / 2));
#pragma unroll
    for (int k = 0; k < E / 8; ++k)
      dst[k] = make_uint4(dev::pack_f16x2(ldexpf(v[8 * k], -qe), ldexpf(v[8 * k + 1], -qe)),
                          dev::pack_f16x2(ldexpf(v[8 * k + 2], -qe), ldexpf(v[8 * k + 3], -qe)),
                          dev::pack_f16x2(ldexpf(v[8 * k + 4], -qe), ldexpf(v[8 * k + 5], -qe)),
                          dev::pack_f16x2(ldexpf(v[8 * k + 6], -qe), ldexpf(v[8 * k + 7], -qe)));
    if (l16 == 0) reinterpret_cast<int*>(a.qp)[a.heads * (D / 2) + row] = qe;
  } else {
    float4* dst = reinterpret_cast<float4*>(a.qp + row * D + l16 * E);
#pragma unroll
    for (int k = 0; k < E / 4; ++k)
      dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
  if (a.qjl) {
    const uint32_t qmask = dev::bitmap_bits(a.qsbits, l16 * E, E);
#pragma unroll
    for (int i = 0; i < E; ++i) if (qmask >> i & 1) v[i] = -v[i];
    dev::fwht16<E, float>(v, l16);
    const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] *= nn;
    float4* dq = reinterpret_cast<float4*>(a.qq + row * D + l16 * E);
#pragma unroll
    for (int k = 0; k < E / 4; ++k)
      dq[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// ---------------------------------------------------------------------------
// Split-K decode over packed codes (BK, BV in {2,3,4}) or, with BK = BV = 16,
// over dense bf16 rows (the comparison baseline).
//
// One workgroup per (split, b, kv head, head chunk); W = D/32 waves, one
// tile = 64*W tokens.
//   K phase  : thread = token. Scores for the GK query heads of the chunk,
//              qp read as wave-uniform values (scalar loads).
//   softmax  : tile max per head across the workgroup, online rescale.
//   V phase  : wave w owns coordinates [32w, 32w+32); lane = token (the
//              tile's tokens are spread over the 64 lanes), accumulating
//              GK x 32 weighted values per lane.
//   epilogue : lane sums by transpose-reduce; write (max, sum, acc[D]) of
//              the split in the rotated frame.
// ---------------------------------------------------------------------------

template <int D, int BK, int BV, int GK, bool QJL>
__global__ void __launch_bounds__(D / 32 * 64)
k_decode(DecodeArgs a, const float* __restrict__ qp_all, const float* __restrict__ qq_all) {
  constexpr int W = D / 32;
  constexpr int T = W * 64;
  constexpr int CW = 32;
  constexpr bool DENSE = (BK == 16);
  constexpr int KREC = D * BK / 8;
  constexpr int VREC = D * BV / 8;
  constexpr int KCW = BK;                      // dwords per 32-coordinate key chunk
  constexpr int VW = CW * BV / 32;             // dwords per value slice

  __shared__ float lut_k[16 * 32];
  __shared__ float lut_v[16 * 32];
  __shared__ float pv[T * GK];
  __shared__ float red[W * GK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x;
  const int unit = blockIdx.y;                 // (b * Hkv + kvh) * chunks + chunk
  const int chunk = unit % a.chunks;
  const int bkv = unit / a.chunks;             // b * Hkv + kvh
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int h0 = kvh * a.G + chunk * GK;       // first query head of this chunk
  const int64_t head0 = int64_t(b) * a.Hq + h0;

  if constexpr (!DENSE) {
    for (int i = tid; i < 16 * 32; i += T) {
      lut_k[i] = a.cbk[i >> 5];
      lut_v[i] = a.cbv[i >> 5];
    }
  }

  const int64_t t_begin = int64_t(split) * a.tps;
  const int64_t t_end = min(a.n_ctx, t_begin + a.tps);
  const int64_t row0 = int64_t(bkv) * a.capacity;

  const float* qp_base = qp_all + head0 * D;
  const float* qq_base = QJL ? qq_all + head0 * D : qp_base;

  float m_run[GK], lpart[GK];
  float acc[GK][CW];
#pragma unroll
  for (int g = 0; g < GK; ++g) {
    m_run[g] = -INFINITY;
    lpart[g] = 0.f;
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[g][c] = 0.f;
  }
  __syncthreads();

  for (int64_t base = t_begin; base < t_end; base += T) {
    // The query rows are re-read every tile as wave-uniform (scalar) loads.
    // An empty asm makes the pointers opaque so the compiler cannot hoist
    // all G*D values into vector registers for the whole loop.
    const float* qpr = qp_base;
    const float* qqr = qq_base;
    asm volatile("" : "+s"(qpr));
    if constexpr (QJL) asm volatile("" : "+s"(qqr));
    const dev::const_f32_ptr qp = dev::as_const(qpr);
    const dev::const_f32_ptr qq = dev::as_const(qqr);
    // ---------------- K phase: one token per thread
    const int64_t j = base + tid;
    const bool valid = j < t_end;
    float s[GK];
#pragma unroll
    for (int g = 0; g < GK; ++g) s[g] = 0.f;
    float nv = 0.f;
    if (valid) {
      // 32 coordinates per chunk: BK dwords of codes (16 for dense bf16)
      const uint32_t* krow = reinterpret_cast<const uint32_t*>(a.kc + (row0 + j) * KREC);
#pragma unroll 1
      for (int ch = 0; ch < D / 32; ++ch) {
        uint32_t kw[KCW];
        const uint32_t* src = krow + ch * KCW;
        if constexpr (KCW % 4 == 0) {
#pragma unroll
          for (int k = 0; k < KCW / 4; ++k) {
            const uint4 q4 = reinterpret_cast<const uint4*>(src)[k];
            kw[4 * k] = q4.x; kw[4 * k + 1] = q4.y; kw[4 * k + 2] = q4.z; kw[4 * k + 3] = q4.w;
          }
        } else {
#pragma unroll
          for (int k = 0; k < KCW; ++k) kw[k] = src[k];
        }
        const dev::const_f32_ptr qc = qp + ch * 32;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          float c;
          if constexpr (DENSE) {
            c = dev::bf16_to_f32(dev::field<16>(kw, e));
          } else {
            c = lut_k[(dev::field<BK>(kw, e) << 5) | (lane & 31)];
          }
#pragma unroll
          for (int g = 0; g < GK; ++g) s[g] = fmaf(qc[g * D + e], c, s[g]);
        }
      }
      if constexpr (!DENSE) {
        const float knrm = a.norm_f16
            ? dev::f16_to_f32(static_cast<const uint16_t*>(a.kn)[row0 + j])
            : static_cast<const float*>(a.kn)[row0 + j];
        const float ks = knrm * a.inv_sqrt_d;
#pragma unroll
        for (int g = 0; g < GK; ++g) s[g] *= ks;
        nv = (a.norm_f16 ? dev::f16_to_f32(static_cast<const uint16_t*>(a.vn)[row0 + j])
                         : static_cast<const float*>(a.vn)[row0 + j]) * a.inv_sqrt_d;
      } else {
        nv = 1.f;
      }
      if constexpr (QJL) {
        uint32_t sw[D / 32];
        const uint4* qs = reinterpret_cast<const uint4*>(a.kq + (row0 + j) * (D / 32));
#pragma unroll
        for (int k = 0; k < D / 128; ++k) {
          const uint4 q4 = qs[k];
          sw[4 * k] = q4.x; sw[4 * k + 1] = q4.y; sw[4 * k + 2] = q4.z; sw[4 * k + 3] = q4.w;
        }
        float tq[GK];
#pragma unroll
        for (int g = 0; g < GK; ++g) tq[g] = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const bool neg = (sw[i >> 5] >> (i & 31)) & 1u;
#pragma unroll
          for (int g = 0; g < GK; ++g) tq[g] += neg ? -qq[g * D + i] : qq[g * D + i];
        }
        const float rho = dev::f16_to_f32(a.kr[row0 + j]) * a.qjl_c;
#pragma unroll
        for (int g = 0; g < GK; ++g) s[g] = fmaf(rho, tq[g], s[g]);
      }
    }

    // ---------------- online softmax over the tile
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      const float mx = dev::wave_max(valid ? s[g] : -INFINITY);
      if (lane == 0) red[wave * GK + g] = mx;
    }
    __syncthreads();
    float alpha[GK];
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      float tmax = red[g];
#pragma unroll
      for (int w = 1; w < W; ++w) tmax = fmaxf(tmax, red[w * GK + g]);
      const float m_new = fmaxf(m_run[g], tmax);
      alpha[g] = exp2f(m_run[g] - m_new);
      m_run[g] = m_new;
      const float p = valid ? exp2f(s[g] - m_new) : 0.f;
      lpart[g] = fmaf(lpart[g], alpha[g], p);
      pv[tid * GK + g] = p * nv;
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[g][c] *= alpha[g];
    }
    __syncthreads();

    // ---------------- V phase: wave owns 32 coordinates, lane = token
#pragma unroll 1
    for (int m = 0; m < T / 64; ++m) {
      const int tl = m * 64 + lane;
      const int64_t jj = base + tl;
      if (jj < t_end) {
        uint32_t vw[VW];
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            a.vc + (row0 + jj) * VREC + wave * (CW * BV / 8));
        if constexpr (VW % 4 == 0) {
#pragma unroll
          for (int k = 0; k < VW / 4; ++k) {
            const uint4 q4 = reinterpret_cast<const uint4*>(src)[k];
            vw[4 * k] = q4.x; vw[4 * k + 1] = q4.y; vw[4 * k + 2] = q4.z; vw[4 * k + 3] = q4.w;
          }
        } else {
#pragma unroll
          for (int k = 0; k < VW; ++k) vw[k] = src[k];
        }
        float p[GK];
#pragma unroll
        for (int g = 0; g < GK; ++g) p[g] = pv[tl * GK + g];
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          float val;
          if constexpr (DENSE) {
            val = dev::bf16_to_f32(dev::field<16>(vw, c));
          } else {
            val = lut_v[(dev::field<BV>(vw, c) << 5) | (lane & 31)];
          }
#pragma unroll
          for (int g = 0; g < GK; ++g) acc[g][c] = fmaf(p[g], val, acc[g][c]);
        }
      }
    }
    __syncthreads();
  }

  // ---------------- epilogue: write the split's partial results
#pragma unroll
  for (int g = 0; g < GK; ++g) {
    const float l = dev::wave_sum(lpart[g]);
    if (lane == 0) red[wave * GK + g] = l;
  }
  __syncthreads();
  if (tid < GK) {
    float l = 0.f;
    for (int w = 0; w < W; ++w) l += red[w * GK + tid];
    float* ml = a.ml + ((head0 + tid) * a.S + split) * 2;
    ml[0] = m_run[tid];
    ml[1] = l;
  }
  constexpr int NV = GK * CW;
  float flat[NV];
#pragma unroll
  for (int g = 0; g < GK; ++g)
#pragma unroll
    for (int c = 0; c < CW; ++c) flat[g * CW + c] = acc[g][c];
  dev::wave_transpose_reduce<NV>(flat, lane);
#pragma unroll
  for (int i = 0; i < dev::reduce_kept<NV>(); ++i) {
    bool writer;
    const int idx = dev::reduce_index<NV>(lane, i, &writer);
    if (writer) {
      const int g = idx / CW, c = idx % CW;
      a.acc[((head0 + g) * a.S + split) * D + wave * CW + c] = flat[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K decode over packed codes, pair tables and fp16 dot products.
//
// Same workgroup layout as k_decode. Differences:
//   * the rotated query arrives as fp16 pairs (q_2m, q_2m+1) in dwords; a key
//     pair index (two consecutive codes, 2*BK bits) selects an fp16 pair
//     (c[code_2m], c[code_2m+1]) from an LDS table replicated RK times across
//     banks, and one v_dot2c_f32_f16 per head adds both products into the
//     fp32 score;
//   * in the V phase a lane holds two tokens (t, t+64); the pair index
//     (code_t | code_{t+64} << BV) of one coordinate selects
//     (c[code_t], c[code_{t+64}]) and one dot2 with the fp16 weight pair
//     (p_t, p_{t+64}) adds both tokens' contributions to the fp32 sum;
//   * the running max is refreshed only when a tile's max exceeds it by more
//     than 8 (log2 units), so weights stay <= 2^8 and the accumulators are
//     rarely rescaled.
// ---------------------------------------------------------------------------

template <int D, int BK, bool QJL>
struct PkKeys {
  uint32_t kw[D * BK / 32];        // this thread's key row (K phase token)
  uint32_t kn, vn;                 // raw norm bits of that token
  uint32_t sw[QJL ? D / 32 : 1];   // QJL sign words
  uint32_t kr;                     // QJL residual norm (fp16 bits)
};

template <int BV, int NP>
struct PkVals {
  uint32_t X[NP][BV], Y[NP][BV];   // value slices of the V-phase token pairs
};

template <int D, int BK, int BV, int GK, bool QJL>
__global__ void __launch_bounds__(D / 32 * 64) __attribute__((amdgpu_waves_per_eu(2)))
k_decode_pk(DecodeArgs a, const uint32_t* __restrict__ qp2_all,
            const float* __restrict__ qq_all) {
  constexpr int W = D / 32;
  constexpr int T = W * 64;
  constexpr int CW = 32;
  constexpr int KREC = D * BK / 8;
  constexpr int VREC = D * BV / 8;
  constexpr int KW = D * BK / 32;              // dwords per key row
  constexpr int VW = BV;                       // dwords per 32 value coordinates
  constexpr int KE = 1 << (2 * BK);            // key pair-table entries
  constexpr int VE = 1 << (2 * BV);            // value pair-table entries
  // Key table: 32 copies of every entry, 128-byte entry stride, so that lane
  // l reads copy (l & 31) and the 32 lanes of a half-wave hit 32 banks.
  constexpr int KT_BYTES = KE * 128;
  // Value table: 256-byte entry stride, 64 copies; the address of entry e
  // for lane l is (e << 8) | 4l, which one v_perm_b32 assembles from the
  // entry byte. Without room for it (QJL), 128-byte stride and 32 copies.
  constexpr bool WIDE_V = !QJL && (KT_BYTES + VE * 256 <= 76 * 1024);
  constexpr int VSH = WIDE_V ? 8 : 7;
  constexpr int VT_BYTES = VE << VSH;
  constexpr int NP = T / 128;                  // token pairs per lane (V phase)
  constexpr float kRescale = 8.0f;
  using KTile = PkKeys<D, BK, QJL>;
  using VTile = PkVals<BV, NP>;

  __shared__ __attribute__((aligned(16))) uint8_t tabs[KT_BYTES + VT_BYTES];
  __shared__ uint32_t pv2[(T / 2) * GK];
  __shared__ float red[W * (GK + 1)];           // per-wave maxima: scores, then nv

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t rl4 = uint32_t(lane & 31) << 2;           // key-table copy
  const uint32_t vl4 = uint32_t(WIDE_V ? lane : (lane & 31)) << 2;
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int chunk = unit % a.chunks;
  const int bkv = unit / a.chunks;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int h0 = kvh * a.G + chunk * GK;
  const int64_t head0 = int64_t(b) * a.Hq + h0;

  for (int i = tid; i < KE * 32; i += T) {
    const int e = i >> 5;
    *reinterpret_cast<uint32_t*>(tabs + (e << 7) + ((i & 31) << 2)) =
        dev::pack_f16x2(a.cbk[e & ((1 << BK) - 1)], a.cbk[e >> BK]);
  }
  constexpr int VCOPIES = WIDE_V ? 64 : 32;
  for (int i = tid; i < VE * VCOPIES; i += T) {
    const int e = i / VCOPIES;
    *reinterpret_cast<uint32_t*>(tabs + KT_BYTES + (e << VSH) + ((i % VCOPIES) << 2)) =
        dev::pack_f16x2(a.cbv[e & ((1 << BV) - 1)], a.cbv[e >> BV]);
  }
  const uint8_t* vtab = tabs + KT_BYTES;

  const int64_t t_begin = int64_t(split) * a.tps;
  const int64_t t_end = min(a.n_ctx, t_begin + a.tps);
  const int64_t row0 = int64_t(bkv) * a.capacity;
  const float* qq_base = QJL ? qq_all + head0 * D : nullptr;
  const bool nf16 = a.norm_f16 != 0;
  // key scale per head with the query pairs' power of two undone (the
  // exponents follow the pairs of all B * Hq heads)
  float ksg[GK];
  {
    const int64_t heads_total = int64_t(gridDim.y / (a.Hkv * a.chunks)) * a.Hq;
    const int* qexp = reinterpret_cast<const int*>(qp2_all) + heads_total * (D / 2) + head0;
#pragma unroll
    for (int g = 0; g < GK; ++g) ksg[g] = ldexpf(a.kscale, qexp[g]);
  }
  // value weights p * nv go to fp16 with p <= 2^8; nv carries a
  // workgroup-uniform power of two 2^-vexp that keeps each tile's largest
  // value norm within [2^-6, 2^6] (moved only when a tile leaves that band)
  float vsc = a.vscale;
  int vexp = 0;

  // The GK x D/2 rotated query pairs stay in VGPRs for the whole split:
  // register r of lane l holds pair 16 r + (l & 15), so every 16-lane row
  // has all of them and the K phase broadcasts one per dot2.
  constexpr int NQR = GK * D / 32;
  uint32_t vq[NQR];
  {
    const uint32_t* qsrc = qp2_all + head0 * (D / 2) + (lane & 15);
#pragma unroll
    for (int r = 0; r < NQR; ++r) vq[r] = qsrc[16 * r];
  }

  // Global loads of one tile: key rows and norms (issued a tile ahead) ...
  auto load_keys = [&](int64_t base, KTile& t) {
    const int64_t j = base + tid;
    if (j < t_end) {
      const uint32_t* kr_ = reinterpret_cast<const uint32_t*>(a.kc + (row0 + j) * KREC);
      if constexpr (KW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < KW / 4; ++k) {
          const uint4 q4 = reinterpret_cast<const uint4*>(kr_)[k];
          t.kw[4 * k] = q4.x; t.kw[4 * k + 1] = q4.y; t.kw[4 * k + 2] = q4.z;
          t.kw[4 * k + 3] = q4.w;
        }
      } else {
#pragma unroll
        for (int k = 0; k < KW; ++k) t.kw[k] = kr_[k];
      }
      t.kn = nf16 ? uint32_t(static_cast<const uint16_t*>(a.kn)[row0 + j])
                  : static_cast<const uint32_t*>(a.kn)[row0 + j];
      t.vn = nf16 ? uint32_t(static_cast<const uint16_t*>(a.vn)[row0 + j])
                  : static_cast<const uint32_t*>(a.vn)[row0 + j];
      if constexpr (QJL) {
        const uint4* qs = reinterpret_cast<const uint4*>(a.kq + (row0 + j) * (D / 32));
#pragma unroll
        for (int k = 0; k < D / 128; ++k) {
          const uint4 q4 = qs[k];
          t.sw[4 * k] = q4.x; t.sw[4 * k + 1] = q4.y; t.sw[4 * k + 2] = q4.z;
          t.sw[4 * k + 3] = q4.w;
        }
        t.kr = a.kr[row0 + j];
      }
    }
  };
  // ... and value slices (issued at the start of their own tile, consumed
  // after the K phase).
  auto load_vals = [&](int64_t base, VTile& t) {
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      const int64_t jj = base + pr * 128 + lane;
      const uint32_t* sx = reinterpret_cast<const uint32_t*>(
          a.vc + (row0 + jj) * VREC + wave * (CW * BV / 8));
      const uint32_t* sy = sx + 64 * (VREC / 4);
      const bool hx = jj < t_end, hy = jj + 64 < t_end;
      if constexpr (VW % 4 == 0) {
        uint4 x4 = make_uint4(0u, 0u, 0u, 0u), y4 = x4;
        if (hx) x4 = reinterpret_cast<const uint4*>(sx)[0];
        if (hy) y4 = reinterpret_cast<const uint4*>(sy)[0];
        t.X[pr][0] = x4.x; t.X[pr][1] = x4.y; t.X[pr][2] = x4.z; t.X[pr][3] = x4.w;
        t.Y[pr][0] = y4.x; t.Y[pr][1] = y4.y; t.Y[pr][2] = y4.z; t.Y[pr][3] = y4.w;
      } else {
#pragma unroll
        for (int k = 0; k < VW; ++k) {
          t.X[pr][k] = hx ? sx[k] : 0u;
          t.Y[pr][k] = hy ? sy[k] : 0u;
        }
      }
    }
  };

  float m_run[GK], lpart[GK];
  float acc[GK][CW];
#pragma unroll
  for (int g = 0; g < GK; ++g) {
    m_run[g] = -INFINITY;
    lpart[g] = 0.f;
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[g][c] = 0.f;
  }

  // One tile of T tokens from registers `cur` (keys) and `vals`.
  auto process = [&](int64_t base, const KTile& cur, const VTile& vals) {
    const float* qqr = qq_base;
    if constexpr (QJL) asm volatile("" : "+s"(qqr));

    // ---------------- K phase: thread = token. Runs on every lane (EXEC
    // full for the DPP broadcasts); lanes past the end are masked below.
    const int64_t j = base + tid;
    const bool valid = j < t_end;
    float s[GK];
#pragma unroll
    for (int g = 0; g < GK; ++g) s[g] = 0.f;
    float nv = 0.f;
    {
#pragma unroll
      for (int ch = 0; ch < D / 32; ++ch) {
        uint32_t qg[GK];
#pragma unroll
        for (int g = 0; g < GK; ++g) qg[g] = vq[g * (D / 32) + ch];
        dev::static_for<0, 16>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          const uint32_t ka = dev::field_at<2 * BK, 7>(cur.kw, ch * 16 + m) | rl4;
          const uint32_t cp = *reinterpret_cast<const uint32_t*>(tabs + ka);
          dev::dot2_bcast<m, GK, m == 15>(s, qg, cp);
          if constexpr (m == 7) __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (valid) {
      const float knrm = nf16 ? dev::f16_to_f32(cur.kn) : __uint_as_float(cur.kn);
#pragma unroll
      for (int g = 0; g < GK; ++g) s[g] *= knrm * ksg[g];
      nv = (nf16 ? dev::f16_to_f32(cur.vn) : __uint_as_float(cur.vn)) * vsc;
      if constexpr (QJL) {
        const dev::const_f32_ptr qq = dev::as_const(qqr);
        float tq[GK];
#pragma unroll
        for (int g = 0; g < GK; ++g) tq[g] = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          const bool neg = (cur.sw[i >> 5] >> (i & 31)) & 1u;
#pragma unroll
          for (int g = 0; g < GK; ++g) tq[g] += neg ? -qq[g * D + i] : qq[g * D + i];
        }
        const float rho = dev::f16_to_f32(cur.kr) * a.qjl_c;
#pragma unroll
        for (int g = 0; g < GK; ++g) s[g] = fmaf(rho, tq[g], s[g]);
      }
    }

    // ---------------- online softmax, lazy rescale
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      const float mx = dev::dpp_wave_max(valid ? s[g] : -INFINITY);
      if (lane == 0) red[wave * GK + g] = mx;
    }
    {
      const float nvm = dev::dpp_wave_max(nv);
      if (lane == 0) red[W * GK + wave] = nvm;
    }
    __syncthreads();
    {
      float tnv = red[W * GK];
#pragma unroll
      for (int w = 1; w < W; ++w) tnv = fmaxf(tnv, red[W * GK + w]);
      if (tnv > 64.f || (tnv > 0.f && tnv < 0.015625f)) {   // uniform, rare
        const int sh = ilogbf(tnv) - 4;
        vsc = ldexpf(vsc, -sh);
        vexp += sh;
        nv = ldexpf(nv, -sh);
#pragma unroll
        for (int g = 0; g < GK; ++g)
#pragma unroll
          for (int c = 0; c < CW; ++c) acc[g][c] = ldexpf(acc[g][c], -sh);
      }
    }
    uint16_t* pv16 = reinterpret_cast<uint16_t*>(pv2);
    const int pslot = ((tid >> 7) * 64 + (tid & 63)) * GK;
    const int phalf = (tid >> 6) & 1;
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      float tmax = red[g];
#pragma unroll
      for (int w = 1; w < W; ++w) tmax = fmaxf(tmax, red[w * GK + g]);
      if (tmax > m_run[g] + kRescale) {          // uniform across the workgroup
        const float alpha = exp2f(m_run[g] - tmax);
        m_run[g] = tmax;
        lpart[g] *= alpha;
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[g][c] *= alpha;
      }
      const float p = valid ? exp2f(s[g] - m_run[g]) : 0.f;
      lpart[g] += p;
      pv16[(pslot + g) * 2 + phalf] = __builtin_bit_cast(uint16_t, _Float16(p * nv));
    }
    __syncthreads();

    // ---------------- V phase: wave owns 32 coordinates, lane = 2 tokens
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      if (base + pr * 128 + lane < t_end) {
        uint32_t p2[GK];
#pragma unroll
        for (int g = 0; g < GK; ++g) p2[g] = pv2[(pr * 64 + lane) * GK + g];
        if constexpr (BV == 4) {
          // byte b of lo/hi = (code of token t) | (code of token t+64) << 4
          // for coordinate 8k + 2b (lo) and 8k + 2b + 1 (hi)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t x = vals.X[pr][k], y = vals.Y[pr][k];
            const uint32_t lo = (x & 0x0F0F0F0Fu) | ((y << 4) & 0xF0F0F0F0u);
            const uint32_t hi = ((x >> 4) & 0x0F0F0F0Fu) | (y & 0xF0F0F0F0u);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t word = (e & 1) ? hi : lo;
              const int bsel = e >> 1;
              uint32_t va;
              if constexpr (WIDE_V) {
                va = __builtin_amdgcn_perm(word, vl4, 0x0C0C0000u | uint32_t(4 + bsel) << 8);
              } else {
                va = ((bsel * 8 >= 7 ? (word >> (bsel * 8 - 7)) : (word << 7)) & 0x7F80u) | vl4;
              }
              const uint32_t vp = *reinterpret_cast<const uint32_t*>(vtab + va);
              const int c = 8 * k + e;
#pragma unroll
              for (int g = 0; g < GK; ++g) acc[g][c] = dev::dot2(p2[g], vp, acc[g][c]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int c = 0; c < CW; ++c) {
            const uint32_t va = dev::field_at<BV, VSH>(vals.X[pr], c) |
                                dev::field_at<BV, VSH + BV>(vals.Y[pr], c) | vl4;
            const uint32_t vp = *reinterpret_cast<const uint32_t*>(vtab + va);
#pragma unroll
            for (int g = 0; g < GK; ++g) acc[g][c] = dev::dot2(p2[g], vp, acc[g][c]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };

  // d = 128: key rows are loaded one tile ahead into two alternating
  // register buffers; d = 256 has no register room for that and loads its
  // key rows at the tile start. Value slices always load at the tile start.
  __syncthreads();
  VTile vals;
  if constexpr (D == 128) {
    KTile ka, kb;
    load_keys(t_begin, ka);
    for (int64_t base = t_begin; base < t_end; base += 2 * T) {
      load_vals(base, vals);
      if (base + T < t_end) load_keys(base + T, kb);
      process(base, ka, vals);
      if (base + T >= t_end) break;
      load_vals(base + T, vals);
      if (base + 2 * T < t_end) load_keys(base + 2 * T, ka);
      process(base + T, kb, vals);
    }
  } else {
    KTile ka;
    for (int64_t base = t_begin; base < t_end; base += T) {
      load_keys(base, ka);
      load_vals(base, vals);
      process(base, ka, vals);
    }
  }

  // ---------------- epilogue: (max, sum) and R^T of the weighted sum
#pragma unroll
  for (int g = 0; g < GK; ++g) {
    const float l = dev::wave_sum(lpart[g]);
    if (lane == 0) red[wave * GK + g] = l;
  }
  constexpr int NV = GK * CW;
  float flat[NV];
#pragma unroll
  for (int g = 0; g < GK; ++g)
#pragma unroll
    for (int c = 0; c < CW; ++c) flat[g * CW + c] = acc[g][c];
  dev::wave_transpose_reduce<NV>(flat, lane);
  // pv2 (D*GK dwords) is free now: stage the partial rows [GK][D] there
  float* obuf = reinterpret_cast<float*>(pv2);
#pragma unroll
  for (int i = 0; i < dev::reduce_kept<NV>(); ++i) {
    bool writer;
    const int idx = dev::reduce_index<NV>(lane, i, &writer);
    if (writer) obuf[(idx / CW) * D + wave * CW + idx % CW] = ldexpf(flat[i], vexp);
  }
  __syncthreads();
  if (tid < GK) {
    float l = 0.f;
    for (int w = 0; w < W; ++w) l += red[w * GK + tid];
    float* ml = a.ml + ((head0 + tid) * a.S + split) * 2;
    ml[0] = m_run[tid];
    ml[1] = l;
  }
  if (tid < 16 * GK) {
    constexpr int E = D / 16;
    const int g = tid >> 4, l16 = tid & 15;
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = obuf[g * D + l16 * E + i];
    dev::fwht16<E, float>(v, l16);
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
    const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (smask >> i & 1) ? -v[i] * nn : v[i] * nn;
    float4* dst = reinterpret_cast<float4*>(a.acc + ((head0 + g) * a.S + split) * D + l16 * E);
#pragma unroll
    for (int k = 0; k < E / 4; ++k)
      dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// ---------------------------------------------------------------------------
// Split-K decode on the matrix cores, d = 128 or 256 with 2- or 4-bit values,
// with or without the QJL score correction. W waves per workgroup (one
// workgroup per compute unit), each with its own online-softmax pass over
// interleaved 64-token tiles, combined once at the end; the two
// contractions of a tile run as MFMAs on fp16 operands dequantized through
// the pair tables:
//   scores  S[g][t] = q_g . k_t with v_mfma_f32_4x4x4_16b_f16: 16 blocks of
//           4 tokens, so lane t supplies 4 coordinates of its own key (two
//           pair lookups) as the B operand and receives the GK scores of
//           token t. The query is the A operand, broadcast from one block
//           (CBSZ 4, ABID j mod 16): lane (block b, row m) keeps only the
//           quads j = b, b + 16, ... of head m.
//   values  O[g][c] += sum_t p[g][t] v_t[c] with v_mfma_f32_16x16x32_f16:
//           one byte of a token's value row codes 2 (4-bit) or 4 (2-bit)
//           consecutive coordinates and is looked up as an fp16 pair or
//           quad; the K dimension is (token slot, coordinate j within the
//           byte): 16 tokens x 2 or 8 tokens x 4. Lane (kq, column n)
//           supplies byte cb of its slice of each of its tokens (B), and row
//           g + 4 j of A holds head g's weights in element j only, so row
//           g + 4 j of C is head g at coordinate j of byte cb of column n's
//           slice: one accumulator per byte of the slice.
//   QJL     the sign dot sum_i q''_i sigma_i is a second chain of the same
//           4x4x4 blocks: B = the key's 4 signs of quad j as fp16 +-1 (one
//           8-byte lookup of a 16-entry table), A = the quad of R_2 q'.
// CHUNK: the instantiation for a chunked append (formats without QJL): each
// workgroup first encodes its split's share of the appended tokens (all 8
// waves, k_encode's row layout), then decodes its older tokens followed by
// those new ones; a separate instantiation so that the encode's registers
// do not weigh on the plain decode.
// ---------------------------------------------------------------------------

typedef _Float16 mx_h4 __attribute__((ext_vector_type(4)));
typedef _Float16 mx_h8 __attribute__((ext_vector_type(8)));
typedef float mx_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t mx_u2 __attribute__((ext_vector_type(2)));
typedef uint32_t mx_u4 __attribute__((ext_vector_type(4)));

template <int D, int BK, int BV, bool QJL>
struct MxTile {
  // value lookups per (token, lane column): one per byte of 2- or 4-bit codes
  // (a quad or a pair), one per pair of 3-bit codes
  static constexpr int SB = BV == 2 ? D / 64 : D / 32;
  // dwords of value bits kept per token: the column's bytes, or for 3-bit
  // codes (3 or 6 bytes at any byte offset) the aligned 8 bytes around them
  static constexpr int SW = BV == 3 ? 2 : (SB + 3) / 4;
  uint32_t kw[D * BK / 32];     // key row of the lane's token
  uint32_t kn, vn;              // its key and value norms (f16 or f32 bits)
  uint32_t vx[16][SW];          // value slices: token 16*(i/4) + 4*kq + i%4
  uint32_t sw[QJL ? D / 32 : 1];  // QJL sign bits of the key (bit set: negative)
  uint32_t kr;                  // QJL residual norm (f16 bits)
};

// tiles each wave loads ahead of the one it processes (1 or 2): two where
// three tile buffers still fit the register budget without spilling
constexpr int mx_prefetch(int d, int bk, int bv, bool qjl) {
  return d == 128 && bk < 4 && bv != 3 ? 2 + 0 * qjl : 1;
}

template <int D, int BK, int BV, int GK, bool QJL, bool NF16, bool CHUNK = false>
__global__ void __launch_bounds__(64 * mx_waves(D))
    __attribute__((amdgpu_waves_per_eu(mx_waves(D) / 4)))
k_decode_mx(DecodeArgs a) {
  static_assert(D == 128 || D == 256, "matrix-core decode: d 128 or 256");
  static_assert(BV >= 2 && BV <= 4, "matrix-core decode: 2- to 4-bit values");
  static_assert(GK == 1 || GK == 2 || GK == 4, "heads per workgroup");
  static_assert(!(CHUNK && QJL), "chunked append: formats without QJL");
  constexpr int W = mx_waves(D);
  constexpr int TW = 64;                       // tokens per wave tile
  constexpr int T = W * TW;                    // tokens per workgroup round
  constexpr int NT = 64 * W;
  constexpr int KREC = D * BK / 8;
  constexpr int VREC = D * BV / 8;
  constexpr int KW = D * BK / 32;
  constexpr int SB = MxTile<D, BK, BV, QJL>::SB;
  constexpr int KE = 1 << (2 * BK);
  constexpr int VE = 1 << (2 * BV);
  // 2-bit codes: one lookup per four codes (a byte indexes a table of fp16
  // quads: 256 entries, 32 copies of 8 B); wider codes: one lookup per two
  // codes (a table of fp16 pairs, 64 copies of 4 B: entry stride 256 B, so
  // that the 64 lanes of a lookup hit 64 different banks)
  constexpr bool KQ4 = BK == 2;
  constexpr bool VQ4 = BV == 2;
  constexpr bool V3 = BV == 3;                 // 3-bit values: pairs of 6-bit fields
  constexpr int KT_BYTES = KQ4 ? 256 * 256 : KE * 256;
  constexpr int VT_BYTES = VQ4 ? 256 * 256 : VE * 256;
  constexpr int NS = D / 4;                    // score steps per token
  constexpr int NQ = NS / 16;                  // query quads kept per lane
  constexpr int PX = GK * TW / 2;              // weight dwords per wave tile
  constexpr float kRescale = 8.0f;
  constexpr int ST_BYTES = QJL ? 16 * 512 : 0; // QJL sign quads: 64 copies of 8 B
  using Tile = MxTile<D, BK, BV, QJL>;
  static_assert(KW % 4 == 0, "key rows are whole 16-byte loads");
  static_assert(SB == 2 || SB == 4 || SB == 8, "value slice width");

  constexpr int SLAB_BYTES = W * GK * D * 4;   // per-wave partials, after the loop
  constexpr int TAB_BYTES = KT_BYTES + VT_BYTES + ST_BYTES;
  __shared__ __attribute__((aligned(16)))
  uint8_t tabs[TAB_BYTES > SLAB_BYTES ? TAB_BYTES : SLAB_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t pex[W][3][PX];
  __shared__ uint32_t qs[GK * (D / 2)];
  __shared__ uint32_t qs2[QJL ? GK * (D / 2) : 1];
  __shared__ float mlx[W][GK][2];
  __shared__ int vexp_w[W];                    // each wave's value exponent (below)
  __shared__ int qexp;                         // the query's power-of-two scale
  __shared__ bool last_arrival;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;                   // V phase: lane column / A row
  const int kq = lane >> 4;                    // V phase: token quad
  const uint32_t kl4 = uint32_t(lane) << 2;    // pair tables: the lane's copy
  // LDS table bases: keys at 0, values at VT_OFF, QJL signs at ST_OFF. The
  // part of a base at or above 64 KB rides in the lane's offset register
  // (byte 2 of a v_perm-built address, or bits a field never reaches), the
  // rest in the instruction's 16-bit offset, so that no address needs an
  // add of its own.
  constexpr uint32_t VT_OFF = KT_BYTES, ST_OFF = KT_BYTES + VT_BYTES;
  constexpr uint32_t VT_HI = VT_OFF & 0xFF0000u, VT_LO = VT_OFF & 0xFFFFu;
  constexpr uint32_t VSEL2 = (VT_HI ? 0x02u : 0x0Cu) << 16;   // byte 2 of a value address
  static_assert(VT_OFF < 0x1000000u && ST_OFF % 0x2000u == 0, "table bases");
  const uint32_t vl4 = (uint32_t(lane) << 2) | VT_HI;
  const uint32_t l8 = uint32_t(lane & 31) << 3;   // quad tables: the lane's copy
  const uint32_t vl8 = l8 | VT_HI;
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int chunk = unit % a.chunks;
  const int bkv = unit / a.chunks;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int h0 = kvh * a.G + chunk * GK;
  const int64_t head0 = int64_t(b) * a.Hq + h0;

  // The split's tokens as positions [0, t_end): its old tokens [0, vlo)
  // are cache rows obeg + v; with a chunked append (append == 2) its new
  // tokens follow from the next 64-token boundary vpad, as rows
  // nbeg + v - vpad (no wave tile holds both).
  int64_t obeg, vlo, vpad, nbeg, t_end;
  if (CHUNK) {
    obeg = int64_t(split) * a.tpo;
    vlo = max(int64_t(0), min(a.tpo, a.n_old - obeg));
    vpad = (vlo + TW - 1) / TW * TW;
    nbeg = a.n_old + int64_t(split) * a.tpn;
    t_end = vpad + max(int64_t(0), min(a.tpn, a.n_ctx - nbeg));
  } else {
    obeg = int64_t(split) * a.tps;
    vlo = max(int64_t(0), min(a.n_ctx, obeg + a.tps) - obeg);
    vpad = vlo;
    nbeg = 0;
    t_end = vlo;
  }
  const int64_t t_begin = 0;
  const int64_t row0 = int64_t(bkv) * a.capacity;
  constexpr int nb = NF16 ? 2 : 4;
  const int iters = int((t_end - t_begin + T - 1) / T);

  // the end of the range the wave tile at position `base` belongs to, and
  // the cache row of that position (base is wave-uniform)
  auto vend = [&](int64_t base) -> int64_t {
    if constexpr (CHUNK) return base < vpad ? vlo : t_end;
    return t_end;
  };
  auto phys = [&](int64_t base) -> int64_t {
    if constexpr (CHUNK) return base < vpad ? obeg + base : nbeg + (base - vpad);
    return obeg + base;
  };
  auto rows_left = [&](int64_t base) -> uint32_t {
    const int64_t n = vend(base) - base;
    return uint32_t(n <= 0 ? 0 : (n < TW ? n : TW));
  };
  // chunked append: every workgroup first encodes its split's new rows
  // (rows nbeg .. of the cache, t_end - vpad of them) with all its waves,
  // before anything else is live. Only its own waves read them, so the
  // workgroup-scope release and acquire of the barrier after the tables make
  // the stores visible to their loads (no device-wide fence, which would
  // write back and invalidate the L2). Other head chunks of the same KV head
  // write the same bytes.
  if constexpr (CHUNK) {
    const int64_t t0 = nbeg - a.n_old, n = t_end - vpad;
    if (a.enc.in_dtype == 0)
      encode_chunk_rows<D, BK, BV, 0>(a.enc, bkv, t0, n, wave, W, lane);
    else if (a.enc.in_dtype == 1)
      encode_chunk_rows<D, BK, BV, 1>(a.enc, bkv, t0, n, wave, W, lane);
    else
      encode_chunk_rows<D, BK, BV, 2>(a.enc, bkv, t0, n, wave, W, lane);
  }
  const uint32_t ko0 = uint32_t(lane) * KREC;
  const uint32_t no0 = uint32_t(lane) * nb;
  // value slice i of a lane is token 16 (i / 4) + 4 (i % 4) + kq, so one load
  // instruction covers four consecutive rows (whole cache lines) and the
  // value, norm and sign-plane loads can stream past the caches (nontemporal)
  // 3-bit values: the column's 3 D / 128 bytes start at byte vby of the row;
  // the lane loads the dword-aligned 8 bytes from vby & ~3 and shifts them
  // down by vsh bits
  const uint32_t vby = uint32_t(col) * (3 * D / 128);
  const uint32_t vsh = (vby & 3u) * 8u;
  const uint32_t vo0 = uint32_t(kq) * VREC + (V3 ? (vby & ~3u) : uint32_t(col) * SB);
  constexpr int kNT = 2;                       // cache policy: nontemporal
  // overlapping windows of 48-byte rows are not whole lines: normal policy
  constexpr int kValNT = V3 ? 0 : kNT;
  constexpr int kSignNT = D / 8 == 16 ? kNT : 0;   // sign rows of 16 B: whole lines
  auto load = [&](int64_t vbase, Tile& t) {
    const uint32_t n = rows_left(vbase);
    const int64_t base = phys(vbase);
    const auto rk = dev::buffer_rsrc(a.kc + (row0 + base) * KREC, n * KREC);
#pragma unroll
    for (int k = 0; k < KW / 4; ++k) {
      const auto q4 = __builtin_amdgcn_raw_buffer_load_b128(rk, ko0, 16 * k, 0);
      t.kw[4 * k] = q4[0]; t.kw[4 * k + 1] = q4[1]; t.kw[4 * k + 2] = q4[2];
      t.kw[4 * k + 3] = q4[3];
    }
    const uint8_t* kn_p = static_cast<const uint8_t*>(a.kn) + (row0 + base) * nb;
    const uint8_t* vn_p = static_cast<const uint8_t*>(a.vn) + (row0 + base) * nb;
    if constexpr (NF16) {
      t.kn = __builtin_amdgcn_raw_buffer_load_b16(dev::buffer_rsrc(kn_p, n * nb), no0, 0, kNT);
      t.vn = __builtin_amdgcn_raw_buffer_load_b16(dev::buffer_rsrc(vn_p, n * nb), no0, 0, kNT);
    } else {
      t.kn = __builtin_amdgcn_raw_buffer_load_b32(dev::buffer_rsrc(kn_p, n * nb), no0, 0, kNT);
      t.vn = __builtin_amdgcn_raw_buffer_load_b32(dev::buffer_rsrc(vn_p, n * nb), no0, 0, kNT);
    }
    if constexpr (QJL) {
      const auto rs = dev::buffer_rsrc(reinterpret_cast<const uint8_t*>(a.kq) +
                                           (row0 + base) * (D / 8), n * (D / 8));
#pragma unroll
      for (int k = 0; k < D / 128; ++k) {
        const auto q4 = __builtin_amdgcn_raw_buffer_load_b128(rs, uint32_t(lane) * (D / 8),
                                                              16 * k, kSignNT);
        t.sw[4 * k] = q4[0]; t.sw[4 * k + 1] = q4[1]; t.sw[4 * k + 2] = q4[2];
        t.sw[4 * k + 3] = q4[3];
      }
      t.kr = __builtin_amdgcn_raw_buffer_load_b16(
          dev::buffer_rsrc(a.kr + (row0 + base), n * 2), uint32_t(lane) * 2, 0, kNT);
    }
    const auto rv = dev::buffer_rsrc(a.vc + (row0 + base) * VREC, n * VREC);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int so = (16 * (i >> 2) + 4 * (i & 3)) * VREC;
      if constexpr (V3 || SB == 8) {
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rv, vo0, so, kValNT);
        t.vx[i][0] = v2[0];
        t.vx[i][Tile::SW - 1] = v2[1];
      } else if constexpr (SB == 4) {
        t.vx[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo0, so, kNT);
      } else {
        t.vx[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rv, vo0, so, kNT);
      }
    }
  };


  // The query rows of this workgroup's heads are loaded, rotated and scaled
  // by wave 0 before it requests any tile: a query load queued behind the
  // whole chip's first round of tile traffic would arrive only after it. The
  // other waves request their first tiles at once, so the stream starts
  // while the query and the tables are set up. With a fused append this
  // needs the first tiles to hold old rows only: the appended rows are the
  // last ones of their split, past position vlo - 1 (chunk) or at vlo - 1
  // (single token), and the first tiles end before position (PF + 1) T.
  constexpr int QE = D / 16;                   // query elements per lane (16 lanes per head)
  if (tid < 16 * GK) {
    const int g = tid >> 4, l16 = tid & 15;
    float v[QE];
    {
      uint4 qraw[QE / 4];
      dev::load_row_raw<QE>(a.q_raw, a.q_dtype, (head0 + g) * D + l16 * QE, qraw);
      dev::convert_row_raw<QE>(qraw, a.q_dtype, v);
    }
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * QE, QE);
#pragma unroll
    for (int i = 0; i < QE; ++i) if (smask >> i & 1) v[i] = -v[i];
    dev::fwht16<QE, float>(v, l16);
    const float mult = a.qmult / sqrtf(float(D));
#pragma unroll
    for (int i = 0; i < QE; ++i) v[i] *= mult;
    float v2[QJL ? QE : 1];
    float vmax = 0.f;
#pragma unroll
    for (int i = 0; i < QE; ++i) vmax = fmaxf(vmax, fabsf(v[i]));
    if constexpr (QJL) {
      // q'' = R_2 q' from the fp32 q'
      const uint32_t qmask = dev::bitmap_bits(a.qsbits, l16 * QE, QE);
#pragma unroll
      for (int i = 0; i < QE; ++i) v2[i] = (qmask >> i & 1) ? -v[i] : v[i];
      dev::fwht16<QE, float>(v2, l16);
      const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
      for (int i = 0; i < QE; ++i) {
        v2[i] *= nn;
        vmax = fmaxf(vmax, fabsf(v2[i]));
      }
    }
    // one power of two for the GK rows (q' and q'') puts their largest
    // element near 2^10, so the fp16 operands neither overflow nor lose
    // small elements to subnormals; it is undone in fp32 with the key scale
    vmax = dev::group_max16(vmax);
    if constexpr (GK >= 2) vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
    if constexpr (GK >= 4) vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
    const int qe = vmax > 0.f ? ilogbf(vmax) - 10 : 0;
    if (tid == 0) qexp = qe;
#pragma unroll
    for (int i = 0; i < QE / 2; ++i)
      qs[g * (D / 2) + l16 * (QE / 2) + i] =
          dev::pack_f16x2(ldexpf(v[2 * i], -qe), ldexpf(v[2 * i + 1], -qe));
    if constexpr (QJL) {
#pragma unroll
      for (int i = 0; i < QE / 2; ++i)
        qs2[g * (D / 2) + l16 * (QE / 2) + i] =
            dev::pack_f16x2(ldexpf(v2[2 * i], -qe), ldexpf(v2[2 * i + 1], -qe));
    }
  }
  constexpr int PF = mx_prefetch(D, BK, BV, QJL);
  const int64_t wb = t_begin + int64_t(wave) * TW;
  const bool early = !a.append || int64_t(PF + 1) * T < vlo;
  // PF + 1 tile buffers, all requested before the set-up; in the loop a
  // buffer is refilled right after it has been processed
  Tile ta, tb, tc;
  auto load_first = [&]() {
    load(wb, ta);
    __builtin_amdgcn_sched_barrier(0);
    load(wb + T, tb);
    if constexpr (PF == 2) {
      __builtin_amdgcn_sched_barrier(0);
      load(wb + 2 * T, tc);
    }
  };
  if (early) load_first();

  // Lookup tables. Each wave writes whole entries with a wave-uniform high
  // code and compile-time low codes, from centroids loaded once (scalar
  // loads of the kernel arguments); one copy per lane.
  constexpr int LK = 1 << BK, LV = 1 << BV;
  float ck[LK], cv[LV];
#pragma unroll
  for (int j = 0; j < LK; ++j) ck[j] = a.cbk[j];
#pragma unroll
  for (int j = 0; j < LV; ++j) cv[j] = a.cbv[j];
  // quad entry e: codes e & 3, e >> 2 & 3, e >> 4 & 3, e >> 6; wave w writes
  // the 32 entries with e >> 5 == w (c0, c1 from the low bits, compile-time;
  // c2, c3 uniform); lane l writes dword l & 1 of copy l / 2
  auto quad_table = [&](uint8_t* base, const float (&c)[4], const float* cu) {
    static_assert(W == 8, "quad tables: 8 waves x 32 entries");
    const float c3 = cu[wave >> 1];
    const uint32_t hi0 = dev::pack_f16x2(cu[(2 * wave) & 3], c3);
    const uint32_t hi1 = dev::pack_f16x2(cu[(2 * wave + 1) & 3], c3);
    dev::static_for<0, 32>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      const uint32_t lo = dev::pack_f16x2(c[r & 3], c[(r >> 2) & 3]);
      *reinterpret_cast<uint32_t*>(base + ((32 * wave + r) << 8) + (lane << 2)) =
          (lane & 1) ? (r < 16 ? hi0 : hi1) : lo;
    });
  };
  // pair entry e = hi << B | lo: (c[lo], c[hi]); wave w writes the entries
  // with hi = w, w + 8; COPIES lanes write one copy each at stride SH bytes
  auto pair_table = [&](uint8_t* base, const auto& c, const float* cu, auto bits_c,
                        auto copies_c) {
    constexpr int B = decltype(bits_c)::value, COPIES = decltype(copies_c)::value;
    constexpr int L = 1 << B;
    constexpr int SH = COPIES == 64 ? 8 : 7;
#pragma unroll
    for (int hi0 = 0; hi0 < L; hi0 += W) {
      const int hi = hi0 + wave;
      if (hi < L) {
        const float ch = cu[hi];             // wave-uniform: a scalar load
        dev::static_for<0, L>([&](auto lc) {
          constexpr int lo = decltype(lc)::value;
          if (COPIES == 64 || lane < 32)
            *reinterpret_cast<uint32_t*>(base + (((hi << B) | lo) << SH) + (lane << 2)) =
                dev::pack_f16x2(c[lo], ch);
        });
      }
    }
  };
  if constexpr (KQ4) quad_table(tabs, ck, a.cbk);
  else pair_table(tabs, ck, a.cbk, std::integral_constant<int, BK>{},
                  std::integral_constant<int, 64>{});
  if constexpr (VQ4) quad_table(tabs + KT_BYTES, cv, a.cbv);
  else pair_table(tabs + KT_BYTES, cv, a.cbv, std::integral_constant<int, BV>{},
                  std::integral_constant<int, 64>{});
  static_assert(KE % W == 0 && VE % W == 0 && 256 % W == 0,
                "table entries split evenly over the waves");
  const uint8_t* vtab = tabs + VT_LO;          // value addresses carry VT_HI
  if constexpr (QJL) {
    // entry e: the fp16 pairs (s0, s1), (s2, s3) with s_k = -1 where bit k
    // of e is set, else +1; lane l reads copy l (entry stride 512 B)
    for (int i = tid; i < 16 * 64; i += NT) {
      const int e = i >> 6;
      const float s0 = (e & 1) ? -1.f : 1.f, s1 = (e & 2) ? -1.f : 1.f;
      const float s2 = (e & 4) ? -1.f : 1.f, s3 = (e & 8) ? -1.f : 1.f;
      *reinterpret_cast<uint2*>(tabs + KT_BYTES + VT_BYTES + (e << 9) + ((i & 63) << 3)) =
          make_uint2(dev::pack_f16x2(s0, s1), dev::pack_f16x2(s2, s3));
    }
  }
  // fused single-token append: the workgroup that owns the last split (the
  // one that reads token n_ctx - 1) encodes that token's K and V rows into
  // the cache first; the barrier below makes the stores visible to its
  // waves' loads. Other head chunks of the same KV head write the same bytes.
  // (Formats with the QJL sketch encode the token in a launch of its own.)
  if (!QJL && !CHUNK && a.append && split == a.S - 1 && wave == 0 && lane < D / 16) {
    if (a.enc.in_dtype == 0)
      encode_append_row<D, BK, BV, 0>(a.enc, bkv, lane);
    else if (a.enc.in_dtype == 1)
      encode_append_row<D, BK, BV, 1>(a.enc, bkv, lane);
    else
      encode_append_row<D, BK, BV, 2>(a.enc, bkv, lane);
  }
  __syncthreads();

  // query quads for the broadcast A operand: lane (block lane/4, row lane%4)
  // keeps coordinates 4j .. 4j+3 of head lane%4 for j = lane/4 + 16*i
  mx_u2 qa[NQ], qa2[QJL ? NQ : 1];
  {
    const int qm = lane & 3, qb = lane >> 2;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int j = qb + 16 * i;
      if (qm < GK) {
        qa[i] = mx_u2{qs[qm * (D / 2) + 2 * j], qs[qm * (D / 2) + 2 * j + 1]};
        if constexpr (QJL) qa2[i] = mx_u2{qs2[qm * (D / 2) + 2 * j], qs2[qm * (D / 2) + 2 * j + 1]};
      } else {
        qa[i][0] = 0u;
        qa[i][1] = 0u;
        if constexpr (QJL) qa2[i] = mx_u2{0u, 0u};
      }
    }
  }
  const uint32_t sl8 = (uint32_t(lane) << 3) | ST_OFF;   // QJL signs: copy and table base
  // Value product (see the kernel comment): the weight slot of this lane's
  // token in the product's K order. 4-bit values: token 16 G + 4 u + kq of
  // 16-token group G sits in slot 16 G + 4 kq + u; 2-bit values: token
  // 8 G + 4 u + kq of 8-token group G in slot 8 G + 2 kq + u.
  const int pslot = VQ4 ? (lane & 0x38) | ((lane & 3) << 1) | ((lane >> 2) & 1)
                        : (lane & 0x30) | ((lane & 3) << 2) | ((lane >> 2) & 3);
  // A-operand selectors: row col = g + 4 j of the product holds head g's
  // weights in half j of each pair (4-bit) or element j of each quad (2-bit)
  // of the K dimension; rows of heads >= GK (and rows >= 8 with 4-bit values)
  // are zero. v_perm selectors on the dword X = (p_slot0, p_slot1): 0x0C
  // gives a zero byte, 0x0100 / 0x0302 the low / high fp16 of X.
  uint32_t asel[4];
  {
    const int ga = col & 3, ja = col >> 2;
    const bool live = ga < GK && (VQ4 || ja < 2);
    constexpr uint32_t kZ = 0x0C0C0C0Cu;
    if constexpr (VQ4) {
      // dwords: (slot 0, j' 0-1), (slot 0, j' 2-3), (slot 1, j' 0-1), (slot 1, j' 2-3)
      const uint32_t lo = (ja & 1) ? 0x01000C0Cu : 0x0C0C0100u;
      const uint32_t hi = (ja & 1) ? 0x03020C0Cu : 0x0C0C0302u;
      asel[0] = live && ja < 2 ? lo : kZ;
      asel[1] = live && ja >= 2 ? lo : kZ;
      asel[2] = live && ja < 2 ? hi : kZ;
      asel[3] = live && ja >= 2 ? hi : kZ;
    } else {
      // dwords: slots 0 .. 3 of the group, weight in half ja
      const uint32_t lo = ja ? 0x01000C0Cu : 0x0C0C0100u;
      const uint32_t hi = ja ? 0x03020C0Cu : 0x0C0C0302u;
      asel[0] = live ? lo : kZ;
      asel[1] = live ? hi : kZ;
      asel[2] = asel[0];
      asel[3] = asel[1];
    }
  }
  const int arow_head = (col & 3) < GK ? (col & 3) : 0;

  float m_run[GK], lpart[GK];
  // key and QJL scales with the query's power of two undone (fp32)
  const float kscale = ldexpf(a.kscale, qexp);
  const float qjl_c = ldexpf(a.qjl_c, qexp);
  // The weights p * nv enter the value product as fp16, with p <= 2^8 (the
  // lazily raised max). nv carries a wave-uniform power of two 2^-vexp that
  // keeps the tile's value norms within [2^-6, 2^6]: only when a tile leaves
  // that band is it moved (and the accumulators with it), so large or tiny
  // value norms neither overflow fp16 nor fall into its subnormals.
  float vsc = a.vscale;                        // a.vscale * 2^-vexp
  int vexp = 0;
  mx_f4 acc[SB];                               // SB = value bytes per (token, column)
#pragma unroll
  for (int g = 0; g < GK; ++g) {
    m_run[g] = -INFINITY;
    lpart[g] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < SB; ++j) acc[j] = mx_f4{0.f, 0.f, 0.f, 0.f};

  // A tile goes through three steps: scores (key lookups and the score
  // products), softmax (running max, weights into LDS) and values (value
  // lookups and the value product). The loop below takes the values of tile
  // k together with the scores of tile k + 1, in one software pipeline: its
  // stage i is value step i and score steps 2i, 2i + 1 (there are D / 8
  // value steps and D / 4 score steps), and the lookups of stage i + 1 are
  // issued before the products of stage i, so that table reads stay in
  // flight while the products run.
  struct Scores {
    mx_f4 sk[2];
    mx_f4 sq[QJL ? 2 : 1];
  };
  struct KLook {
    mx_u2 kb;                                  // fp16 centroids of the step's coordinates
    mx_u2 sb;                                  // their QJL signs (+-1)
  };
  // score step j: coordinates 4j .. 4j + 3 of the lane's token
  auto k_issue = [&](auto jc, const Tile& cur) {
    constexpr int j = decltype(jc)::value;
    KLook l;
    if constexpr (KQ4) {
      // byte j of the row = the codes of coordinates 4j .. 4j + 3
      const uint32_t ka = __builtin_amdgcn_perm(cur.kw[j >> 2], l8,
                                                0x0C0C0000u | uint32_t(4 + (j & 3)) << 8);
      l.kb = *reinterpret_cast<const mx_u2*>(tabs + ka);
    } else {
      const uint32_t ka0 = dev::field_at<2 * BK, 8>(cur.kw, 2 * j) | kl4;
      const uint32_t ka1 = dev::field_at<2 * BK, 8>(cur.kw, 2 * j + 1) | kl4;
      l.kb[0] = *reinterpret_cast<const uint32_t*>(tabs + ka0);
      l.kb[1] = *reinterpret_cast<const uint32_t*>(tabs + ka1);
    }
    if constexpr (QJL) {
      const uint32_t sa = dev::field_at<4, 9>(cur.sw, j) | sl8;
      const uint2 sp = *reinterpret_cast<const uint2*>(tabs + sa);
      l.sb = mx_u2{sp.x, sp.y};
    }
    return l;
  };
  // scores: lane = token, 4 coordinates per MFMA, query block j % 16 broadcast
  auto k_take = [&](auto jc, const KLook& l, Scores& r) {
    constexpr int j = decltype(jc)::value;
    r.sk[j & 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(
        __builtin_bit_cast(mx_h4, qa[j / 16]), __builtin_bit_cast(mx_h4, l.kb), r.sk[j & 1], 4,
        j % 16, 0);
    if constexpr (QJL)
      r.sq[j & 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(
          __builtin_bit_cast(mx_h4, qa2[j / 16]), __builtin_bit_cast(mx_h4, l.sb), r.sq[j & 1], 4,
          j % 16, 0);
  };
  // Values: one 16x16x32 MFMA per (token group G, value byte cb of the
  // lane's slice); a token's byte holds the codes of two (4-bit) or four
  // (2-bit) consecutive coordinates, looked up as an fp16 pair or quad, and
  // the coordinate within the byte is the product's row half / quad element:
  // row g + 4 j of A carries head g's weights in element j only, so row
  // g + 4 j of C is head g at coordinate j of the byte. Column n = the lane's
  // slice of the rows. 4-bit values: 16-token groups, the lane's slots
  // 4 kq + u are tokens 16 G + 4 u + kq; 2-bit values: 8-token groups, slots
  // 2 kq + u are tokens 8 G + 4 u + kq. Value step i is (G, cb) = (i / SB,
  // i % SB).
  constexpr int NV = D / 8;
  constexpr int NG = VQ4 ? 8 : 4;
  static_assert(NV == NG * SB, "value steps");
  // 3-bit values: the token's bits of the column, shifted to bit 0 (24 or 48
  // bits), taken once per token when its group starts
  uint32_t xw[4][2];
  auto v_issue = [&](auto ic, const Tile& cur) {
    constexpr int i = decltype(ic)::value, G = i / SB, cb = i % SB;
    constexpr uint32_t sel = 0x0C000000u | VSEL2 | uint32_t(4 + (cb & 3)) << 8;
    mx_u4 vb;
    if constexpr (V3) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (cb == 0) {
          const uint32_t w0 = cur.vx[4 * G + u][0], w1 = cur.vx[4 * G + u][1];
          xw[u][0] = __builtin_amdgcn_alignbit(w1, w0, vsh);
          xw[u][1] = w1 >> vsh;
        }
        vb[u] = *reinterpret_cast<const uint32_t*>(vtab + (dev::bits_at<6, 8>(xw[u], 6 * cb) | vl4));
      }
    } else if constexpr (!VQ4) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        vb[u] = *reinterpret_cast<const uint32_t*>(
            vtab + __builtin_amdgcn_perm(cur.vx[4 * G + u][cb >> 2], vl4, sel));
    } else {
      constexpr int i0 = 4 * (G >> 1) + 2 * (G & 1);
      const mx_u2 q0 = *reinterpret_cast<const mx_u2*>(
          vtab + __builtin_amdgcn_perm(cur.vx[i0][cb >> 2], vl8, sel));
      const mx_u2 q1 = *reinterpret_cast<const mx_u2*>(
          vtab + __builtin_amdgcn_perm(cur.vx[i0 + 1][cb >> 2], vl8, sel));
      vb = mx_u4{q0[0], q0[1], q1[0], q1[1]};
    }
    return vb;
  };
  // the weights of group G as the A operand (v_perm into the head's rows)
  using WX = std::conditional_t<VQ4, uint32_t, mx_u2>;
  auto w_operand = [&](const WX& X) {
    mx_u4 aw;
    if constexpr (!VQ4)
      aw = mx_u4{__builtin_amdgcn_perm(X[0], X[0], asel[0]),
                 __builtin_amdgcn_perm(X[0], X[0], asel[1]),
                 __builtin_amdgcn_perm(X[1], X[1], asel[0]),
                 __builtin_amdgcn_perm(X[1], X[1], asel[1])};
    else
      aw = mx_u4{__builtin_amdgcn_perm(X, X, asel[0]), __builtin_amdgcn_perm(X, X, asel[1]),
                 __builtin_amdgcn_perm(X, X, asel[2]), __builtin_amdgcn_perm(X, X, asel[3])};
    return __builtin_bit_cast(mx_h8, aw);
  };
  // The pipeline: the values of the tile in vt with its weights in px (when
  // WV) and the scores of the tile in kt.
  auto pipeline = [&](auto wv_c, const uint32_t* px, const Tile& vt, const Tile& kt) {
    constexpr bool WV = decltype(wv_c)::value;
    Scores r;
    r.sk[0] = r.sk[1] = mx_f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (QJL) r.sq[0] = r.sq[1] = mx_f4{0.f, 0.f, 0.f, 0.f};
    WX X[WV ? NG : 1];
    if constexpr (WV) {
      const uint16_t* pr = reinterpret_cast<const uint16_t*>(px) + arow_head * TW +
                           (VQ4 ? 2 : 4) * kq;
#pragma unroll
      for (int G = 0; G < NG; ++G)
        X[G] = *reinterpret_cast<const WX*>(pr + (VQ4 ? 8 : 16) * G);
    }
    // stage i takes score steps 2i, 2i + 1
    static_assert(NS == 2 * NV, "two score steps per value step");
    KLook kl[2][2];
    mx_u4 vl[2];
    mx_h8 pa;
    auto k_stage = [&](auto sc, auto issue_c) {
      constexpr int st = decltype(sc)::value;
      constexpr int a0 = 2 * st, a1 = 2 * st + 2;
      dev::static_for<a0, a1>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (decltype(issue_c)::value)
          kl[st & 1][m - a0] = k_issue(std::integral_constant<int, m>{}, kt);
        else
          k_take(std::integral_constant<int, m>{}, kl[st & 1][m - a0], r);
      });
    };
    k_stage(std::integral_constant<int, 0>{}, std::true_type{});
    if constexpr (WV) vl[0] = v_issue(std::integral_constant<int, 0>{}, vt);
    dev::static_for<0, NV>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + 1 < NV) {
        k_stage(std::integral_constant<int, i + 1>{}, std::true_type{});
        if constexpr (WV) vl[(i + 1) & 1] = v_issue(std::integral_constant<int, i + 1>{}, vt);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (WV) {
        if constexpr (i % SB == 0) pa = w_operand(X[i / SB]);
        acc[i % SB] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            pa, __builtin_bit_cast(mx_h8, vl[i & 1]), acc[i % SB], 0, 0, 0);
      }
      k_stage(ic, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    });
    // computed here, not on the path past the loop exit that follows
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(r.sk[i]));
    if constexpr (QJL) {
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(r.sq[i]));
    }
    return r;
  };
  const std::true_type with_values{};
  const std::false_type scores_only{};

  auto softmax = [&](int64_t base, uint32_t* px, const Tile& cur, const Scores& sc) {
    const bool valid = base + lane < vend(base);
    const mx_f4 (&sk)[2] = sc.sk;
    const mx_f4 (&sq)[QJL ? 2 : 1] = sc.sq;
    const float knrm = NF16 ? dev::f16_to_f32(cur.kn) : __uint_as_float(cur.kn);
    const float vnrm = NF16 ? dev::f16_to_f32(cur.vn) : __uint_as_float(cur.vn);
    const float ks = knrm * kscale;
    float nv = vnrm * vsc;
    const float rho = QJL ? dev::f16_to_f32(cur.kr) * qjl_c : 0.f;
    {
      const bool high = __ballot(nv > 64.f) != 0;
      const bool low = __ballot(nv >= 0.015625f) == 0 && __ballot(nv > 0.f) != 0;
      if (high || low) {                      // wave-uniform, rare
        const int sh = ilogbf(dev::dpp_wave_max(nv)) - 4;
        vsc = ldexpf(vsc, -sh);
        vexp += sh;
        nv = ldexpf(nv, -sh);
#pragma unroll
        for (int j = 0; j < SB; ++j)
#pragma unroll
          for (int g = 0; g < GK; ++g) acc[j][g] = ldexpf(acc[j][g], -sh);
      }
    }

    // ---------------- online softmax with a lazily raised running max
    uint16_t* p16 = reinterpret_cast<uint16_t*>(px);
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      // t = score - running max, in one step; the branch rebuilds the score
      // itself (the running max starts at -inf)
      const float dk = sk[0][g] + sk[1][g];
      const float dq = QJL ? sq[0][g] + sq[1][g] : 0.f;
      float t = fmaf(dk, ks, -m_run[g]);
      if constexpr (QJL) t = fmaf(rho, dq, t);
      if (__ballot(valid && t > kRescale)) {              // wave-uniform, rare
        float s = dk * ks;
        if constexpr (QJL) s = fmaf(rho, dq, s);
        const float mx = dev::dpp_wave_max(valid ? s : -INFINITY);
        const float m_new = fmaxf(m_run[g], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
        m_run[g] = m_new;
        lpart[g] *= alpha;
#pragma unroll
        for (int j = 0; j < SB; ++j) acc[j][g] *= alpha;
        t = s - m_new;
      }
      // branch-free: rows past the split have zero norms and weight 0
      const float e = __builtin_amdgcn_exp2f(t);
      const float p = valid ? e : 0.f;
      lpart[g] += p;
      p16[g * TW + pslot] = __builtin_bit_cast(uint16_t, _Float16(p * nv));
    }
    // the weights written above are read back by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  {
    uint32_t* px0 = pex[wave][0];
    uint32_t* px1 = pex[wave][1];
    uint32_t* px2 = pex[wave][2];
    if (!early) load_first();
    __builtin_amdgcn_sched_barrier(0);
    // tile k is in buffer k mod (PF + 1) with its weights in slot k mod
    // (PF + 1); a buffer is refilled once its values have been taken
    softmax(wb, px0, ta, pipeline(scores_only, nullptr, ta, ta));
    if constexpr (PF == 1) {
      for (int it = 0; it < iters; it += 2) {
        const int64_t base = wb + int64_t(it) * T;
        Scores sc = pipeline(with_values, px0, ta, tb);
        if (it + 1 >= iters) break;
        load(base + 2 * T, ta);
        softmax(base + T, px1, tb, sc);
        sc = pipeline(with_values, px1, tb, ta);
        if (it + 2 >= iters) break;
        load(base + 3 * T, tb);
        softmax(base + 2 * T, px0, ta, sc);
      }
    } else {
      for (int it = 0; it < iters; it += 3) {
        const int64_t base = wb + int64_t(it) * T;
        Scores sc = pipeline(with_values, px0, ta, tb);
        if (it + 1 >= iters) break;
        load(base + 3 * T, ta);
        softmax(base + T, px1, tb, sc);
        sc = pipeline(with_values, px1, tb, tc);
        if (it + 2 >= iters) break;
        load(base + 4 * T, tb);
        softmax(base + 2 * T, px2, tc, sc);
        sc = pipeline(with_values, px2, tc, ta);
        if (it + 3 >= iters) break;
        load(base + 5 * T, tc);
        softmax(base + 3 * T, px0, ta, sc);
      }
    }
  }

  // ---------------- combine the waves of this split (rotated frame): each
  // wave leaves (max, sum) and its unscaled weighted sums in LDS, then every
  // thread rescales and adds the W waves' values of its coordinate
  float lw[GK];
#pragma unroll
  for (int g = 0; g < GK; ++g) lw[g] = dev::wave_sum(lpart[g]);
  __syncthreads();                       // tables are dead: reuse them below
  float* slab = reinterpret_cast<float*>(tabs);          // [W][GK][D]
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      mlx[wave][g][0] = m_run[g];
      mlx[wave][g][1] = lw[g];
    }
    vexp_w[wave] = vexp;
  }
  // C row g + 4 j of lane (col, kq = j) is head g at coordinate
  // (bits / 2 ... ) j of value byte cb of column col's slice
  constexpr int CPB = VQ4 ? 4 : 2;             // coordinates per value byte
  if (kq < CPB) {
#pragma unroll
    for (int g = 0; g < GK; ++g)
#pragma unroll
      for (int cb = 0; cb < SB; ++cb)
        slab[(wave * GK + g) * D + CPB * (SB * col + cb) + kq] = acc[cb][g];
  }
  __syncthreads();
  // This split's partial, (max, sum) per head and the weighted value sum in
  // the rotated frame, goes out with device-scope stores: they write through
  // this XCD's L2, so the workgroup that merges the unit (on any XCD) reads
  // them without an L2 write-back here.
  for (int i = tid; i < GK * D; i += NT) {
    const int g = i / D;
    float Mg = mlx[0][g][0];
#pragma unroll
    for (int w = 1; w < W; ++w) Mg = fmaxf(Mg, mlx[w][g][0]);
    float sum = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = mlx[w][g][0];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - Mg);
      sum = fmaf(slab[w * GK * D + i], ldexpf(f, vexp_w[w]), sum);
      l = fmaf(mlx[w][g][1], f, l);
    }
    dev::store_dev(a.acc + ((head0 + g) * a.S + split) * D + (i - g * D), sum);
    if (i - g * D == 0) dev::store_dev2(a.ml + ((head0 + g) * a.S + split) * 2, Mg, l);
  }
  // every store of this workgroup has completed before the arrival count
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    last_arrival = __hip_atomic_fetch_add(a.cnt + unit, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == uint32_t(a.S - 1);
  __syncthreads();
  if (!last_arrival) return;

  // ---------------- last split of the unit: merge the S partials of each
  // head (online log-sum-exp), then R^T, then the output. Thread (sg, item)
  // merges splits sg, sg + SG, ... of four coordinates (one 16-byte load per
  // split, device-scope so that no stale L2 line is read); the SG partial
  // merges of an item are then combined in split-group order through LDS.
  constexpr int ITEMS = GK * D / 4;
  constexpr int SG = NT / ITEMS;
  static_assert(NT % ITEMS == 0 && SG >= 1, "merge work split");
  float* obuf = reinterpret_cast<float*>(pex);            // [GK][D]
  float* mpart = reinterpret_cast<float*>(tabs);          // [SG][ITEMS][6]
  static_assert(sizeof(tabs) >= NT * 6 * 4, "merge partials fit the table space");
  static_assert(sizeof(pex) >= GK * D * 4, "output staging fits the weight slots");
  {
    const int item = tid % ITEMS, sg = tid / ITEMS;
    const int g = item / (D / 4), c4 = item % (D / 4);
    // one descriptor per plane over this unit's GK heads (wave-uniform base);
    // a split past S is masked below (past the last head it reads as zero)
    const auto racc = dev::buffer_rsrc(a.acc + head0 * a.S * D, uint32_t(GK * a.S) * D * 4);
    const auto rml = dev::buffer_rsrc(a.ml + head0 * a.S * 2, uint32_t(GK * a.S) * 8);
    float Mx = -INFINITY, L = 0.f, sum[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int U = 8;
    constexpr int kDev = 16;                 // cache policy: device scope (sc1)
    for (int s0 = sg; s0 < a.S; s0 += U * SG) {
      mx_u4 av[U];
      mx_u2 mv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t sp = uint32_t(g * a.S + s0 + u * SG);
        av[u] = __builtin_amdgcn_raw_buffer_load_b128(racc, sp * (D * 4) + c4 * 16, 0, kDev);
        mv[u] = __builtin_amdgcn_raw_buffer_load_b64(rml, sp * 8, 0, kDev);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float m = __uint_as_float(mv[u][0]);
        if (s0 + u * SG < a.S && m != -INFINITY) {
          const float nm = fmaxf(Mx, m);
          const float a1 = __builtin_amdgcn_exp2f(Mx - nm);
          const float a2 = __builtin_amdgcn_exp2f(m - nm);
#pragma unroll
          for (int k = 0; k < 4; ++k) sum[k] = fmaf(__uint_as_float(av[u][k]), a2, sum[k] * a1);
          L = fmaf(__uint_as_float(mv[u][1]), a2, L * a1);
          Mx = nm;
        }
      }
    }
    float* mp = mpart + (sg * ITEMS + item) * 6;
    mp[0] = Mx;
    mp[1] = L;
#pragma unroll
    for (int k = 0; k < 4; ++k) mp[2 + k] = sum[k];
  }
  __syncthreads();
  if (tid < ITEMS) {
    float Mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < SG; ++q) Mx = fmaxf(Mx, mpart[(q * ITEMS + tid) * 6]);
    float L = 0.f, sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      const float* mp = mpart + (q * ITEMS + tid) * 6;
      const float f = mp[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp[0] - Mx);
      L = fmaf(mp[1], f, L);
#pragma unroll
      for (int k = 0; k < 4; ++k) sum[k] = fmaf(mp[2 + k], f, sum[k]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int k = 0; k < 4; ++k) obuf[4 * tid + k] = sum[k] * inv;
  }
  __syncthreads();
  if (tid < 16 * GK) {
    constexpr int E = D / 16;
    const int g = tid >> 4, l16 = tid & 15;
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = obuf[g * D + l16 * E + i];
    dev::fwht16<E, float>(v, l16);
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
    const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = (smask >> i & 1) ? -v[i] * nn : v[i] * nn;
    float4* dst = reinterpret_cast<float4*>(a.out + (head0 + g) * D + l16 * E);
#pragma unroll
    for (int k = 0; k < E / 4; ++k)
      dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
  // the counter goes back to zero for the next call on this workspace
  if (tid == 0) __hip_atomic_store(a.cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Merge of split partials (exact log-sum-exp in a fixed order) and 1/l.
// The partials are already in the original frame, so every coordinate is
// independent: grid (query head, block of 32 coordinates), 256 threads =
// 32 coordinates x 8 split groups.
// ---------------------------------------------------------------------------

constexpr int kMaxSplits = 4096;

template <int D>
__global__ void __launch_bounds__(256) k_merge(MergeArgs a) {
  __shared__ float wts[kMaxSplits];
  __shared__ float red[2][4];
  __shared__ float part[8][32];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t head = blockIdx.x;
  const int cb = blockIdx.y;
  const float2* ml = reinterpret_cast<const float2*>(a.ml + head * a.S * 2);
  const int c = tid & 31, sg = tid >> 5;
  const float* col = a.acc + head * int64_t(a.S) * D + cb * 32 + c;

  // the first U partials of this (coordinate, split group) are loaded
  // before the reductions, so both memory round trips overlap
  constexpr int U = 8;
  float v0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int sp = sg + 8 * u;
    v0[u] = sp < a.S ? col[int64_t(sp) * D] : 0.f;
  }
  float mx = -INFINITY;
  for (int sp = tid; sp < a.S; sp += 256) mx = fmaxf(mx, ml[sp].x);
  mx = dev::wave_max(mx);
  if (lane == 0) red[0][wv] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float l = 0.f;
  for (int sp = tid; sp < a.S; sp += 256) {
    const float2 m2 = ml[sp];
    const float w = exp2f(m2.x - M);
    wts[sp] = w;
    l = fmaf(m2.y, w, l);
  }
  l = dev::wave_sum(l);
  if (lane == 0) red[1][wv] = l;
  __syncthreads();
  const float inv_l = 1.f / ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3]));

  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int sp = sg + 8 * u;
    if (sp < a.S) sum = fmaf(wts[sp], v0[u], sum);
  }
  int sp = sg + 8 * U;
  for (; sp + 7 * 8 < a.S; sp += 8 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = col[int64_t(sp + 8 * u) * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum = fmaf(wts[sp + 8 * u], v[u], sum);
  }
  for (; sp < a.S; sp += 8) sum = fmaf(wts[sp], col[int64_t(sp) * D], sum);
  part[sg][c] = sum;
  __syncthreads();
  if (tid < 32) {
    float t = part[0][tid];
#pragma unroll
    for (int g = 1; g < 8; ++g) t += part[g][tid];
    a.out[head * D + cb * 32 + tid] = t * inv_l;
  }
}

}  // namespace tq
