// Group-affine KV cache with rotated keys: encode and split-K decode.
//
// The cache layout of the mlx-turboquant README ("Quantize the KV cache",
// "How it plugs in", "Memory footprint over long context"): per token and KV
// head, d codes of b bits (LSB-first bitstream) and, per group of 64
// coordinates, an fp16 scale and an fp16 bias; the keys are rotated by the
// same seeded Hadamard rotation as the codebook cache, the values are not.
// Dequantized coordinate: scale * code + bias.
//
// Encode: 16 lanes per row, fp64 arithmetic (rotation, group min/max, the
// code division), fp16 scale and bias rounded once from fp64.
// Decode: one workgroup of 4 waves per (split, KV head, chunk of GK query
// heads); wave w runs its own online softmax for head w % GK over every
// (4 / GK)-th 64-token tile and the waves of a head are combined at the end;
// partials are merged by the codebook path's log-sum-exp merge kernel.
//   scores  lane = token: s_g = sum_grp scale_grp * (q'_g . codes)_grp
//           + bias_grp * (sum of q'_g over the group), q' = R q * tau * log2 e
//   values  lane = (quarter of the tile's tokens, d/16 consecutive
//           coordinates): the wave's 64 value rows are staged in its own LDS
//           slot and each lane reads its bits of its 16 rows; o_c = sum_t
//           p_t scale_t code_tc + sum_t p_t bias_t, quarters summed at the end.
#include <algorithm>
#include <cmath>

#include "tq_internal.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kAffGroup = 64;
constexpr int kAffWaves = 4;
constexpr int kAffTile = 64;

struct AffEncodeArgs {
  const void* x;          // [rows_bh][n_new][D] of dt
  uint8_t* codes;         // [rows_bh][capacity][D * BITS / 8]
  uint16_t* scale;        // [rows_bh][capacity][D / 64]
  uint16_t* bias;
  int64_t rows;           // rows_bh * n_new
  int64_t n_new;
  int64_t offset;
  int64_t capacity;
  uint64_t seed;
  int dt;
};

template <int D, int BITS, bool ROT>
__global__ void __launch_bounds__(256) k_affine_encode(AffEncodeArgs a) {
  constexpr int E = D / 16;                   // coordinates per lane
  constexpr int LPG = kAffGroup / E;          // lanes per group (8 or 4)
  constexpr int L = (1 << BITS) - 1;
  constexpr int NG = D / kAffGroup;
  constexpr int LBITS = E * BITS;             // bits per lane: 16 .. 64
  const int l16 = threadIdx.x & 15;
  const int64_t stride = int64_t(gridDim.x) * 16;
  for (int64_t r = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4); r < a.rows; r += stride) {
    const int64_t bh = r / a.n_new;
    const int64_t t = r - bh * a.n_new;
    float f[E];
    dev::load_row_part<E>(a.x, a.dt, r * D + l16 * E, f);
    double u[E];
#pragma unroll
    for (int i = 0; i < E; ++i) u[i] = double(f[i]);
    if constexpr (ROT) {
      const uint32_t neg = dev::sign_mask(a.seed, l16 * E, E);
#pragma unroll
      for (int i = 0; i < E; ++i) if (neg >> i & 1) u[i] = -u[i];
      dev::fwht16<E, double>(u, l16);
      const double rd = sqrt(double(D));
#pragma unroll
      for (int i = 0; i < E; ++i) u[i] /= rd;
    }
    double lo = u[0], hi = u[0];
#pragma unroll
    for (int i = 1; i < E; ++i) {
      lo = fmin(lo, u[i]);
      hi = fmax(hi, u[i]);
    }
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) {
      lo = fmin(lo, __shfl_xor(lo, m, 16));
      hi = fmax(hi, __shfl_xor(hi, m, 16));
    }
    const uint16_t s16 = dev::f64_to_f16_bits((hi - lo) / double(L));
    const uint16_t b16 = dev::f64_to_f16_bits(lo);
    const double s = dev::f16_bits_to_f64(s16), b = dev::f16_bits_to_f64(b16);
    uint64_t w0 = 0, w1 = 0;                  // the lane's LBITS bits
#pragma unroll
    for (int i = 0; i < E; ++i) {
      double c = 0.0;
      if (s > 0.0) c = fmin(fmax(rint((u[i] - b) / s), 0.0), double(L));
      const uint64_t code = uint64_t(c);
      const int pos = i * BITS;
      if (pos < 64) {
        w0 |= code << pos;
        if (pos + BITS > 64) w1 |= code >> (64 - pos);
      } else {
        w1 |= code << (pos - 64);
      }
    }
    const int64_t rec = bh * a.capacity + a.offset + t;
    uint8_t* dst = a.codes + rec * (D * BITS / 8) + l16 * (LBITS / 8);
    if constexpr (LBITS <= 64) {
      dev::store_bytes(dst, w0, LBITS / 8);
    } else {
      dev::store_bytes(dst, w0, 8);
      dev::store_bytes(dst + 8, w1, LBITS / 8 - 8);
    }
    if (l16 % LPG == 0) {
      a.scale[rec * NG + l16 / LPG] = s16;
      a.bias[rec * NG + l16 / LPG] = b16;
    }
  }
}

struct AffDecodeArgs {
  const void* q;          // [B][Hq][D] of q_dtype
  const uint8_t* kc;      // [B*Hkv][capacity][D*BK/8]
  const uint8_t* vc;
  const uint16_t* ks;     // [B*Hkv][capacity][D/64] fp16
  const uint16_t* kb;
  const uint16_t* vs;
  const uint16_t* vb;
  float* acc;             // [B*Hq][S][D] partial sums (original value frame)
  float* ml;              // [B*Hq][S][2]: running max (log2 units), sum
  int64_t capacity;
  int64_t n_ctx;
  int64_t tps;            // tokens per split (multiple of 64)
  int S;
  int Hq, Hkv, G, chunks;
  int q_dtype;
  float qmult;            // tau * log2(e)
  uint32_t sbits[8];      // key rotation signs (bit set: negative)
};

template <int D, int BK, int BV, int GK>
__global__ void __launch_bounds__(64 * kAffWaves) k_affine_decode(AffDecodeArgs a) {
  constexpr int W = kAffWaves;
  constexpr int R = W / GK;                    // token streams per workgroup
  constexpr int NG = D / kAffGroup;
  constexpr int KREC = D * BK / 8;
  constexpr int VREC = D * BV / 8;
  constexpr int KW = KREC / 4;
  constexpr int VLD = VREC / 16;               // 16-byte value loads per lane
  constexpr int VS = VREC + 16;                // staged row stride (bytes)
  constexpr int CPL = D / 16;                  // value coordinates per lane
  constexpr int LB = CPL * BV;                 // value bits per lane and row (<= 64)
  constexpr int TQ = kAffTile / 4;             // tokens per lane quarter
  static_assert(KREC % 16 == 0 && VREC % 16 == 0, "records are whole 16-byte loads");

  __shared__ __attribute__((aligned(16))) float qs[GK][D];
  __shared__ float qsum[GK][NG];
  // 4-bit keys: q' as fp16 pairs in the order of the nibble-pair extraction
  // (pair 4k + m = coordinates 8k + m and 8k + m + 4)
  __shared__ __attribute__((aligned(16))) uint32_t qh[GK][D / 2];
  __shared__ __attribute__((aligned(16))) uint8_t vst[W][kAffTile * VS];
  __shared__ float2 vsb[W][kAffTile][NG];
  __shared__ float pw[W][kAffTile];
  __shared__ float mlx[W][2];
  // after the tile loop the value slots hold the per-wave partial rows
  static_assert(sizeof(vst) >= sizeof(float) * W * D, "partials fit the value slots");
  float (*slab)[D] = reinterpret_cast<float (*)[D]>(&vst[0][0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int chunk = unit % a.chunks;
  const int bkv = unit / a.chunks;
  const int b = bkv / a.Hkv;
  const int kvh = bkv - b * a.Hkv;
  const int64_t head0 = int64_t(b) * a.Hq + kvh * a.G + chunk * GK;
  const int64_t t_begin = int64_t(split) * a.tps;
  const int64_t t_end = min(a.n_ctx, t_begin + a.tps);
  const int64_t row0 = int64_t(bkv) * a.capacity;

  // rotated, scaled query rows (16 lanes per head) and their group sums
  if (tid < 16 * GK) {
    constexpr int E = D / 16;
    const int g = tid >> 4, l16 = tid & 15;
    float v[E];
    dev::load_row_part<E>(a.q, a.q_dtype, (head0 + g) * D + l16 * E, v);
    const uint32_t neg = dev::bitmap_bits(a.sbits, l16 * E, E);
#pragma unroll
    for (int i = 0; i < E; ++i) if (neg >> i & 1) v[i] = -v[i];
    dev::fwht16<E, float>(v, l16);
    const float mult = a.qmult / sqrtf(float(D));
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      v[i] *= mult;
      qs[g][l16 * E + i] = v[i];
      part += v[i];
    }
#pragma unroll
    for (int kk = 0; kk < E / 8; ++kk) {
      const int k = l16 * (E / 8) + kk;
#pragma unroll
      for (int m = 0; m < 4; ++m) qh[g][4 * k + m] = dev::pack_f16x2(v[8 * kk + m], v[8 * kk + m + 4]);
    }
    // lanes l16 .. of one group: 64 / E consecutive lanes
    constexpr int LPG = kAffGroup / E;
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) part += __shfl_xor(part, m, 16);
    if (l16 % LPG == 0) qsum[g][l16 / LPG] = part;
  }
  __syncthreads();

  struct Tile {
    uint32_t kw[KW];
    uint32_t kscale[NG], kbias[NG];     // fp16 bits in the low half
    uint32_t vscale[NG], vbias[NG];
    uint32_t vx[VLD][4];
  };
  auto rows_left = [&](int64_t base) -> uint32_t {
    const int64_t n = t_end - base;
    return uint32_t(n <= 0 ? 0 : (n < kAffTile ? n : kAffTile));
  };
  auto load = [&](int64_t base, Tile& t) {
    const uint32_t n = rows_left(base);
    const auto rk = dev::buffer_rsrc(a.kc + (row0 + base) * KREC, n * KREC);
#pragma unroll
    for (int k = 0; k < KW / 4; ++k) {
      const auto q4 = __builtin_amdgcn_raw_buffer_load_b128(rk, uint32_t(lane) * KREC, 16 * k, 0);
      t.kw[4 * k] = q4[0]; t.kw[4 * k + 1] = q4[1]; t.kw[4 * k + 2] = q4[2];
      t.kw[4 * k + 3] = q4[3];
    }
    const auto rks = dev::buffer_rsrc(a.ks + (row0 + base) * NG, n * NG * 2);
    const auto rkb = dev::buffer_rsrc(a.kb + (row0 + base) * NG, n * NG * 2);
    const auto rvs = dev::buffer_rsrc(a.vs + (row0 + base) * NG, n * NG * 2);
    const auto rvb = dev::buffer_rsrc(a.vb + (row0 + base) * NG, n * NG * 2);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const uint32_t off = uint32_t(lane) * NG * 2 + 2 * gi;
      t.kscale[gi] = __builtin_amdgcn_raw_buffer_load_b16(rks, off, 0, 0);
      t.kbias[gi] = __builtin_amdgcn_raw_buffer_load_b16(rkb, off, 0, 0);
      t.vscale[gi] = __builtin_amdgcn_raw_buffer_load_b16(rvs, off, 0, 0);
      t.vbias[gi] = __builtin_amdgcn_raw_buffer_load_b16(rvb, off, 0, 0);
    }
    // value tile, flat: 16-byte chunk (lane + 64 k) of the 64 rows
    const auto rv = dev::buffer_rsrc(a.vc + (row0 + base) * VREC, n * VREC);
#pragma unroll
    for (int k = 0; k < VLD; ++k) {
      const auto q4 = __builtin_amdgcn_raw_buffer_load_b128(rv, uint32_t(lane + 64 * k) * 16, 0, 0);
      t.vx[k][0] = q4[0]; t.vx[k][1] = q4[1]; t.vx[k][2] = q4[2]; t.vx[k][3] = q4[3];
    }
  };

  // wave w serves query head hg = w % GK of the workgroup and token stream
  // w / GK (R = W / GK streams of interleaved 64-token tiles)
  const int hg = wave % GK;
  const int stream = wave / GK;
  float m_run = -INFINITY, lsum = 0.f, accb = 0.f, acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  uint8_t* my_v = vst[wave];
  // value phase: lane = (token quarter lane / 16, coordinates
  // CPL * (lane % 16) .. + CPL - 1); the quarters are summed at the end
  const int vcg = lane & 15, vtq = lane >> 4;
  const int vgrp = (vcg * CPL) / kAffGroup;          // the lane's value group
  const float* qrow = qs[hg];

  auto process = [&](int64_t base, const Tile& t) {
    const bool valid = base + lane < t_end;
    // ---- scores
    float dots[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) dots[gi] = 0.f;
    if constexpr (BK == 4) {
      // two codes per fp16 pair: (nibble | 0x6400) is 1024 + code in fp16,
      // a packed fp16 subtract leaves the exact codes, and v_dot2 against
      // the fp16 query pair accumulates in fp32
      const uint32_t* qhr = qh[hg];
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int gi = (8 * k) / kAffGroup;
        const uint4 qq = *reinterpret_cast<const uint4*>(qhr + 4 * k);
        const uint32_t qm[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t cp = ((t.kw[k] >> (4 * m)) & 0x000F000Fu) | 0x64006400u;
          const dev::half2_t ch =
              __builtin_bit_cast(dev::half2_t, cp) - dev::half2_t{_Float16(1024.f), _Float16(1024.f)};
          dots[gi] = dev::dot2(qm[m], __builtin_bit_cast(uint32_t, ch), dots[gi]);
        }
      }
    } else {
#pragma unroll
      for (int i4 = 0; i4 < D / 4; ++i4) {
        const int gi = (4 * i4) / kAffGroup;
        const float4 qv = *reinterpret_cast<const float4*>(qrow + 4 * i4);
        dots[gi] = fmaf(qv.x, float(dev::field<BK>(t.kw, 4 * i4)), dots[gi]);
        dots[gi] = fmaf(qv.y, float(dev::field<BK>(t.kw, 4 * i4 + 1)), dots[gi]);
        dots[gi] = fmaf(qv.z, float(dev::field<BK>(t.kw, 4 * i4 + 2)), dots[gi]);
        dots[gi] = fmaf(qv.w, float(dev::field<BK>(t.kw, 4 * i4 + 3)), dots[gi]);
      }
    }
    // ---- stage the value tile and its scales in this wave's LDS slot
#pragma unroll
    for (int k = 0; k < VLD; ++k) {
      const uint32_t flat = uint32_t(lane + 64 * k) * 16;
      const uint32_t row = flat / VREC, off = flat - row * VREC;
      *reinterpret_cast<uint4*>(my_v + row * VS + off) =
          make_uint4(t.vx[k][0], t.vx[k][1], t.vx[k][2], t.vx[k][3]);
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      vsb[wave][lane][gi] = make_float2(dev::f16_to_f32(t.vscale[gi]), dev::f16_to_f32(t.vbias[gi]));
    // ---- online softmax
    float s = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      s = fmaf(dev::f16_to_f32(t.kscale[gi]), dots[gi],
               fmaf(dev::f16_to_f32(t.kbias[gi]), qsum[hg][gi], s));
    const float mx = dev::dpp_wave_max(valid ? s : -INFINITY);
    if (mx > m_run) {                        // wave-uniform
      const float alpha = exp2f(m_run - mx);
      m_run = mx;
      lsum *= alpha;
      accb *= alpha;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] *= alpha;
    }
    const float p = valid ? exp2f(s - m_run) : 0.f;
    lsum += p;
    pw[wave][lane] = p;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- values: the lane's CPL coordinates over its 16 tokens
    const uint32_t bit0 = uint32_t(vcg) * LB;
    const uint32_t wsel = (bit0 >> 5) * 4, sh = bit0 & 31;
#pragma unroll 2
    for (int jj = 0; jj < TQ; ++jj) {
      const int j = vtq * TQ + jj;
      const uint8_t* rowp = my_v + j * VS + wsel;
      uint64_t x = *reinterpret_cast<const uint32_t*>(rowp);
      if (sh + LB > 32) x |= uint64_t(*reinterpret_cast<const uint32_t*>(rowp + 4)) << 32;
      x >>= sh;
      if (sh + LB > 64) x |= uint64_t(*reinterpret_cast<const uint32_t*>(rowp + 8)) << (64 - sh);
      const float2 sb = vsb[wave][j][vgrp];
      const float pj = pw[wave][j];
      const float ws = pj * sb.x;
      accb = fmaf(pj, sb.y, accb);
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        acc[c] = fmaf(ws, float(uint32_t(x >> (c * BV)) & ((1u << BV) - 1u)), acc[c]);
    }
    // the slot is rewritten by the next tile of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  const int64_t step = int64_t(R) * kAffTile;
  const int iters = int((t_end - t_begin + step - 1) / step);
  const int64_t wb = t_begin + int64_t(stream) * kAffTile;
  {
    Tile ta, tb;
    load(wb, ta);
    for (int it = 0; it < iters; it += 2) {
      const int64_t base = wb + int64_t(it) * step;
      if (it + 1 < iters) load(base + step, tb);
      process(base, ta);
      if (it + 1 >= iters) break;
      if (it + 2 < iters) load(base + 2 * step, ta);
      process(base + step, tb);
    }
  }

  // ---- combine the waves of each head
  {
    const float l = dev::wave_sum(lsum);
    if (lane == 0) {
      mlx[wave][0] = m_run;
      mlx[wave][1] = l;
    }
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = hg; w < W; w += GK) M = fmaxf(M, mlx[w][0]);
  {
    // sum the four token quarters (lanes vcg, vcg + 16, vcg + 32, vcg + 48)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      acc[c] += __shfl_xor(acc[c], 16);
      acc[c] += __shfl_xor(acc[c], 32);
    }
    accb += __shfl_xor(accb, 16);
    accb += __shfl_xor(accb, 32);
    const float f = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
    if (vtq == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) slab[wave][vcg * CPL + c] = (acc[c] + accb) * f;
    }
  }
  __syncthreads();
  for (int i = tid; i < GK * D; i += 64 * W) {
    const int g = i / D, c = i - g * D;
    float sum = 0.f;
#pragma unroll
    for (int w = g; w < W; w += GK) sum += slab[w][c];
    a.acc[((head0 + g) * a.S + split) * D + c] = sum;
  }
  if (tid < GK) {
    float Mg = -INFINITY;
    for (int w = tid; w < W; w += GK) Mg = fmaxf(Mg, mlx[w][0]);
    float l = 0.f;
    for (int w = tid; w < W; w += GK) {
      const float mw = mlx[w][0];
      if (mw != -INFINITY) l += mlx[w][1] * exp2f(mw - Mg);
    }
    float* ml = a.ml + ((head0 + tid) * a.S + split) * 2;
    ml[0] = Mg;
    ml[1] = l;
  }
}

// ----------------------------------------------------------------------------
// host side

int aff_device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return TQ_ERR_NO_DEVICE;
  return TQ_OK;
}

int aff_last_launch() { return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

bool aff_bits_ok(int b) { return b >= 2 && b <= 4; }

int aff_check_config(const tq_affine_config* c) {
  if (!c) return TQ_ERR_ARG;
  if (!valid_d(c->d) || !aff_bits_ok(c->bits_k) || !aff_bits_ok(c->bits_v) ||
      c->group != kAffGroup)
    return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

int64_t aff_plane(const tq_affine_config* c, int B, int Hkv, int64_t cap, int which) {
  const int64_t rows = int64_t(B) * Hkv * cap;
  switch (which) {
    case 0: return rows * (c->d * c->bits_k / 8);
    case 1: return rows * (c->d * c->bits_v / 8);
    default: return rows * (c->d / kAffGroup) * 2;
  }
}

int aff_check_cache(const tq_affine_config* c, const tq_affine_cache* k) {
  if (!k || k->B < 0 || k->Hkv < 1 || k->capacity < 0) return TQ_ERR_ARG;
  const void* p[6] = {k->kc, k->vc, k->ks, k->kb, k->vs, k->vb};
  for (const void* x : p) {
    if (!x && int64_t(k->B) * k->capacity > 0) return TQ_ERR_ARG;
    if (x && !aligned16(x)) return TQ_ERR_ALIGN;
  }
  (void)c;
  return TQ_OK;
}

struct AffPlan {
  int gk, chunks, S;
  int64_t tps;
  int64_t acc_bytes, total;
};

int aff_plan(const tq_affine_config* c, int B, int Hq, int Hkv, int64_t n_ctx, int splits,
             AffPlan* p) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 1 || splits < 0) return TQ_ERR_ARG;
  const int G = Hq / Hkv;
  p->gk = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  p->chunks = G / p->gk;
  const int64_t units = int64_t(B) * Hkv * p->chunks;
  const int64_t round = int64_t(kAffWaves) * kAffTile;
  const int64_t max_s = std::min<int64_t>(kMaxSplitCount, (n_ctx + round - 1) / round);
  // about 2048 workgroups by default (8 per compute unit, two resident at
  // a time): measured fastest for long contexts
  int64_t S = splits > 0 ? splits : (2048 + units - 1) / units;
  S = std::max<int64_t>(1, std::min(S, max_s));
  int64_t tps = (n_ctx + S - 1) / S;
  tps = (tps + kAffTile - 1) / kAffTile * kAffTile;
  S = (n_ctx + tps - 1) / tps;
  if (units * S > (int64_t(1) << 31) - 1 || units > 65535) return TQ_ERR_UNSUPPORTED;
  p->S = int(S);
  p->tps = tps;
  const int64_t heads = int64_t(B) * Hq;
  p->acc_bytes = (heads * S * c->d * 4 + 255) / 256 * 256;
  p->total = p->acc_bytes + heads * S * 2 * 4;
  return TQ_OK;
}

template <int D, int BK>
int launch_aff_decode_bv(int bv, int gk, const AffDecodeArgs& a, dim3 grid, hipStream_t st) {
#define TQ_AFF_GO(BV, GK) \
  hipLaunchKernelGGL((k_affine_decode<D, BK, BV, GK>), grid, dim3(64 * kAffWaves), 0, st, a)
  if (bv == 2) {
    if (gk == 4) TQ_AFF_GO(2, 4); else if (gk == 2) TQ_AFF_GO(2, 2); else TQ_AFF_GO(2, 1);
  } else if (bv == 3) {
    if (gk == 4) TQ_AFF_GO(3, 4); else if (gk == 2) TQ_AFF_GO(3, 2); else TQ_AFF_GO(3, 1);
  } else {
    if (gk == 4) TQ_AFF_GO(4, 4); else if (gk == 2) TQ_AFF_GO(4, 2); else TQ_AFF_GO(4, 1);
  }
#undef TQ_AFF_GO
  return aff_last_launch();
}

template <int D>
int launch_aff_decode(int bk, int bv, int gk, const AffDecodeArgs& a, dim3 grid, hipStream_t st) {
  if (bk == 2) return launch_aff_decode_bv<D, 2>(bv, gk, a, grid, st);
  if (bk == 3) return launch_aff_decode_bv<D, 3>(bv, gk, a, grid, st);
  return launch_aff_decode_bv<D, 4>(bv, gk, a, grid, st);
}

template <int D>
int launch_aff_encode(int bits, bool rot, const AffEncodeArgs& a, hipStream_t st) {
  const int64_t g = (a.rows + 15) / 16;
  const dim3 grid(unsigned(g < 16384 ? g : 16384));
#define TQ_AFF_ENC(BITS) \
  do { \
    if (rot) hipLaunchKernelGGL((k_affine_encode<D, BITS, true>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((k_affine_encode<D, BITS, false>), grid, dim3(256), 0, st, a); \
  } while (0)
  if (bits == 2) TQ_AFF_ENC(2); else if (bits == 3) TQ_AFF_ENC(3); else TQ_AFF_ENC(4);
#undef TQ_AFF_ENC
  return aff_last_launch();
}

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" {

int64_t tq_affine_cache_bytes(const tq_affine_config* cfg, int B, int Hkv, int64_t capacity,
                              int64_t* plane_bytes) {
  const int st = aff_check_config(cfg);
  if (st != TQ_OK) return st;
  if (B < 0 || Hkv < 1 || capacity < 0) return TQ_ERR_ARG;
  int64_t total = 0;
  for (int i = 0; i < 6; ++i) {
    const int64_t n = aff_plane(cfg, B, Hkv, capacity, i < 2 ? i : 2);
    if (plane_bytes) plane_bytes[i] = n;
    total += n;
  }
  return total;
}

int tq_affine_encode_kv(const tq_affine_config* cfg, const void* k, const void* v, int in_dtype,
                        int64_t offset, int64_t n_new, const tq_affine_cache* cache,
                        hipStream_t stream) {
  int st = aff_check_config(cfg);
  if (st != TQ_OK) return st;
  st = aff_check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!valid_in_dtype(in_dtype)) return TQ_ERR_UNSUPPORTED;
  if (offset < 0 || n_new < 0) return TQ_ERR_ARG;
  if (offset + n_new > cache->capacity) return TQ_ERR_CAPACITY;
  const int64_t rows = int64_t(cache->B) * cache->Hkv * n_new;
  if (rows == 0) return TQ_OK;
  if (!k || !v) return TQ_ERR_ARG;
  if (!aligned16(k) || !aligned16(v)) return TQ_ERR_ALIGN;
  st = aff_device_ready();
  if (st != TQ_OK) return st;
  AffEncodeArgs a{};
  a.rows = rows;
  a.n_new = n_new;
  a.offset = offset;
  a.capacity = cache->capacity;
  a.seed = cfg->seed;
  a.dt = in_dtype;
  for (int kv = 0; kv < 2; ++kv) {
    a.x = kv == 0 ? k : v;
    a.codes = static_cast<uint8_t*>(kv == 0 ? cache->kc : cache->vc);
    a.scale = static_cast<uint16_t*>(kv == 0 ? cache->ks : cache->vs);
    a.bias = static_cast<uint16_t*>(kv == 0 ? cache->kb : cache->vb);
    const int bits = kv == 0 ? cfg->bits_k : cfg->bits_v;
    st = cfg->d == 128 ? launch_aff_encode<128>(bits, kv == 0, a, stream)
                       : launch_aff_encode<256>(bits, kv == 0, a, stream);
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

int tq_affine_num_splits(const tq_affine_config* cfg, int B, int Hq, int Hkv, int64_t n_ctx,
                         int splits) {
  int st = aff_check_config(cfg);
  if (st != TQ_OK) return st;
  AffPlan p;
  st = aff_plan(cfg, B, Hq, Hkv, n_ctx, splits, &p);
  return st != TQ_OK ? st : p.S;
}

int64_t tq_affine_workspace_bytes(const tq_affine_config* cfg, int B, int Hq, int Hkv,
                                  int64_t n_ctx, int splits) {
  int st = aff_check_config(cfg);
  if (st != TQ_OK) return st;
  AffPlan p;
  st = aff_plan(cfg, B, Hq, Hkv, n_ctx, splits, &p);
  return st != TQ_OK ? st : p.total;
}

int tq_affine_attend_decode(const tq_affine_config* cfg, const void* q, int q_dtype, int B,
                            int Hq, const tq_affine_cache* cache, int64_t n_ctx, float scale,
                            int splits, float* out, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  int st = aff_check_config(cfg);
  if (st != TQ_OK) return st;
  st = aff_check_cache(cfg, cache);
  if (st != TQ_OK) return st;
  if (!q || !out || !ws || B != cache->B) return TQ_ERR_ARG;
  if (!valid_in_dtype(q_dtype)) return TQ_ERR_UNSUPPORTED;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return TQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return TQ_ERR_ALIGN;
  if (n_ctx > cache->capacity) return TQ_ERR_CAPACITY;
  AffPlan p;
  st = aff_plan(cfg, B, Hq, cache->Hkv, n_ctx, splits, &p);
  if (st != TQ_OK) return st;
  if (int64_t(ws_bytes) < p.total) return TQ_ERR_WORKSPACE;
  st = aff_device_ready();
  if (st != TQ_OK) return st;

  AffDecodeArgs a{};
  a.q = q;
  a.kc = static_cast<const uint8_t*>(cache->kc);
  a.vc = static_cast<const uint8_t*>(cache->vc);
  a.ks = static_cast<const uint16_t*>(cache->ks);
  a.kb = static_cast<const uint16_t*>(cache->kb);
  a.vs = static_cast<const uint16_t*>(cache->vs);
  a.vb = static_cast<const uint16_t*>(cache->vb);
  a.acc = static_cast<float*>(ws);
  a.ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.acc_bytes);
  a.capacity = cache->capacity;
  a.n_ctx = n_ctx;
  a.tps = p.tps;
  a.S = p.S;
  a.Hq = Hq;
  a.Hkv = cache->Hkv;
  a.G = Hq / cache->Hkv;
  a.chunks = p.chunks;
  a.q_dtype = q_dtype;
  const double tau = scale > 0.f ? double(scale) : 1.0 / std::sqrt(double(cfg->d));
  a.qmult = float(tau * 1.4426950408889634);
  for (int w = 0; w < 8; ++w) a.sbits[w] = 0;
  for (int i = 0; i < cfg->d; ++i)
    if (splitmix64_at(cfg->seed, uint64_t(i)) >> 63) a.sbits[i >> 5] |= 1u << (i & 31);

  const dim3 grid(unsigned(p.S), unsigned(int64_t(B) * cache->Hkv * p.chunks));
  st = cfg->d == 128 ? launch_aff_decode<128>(cfg->bits_k, cfg->bits_v, p.gk, a, grid, stream)
                     : launch_aff_decode<256>(cfg->bits_k, cfg->bits_v, p.gk, a, grid, stream);
  if (st != TQ_OK) return st;
  MergeArgs m{};
  m.ml = a.ml;
  m.acc = a.acc;
  m.out = out;
  m.heads = int64_t(B) * Hq;
  m.S = p.S;
  const dim3 mgrid(unsigned(m.heads), unsigned(cfg->d / 32));
  if (cfg->d == 128)
    hipLaunchKernelGGL(k_merge<128>, mgrid, dim3(256), 0, stream, m);
  else
    hipLaunchKernelGGL(k_merge<256>, mgrid, dim3(256), 0, stream, m);
  return aff_last_launch();
}

}  // extern "C"
