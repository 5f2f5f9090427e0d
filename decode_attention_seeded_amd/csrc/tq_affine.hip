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
#include <cstdlib>

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
// Matrix-core decode of the 4-bit affine format at d 128 (up to 4 query
// heads per workgroup; the layout also takes d 256 with up to 2). A 4-bit code c enters the
// products as the fp16 number 64 + c: low byte c << 4 (a byte's high
// nibble as it is, or its low nibble shifted up) and high byte 0x54, placed
// by one v_perm (exact: fp16 spacing is 1/16 in [64, 128), and an offset
// small enough next to the codes' own contribution that the fp32 sums keep
// their precision); the offset is taken back out in fp32 per group, from the
// query's group sums (scores) and from the sum of the rounded weights
// (values). Per 64-token wave tile:
//   scores  lane = token, v_mfma_f32_4x4x4_16b_f16 with the query block
//           broadcast: step j takes 4 coordinates of one key dword, in the
//           order (0, 2, 1, 3) or (4, 6, 5, 7) of its 8 codes (the even and
//           the odd nibbles, each masked out with one AND); one accumulator
//           pair per group of 64 coordinates, then
//           s = sum_grp ks_grp (dot_grp - 64 qsum16_grp) 2^qe + kb_grp qsum_grp
//   values  v_mfma_f32_16x16x32_f16: column n = the lane's D/16 coordinates,
//           K = (token, pair element), and A row g + GK (j + 2 grp) carries
//           head g's weight p * vscale_grp for pair element j; a column only
//           keeps the rows of its own group. sum_t p vbias_grp and the
//           weights' own sum (for the offset) are per-lane fp32 sums.
// Split partials (original value frame) are merged by k_merge.
template <int D, int GK>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
k_affine_decode_mx(AffDecodeArgs a) {
  constexpr int W = 8, TW = 64, T = W * TW;
  constexpr int NG = D / kAffGroup;            // groups per row
  constexpr int KREC = D / 2, VREC = D / 2;    // 4-bit rows
  constexpr int KW = D / 8;                    // key dwords per row (lane = token)
  constexpr int NS = D / 4;                    // score steps
  constexpr int NQ = NS / 16;                  // query quads per lane
  constexpr int SB = D / 32;                   // value slots (pairs) per (token, column)
  constexpr int VW = D / 128;                  // value dwords per (token, column)
  constexpr int CPC = D / 16;                  // coordinates per column
  constexpr int CPG = 16 / NG;                 // columns per group
  constexpr int NROW = GK * 2 * NG;            // live A rows
  constexpr int PX = GK * NG * TW / 2;         // weight dwords per wave tile
  constexpr float kRescale = 8.0f;
  static_assert(NROW <= 16, "A rows: heads x pair element x group");
  using mx_h4 = _Float16 __attribute__((ext_vector_type(4)));
  using mx_h8 = _Float16 __attribute__((ext_vector_type(8)));
  using mx_f4 = float __attribute__((ext_vector_type(4)));
  using mx_u2 = uint32_t __attribute__((ext_vector_type(2)));
  using mx_u4 = uint32_t __attribute__((ext_vector_type(4)));

  __shared__ __attribute__((aligned(16))) uint32_t pex[W][2][PX];
  __shared__ __attribute__((aligned(16))) uint32_t qs[GK][NS * 2];   // fp16 steps
  __shared__ float qsum[GK][NG], qsum16[GK][NG];
  __shared__ int qexp;
  __shared__ __attribute__((aligned(16))) float slab[W][GK][D];
  __shared__ float wst[W][GK][2 + 2 * NG];      // m, l, then per group bias and weight sums
  __shared__ int vexp_w[W];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kq = lane >> 4;
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
  const int iters = int((t_end - t_begin + T - 1) / T);

  // ---- query rows: R q * tau * log2 e, one power of two 2^-qe for the GK
  // rows (largest element near 2^10), fp16 in score-step order
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
    float vmax = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      v[i] *= mult;
      vmax = fmaxf(vmax, fabsf(v[i]));
    }
    vmax = dev::group_max16(vmax);
    if constexpr (GK >= 2) vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
    if constexpr (GK >= 4) vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
    const int qe = vmax > 0.f ? ilogbf(vmax) - 10 : 0;
    if (tid == 0) qexp = qe;
    // the lane's E coordinates l16 E .. are whole key dwords (8 codes):
    // steps 2k, 2k + 1 of dword k take coordinates (0, 2, 1, 3), (4, 6, 5, 7)
    float part = 0.f, part16 = 0.f;
#pragma unroll
    for (int kk = 0; kk < E / 8; ++kk) {
      const int k = l16 * (E / 8) + kk;
      _Float16 h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[e] = _Float16(ldexpf(v[8 * kk + e], -qe));
        part += v[8 * kk + e];
        part16 += float(h[e]);
      }
      qs[g][4 * k + 0] = __builtin_bit_cast(uint32_t, dev::half2_t{h[0], h[2]});
      qs[g][4 * k + 1] = __builtin_bit_cast(uint32_t, dev::half2_t{h[1], h[3]});
      qs[g][4 * k + 2] = __builtin_bit_cast(uint32_t, dev::half2_t{h[4], h[6]});
      qs[g][4 * k + 3] = __builtin_bit_cast(uint32_t, dev::half2_t{h[5], h[7]});
    }
    constexpr int LPG = kAffGroup / E;          // lanes per group
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) {
      part += __shfl_xor(part, m, 16);
      part16 += __shfl_xor(part16, m, 16);
    }
    if (l16 % LPG == 0) {
      qsum[g][l16 / LPG] = part;
      qsum16[g][l16 / LPG] = part16;
    }
  }

  // ---- tiles: keys lane = token; values lane = (token kq + 4 (i % 4) +
  // 16 (i / 4), column col), whole 64-byte rows per four lanes
  struct Tile {
    uint32_t kw[KW];
    uint32_t ks[NG], kb[NG], vs[NG], vb[NG];     // fp16 bits
    uint32_t vx[16][VW];
  };
  auto rows_left = [&](int64_t base) -> uint32_t {
    const int64_t n = t_end - base;
    return uint32_t(n <= 0 ? 0 : (n < TW ? n : TW));
  };
  constexpr int kNT = 2;                       // nontemporal
  const uint32_t vo0 = uint32_t(kq) * VREC + uint32_t(col) * (4 * VW);
  auto load = [&](int64_t base, Tile& t) {
    const uint32_t n = rows_left(base);
    const auto rk = dev::buffer_rsrc(a.kc + (row0 + base) * KREC, n * KREC);
#pragma unroll
    for (int k = 0; k < KW / 4; ++k) {
      const auto q4 = __builtin_amdgcn_raw_buffer_load_b128(rk, uint32_t(lane) * KREC, 16 * k, 0);
      t.kw[4 * k] = q4[0]; t.kw[4 * k + 1] = q4[1]; t.kw[4 * k + 2] = q4[2];
      t.kw[4 * k + 3] = q4[3];
    }
    const uint16_t* pl[4] = {a.ks, a.kb, a.vs, a.vb};
    uint32_t* dst[4] = {t.ks, t.kb, t.vs, t.vb};
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) {
      const auto rs = dev::buffer_rsrc(pl[pi] + (row0 + base) * NG, n * NG * 2);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        dst[pi][gi] = __builtin_amdgcn_raw_buffer_load_b16(rs, uint32_t(lane) * NG * 2 + 2 * gi,
                                                           0, kNT);
    }
    const auto rv = dev::buffer_rsrc(a.vc + (row0 + base) * VREC, n * VREC);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int so = (16 * (i >> 2) + 4 * (i & 3)) * VREC;
      if constexpr (VW == 2) {
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rv, vo0, so, kNT);
        t.vx[i][0] = v2[0];
        t.vx[i][1] = v2[1];
      } else {
        t.vx[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo0, so, kNT);
      }
    }
  };
  const int64_t wb = t_begin + int64_t(wave) * TW;
  Tile ta, tb;
  load(wb, ta);
  load(wb + T, tb);
  __syncthreads();

  // query quads for the broadcast A operand (lane block lane/4 = step j % 16,
  // row lane % 4 = head)
  mx_u2 qa[NQ];
  {
    const int qm = lane & 3, qb = lane >> 2;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int j = qb + 16 * i;
      qa[i] = qm < GK ? mx_u2{qs[qm][2 * j], qs[qm][2 * j + 1]} : mx_u2{0u, 0u};
    }
  }
  const float qsc = ldexpf(1.f, qexp);
  float qs16[GK][NG], qsf[GK][NG];
#pragma unroll
  for (int g = 0; g < GK; ++g)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      qs16[g][gi] = 64.f * qsum16[g][gi];
      qsf[g][gi] = qsum[g][gi];
    }

  // weight slots (token 16 G + 4 u + kq at slot 16 G + 4 kq + u) and the A
  // operand selectors of the lane's row r = g + GK (j + 2 grp)
  const int pslot = (lane & 0x30) | ((lane & 3) << 2) | ((lane >> 2) & 3);
  uint32_t asel[2];
  int arow = 0;
  {
    const int r = col;
    const bool live = r < NROW;
    const int rg = r % GK, rj = (r / GK) & 1, rgrp = r / (2 * GK);
    constexpr uint32_t kZ = 0x0C0C0C0Cu;
    const uint32_t lo = rj ? 0x01000C0Cu : 0x0C0C0100u;
    const uint32_t hi = rj ? 0x03020C0Cu : 0x0C0C0302u;
    asel[0] = live ? lo : kZ;
    asel[1] = live ? hi : kZ;
    arow = live ? (rg * NG + rgrp) * TW : 0;
  }
  constexpr uint32_t kC54 = 0x54545454u;      // the high byte of 64 + c
  // halfwords (0x54 << 8 | byte b): bytes 0, 1 or 2, 3 of the nibble source
  constexpr uint32_t kLo = 0x04010400u, kHi = 0x04030402u;

  float m_run[GK], lpart[GK], bsum[GK][NG], wsum[GK][NG];
  int vexp = 0;
  float vsc = 1.f;                             // 2^-vexp
  mx_f4 acc[SB];
#pragma unroll
  for (int g = 0; g < GK; ++g) {
    m_run[g] = -INFINITY;
    lpart[g] = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) bsum[g][gi] = wsum[g][gi] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < SB; ++s) acc[s] = mx_f4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](int64_t base, uint32_t* px, const Tile& cur) {
    const bool valid = base + lane < t_end;
    // ---- scores
    mx_f4 sk[NG][2];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) sk[gi][0] = sk[gi][1] = mx_f4{0.f, 0.f, 0.f, 0.f};
    dev::static_for<0, KW>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      // even codes (low nibbles) and odd codes (high nibbles) as c << 4
      const uint32_t t0 = (cur.kw[k] << 4) & 0xF0F0F0F0u;
      const uint32_t t1 = cur.kw[k] & 0xF0F0F0F0u;
      dev::static_for<0, 2>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        constexpr int j = 2 * k + h;
        constexpr uint32_t sel = h ? kHi : kLo;
        const mx_u2 kb = {__builtin_amdgcn_perm(kC54, t0, sel), __builtin_amdgcn_perm(kC54, t1, sel)};
        constexpr int gi = (4 * j) / kAffGroup;
        sk[gi][j & 1] = __builtin_amdgcn_mfma_f32_4x4x4f16(
            __builtin_bit_cast(mx_h4, qa[j / 16]), __builtin_bit_cast(mx_h4, kb), sk[gi][j & 1], 4,
            j % 16, 0);
      });
    });
    float ksf[NG], kbf[NG], vw[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      ksf[gi] = dev::f16_to_f32(cur.ks[gi]) * qsc;
      kbf[gi] = dev::f16_to_f32(cur.kb[gi]);
      vw[gi] = dev::f16_to_f32(cur.vs[gi]) * vsc;
    }
    // value weights stay in fp16's normal range: the tile's largest scale
    // times 2^-vexp within [2^-6, 2^6] (p <= 2^8)
    {
      float vm = 0.f;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) vm = fmaxf(vm, vw[gi]);
      const bool high = __ballot(vm > 64.f) != 0;
      const bool low = __ballot(vm >= 0.015625f) == 0 && __ballot(vm > 0.f) != 0;
      if (high || low) {                       // wave-uniform, rare
        const int sh = ilogbf(dev::dpp_wave_max(vm)) - 4;
        vsc = ldexpf(vsc, -sh);
        vexp += sh;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) vw[gi] = ldexpf(vw[gi], -sh);
#pragma unroll
        for (int s = 0; s < SB; ++s)
#pragma unroll
          for (int g = 0; g < GK; ++g) acc[s][g] = ldexpf(acc[s][g], -sh);
        // (the weight sums are rescaled with them: they stay in acc's units)
#pragma unroll
        for (int g = 0; g < GK; ++g)
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) wsum[g][gi] = ldexpf(wsum[g][gi], -sh);
      }
    }
    // ---- online softmax, lazily raised running max
    uint16_t* p16 = reinterpret_cast<uint16_t*>(px);
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      float s = 0.f;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        s = fmaf(ksf[gi], (sk[gi][0][g] + sk[gi][1][g]) - qs16[g][gi], fmaf(kbf[gi], qsf[g][gi], s));
      if (__ballot(valid && s > m_run[g] + kRescale)) {      // wave-uniform
        const float mx = dev::dpp_wave_max(valid ? s : -INFINITY);
        const float m_new = fmaxf(m_run[g], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
        m_run[g] = m_new;
        lpart[g] *= alpha;
#pragma unroll
        for (int s2 = 0; s2 < SB; ++s2) acc[s2][g] *= alpha;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          bsum[g][gi] *= alpha;
          wsum[g][gi] *= alpha;
        }
      }
      const float e = __builtin_amdgcn_exp2f(s - m_run[g]);
      const float p = valid ? e : 0.f;
      lpart[g] += p;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const _Float16 w16 = _Float16(p * vw[gi]);
        p16[(g * NG + gi) * TW + pslot] = __builtin_bit_cast(uint16_t, w16);
        wsum[g][gi] += float(w16);
        bsum[g][gi] = fmaf(p, dev::f16_to_f32(cur.vb[gi]), bsum[g][gi]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- values: 16-token groups G; slot s of the column's dword s / 4:
    // pair (0, 2), (1, 3), (4, 6), (5, 7) of its 8 codes
    const uint16_t* pr = reinterpret_cast<const uint16_t*>(px) + arow + 4 * kq;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const mx_u2 X = *reinterpret_cast<const mx_u2*>(pr + 16 * G);
      const mx_u4 aw = {__builtin_amdgcn_perm(X[0], X[0], asel[0]),
                        __builtin_amdgcn_perm(X[0], X[0], asel[1]),
                        __builtin_amdgcn_perm(X[1], X[1], asel[0]),
                        __builtin_amdgcn_perm(X[1], X[1], asel[1])};
      const mx_h8 pa = __builtin_bit_cast(mx_h8, aw);
      uint32_t t0[4][VW], t1[4][VW];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int d = 0; d < VW; ++d) {
          t0[u][d] = (cur.vx[4 * G + u][d] << 4) & 0xF0F0F0F0u;
          t1[u][d] = cur.vx[4 * G + u][d] & 0xF0F0F0F0u;
        }
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int d = s >> 2, m = s & 3;
        const uint32_t sel = (m & 2) ? kHi : kLo;
        mx_u4 vb;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          vb[u] = __builtin_amdgcn_perm(kC54, (m & 1) ? t1[u][d] : t0[u][d], sel);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(mx_h8, vb), acc[s],
                                                        0, 0, 0);
      }
    }
  };

  {
    uint32_t* px0 = pex[wave][0];
    uint32_t* px1 = pex[wave][1];
    for (int it = 0; it < iters; it += 2) {
      const int64_t base = wb + int64_t(it) * T;
      process(base, px0, ta);
      if (it + 1 >= iters) break;
      load(base + 2 * T, ta);
      process(base + T, px1, tb);
      if (it + 2 >= iters) break;
      load(base + 3 * T, tb);
    }
  }

  // ---- this wave's partial: C row r = 4 kq + i is (head r % GK, pair
  // element (r / GK) & 1, group r / (2 GK)); a column keeps its own group
  {
    const int cgrp = col / CPG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kq + i;
      const int rg = r % GK, rj = (r / GK) & 1, rgrp = r / (2 * GK);
      if (r < NROW && rgrp == cgrp) {
#pragma unroll
        for (int s = 0; s < SB; ++s) {
          const int m = s & 3;
          const int c = CPC * col + 8 * (s >> 2) + ((m & 1) | ((m & 2) << 1)) + 2 * rj;
          slab[wave][rg][c] = acc[s][i];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GK; ++g) {
      const float l = dev::wave_sum(lpart[g]);
      float bs[NG], ws[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        bs[gi] = dev::wave_sum(bsum[g][gi]);
        ws[gi] = dev::wave_sum(wsum[g][gi]);
      }
      if (lane == 0) {
        wst[wave][g][0] = m_run[g];
        wst[wave][g][1] = l;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          wst[wave][g][2 + gi] = bs[gi];
          wst[wave][g][2 + NG + gi] = ws[gi];
        }
      }
    }
    if (lane == 0) vexp_w[wave] = vexp;
  }
  __syncthreads();
  // ---- combine the waves: o_c = sum_w f_w (2^vexp_w (C_w,c - 64 wsum_w)
  // + bsum_w) with f_w = 2^(m_w - M); unnormalized partial and (M, l) out
  for (int i = tid; i < GK * D; i += 64 * W) {
    const int g = i / D, c = i - g * D, gi = c / kAffGroup;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, wst[w][g][0]);
    float sum = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = wst[w][g][0];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      const float v = ldexpf(slab[w][g][c] - 64.f * wst[w][g][2 + NG + gi], vexp_w[w]) +
                      wst[w][g][2 + gi];
      sum = fmaf(v, f, sum);
      l = fmaf(wst[w][g][1], f, l);
    }
    a.acc[((head0 + g) * a.S + split) * D + c] = sum;
    if (c == 0) {
      float* ml = a.ml + ((head0 + g) * a.S + split) * 2;
      ml[0] = M;
      ml[1] = l;
    }
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
  int mx;              // 1: the matrix-core kernel (4-bit keys and values)
  int64_t tps;
  int64_t acc_bytes, total;
};

// The matrix-core kernel takes 4-bit keys and values at d 128
// (TQ_DECODE_VALU=1 in the environment keeps every format on the VALU kernel).
bool aff_use_mx(const tq_affine_config* c) {
  const char* v = std::getenv("TQ_DECODE_VALU");
  if (v && v[0] == '1') return false;
  return c->bits_k == 4 && c->bits_v == 4 && c->d == 128;
}

int aff_plan(const tq_affine_config* c, int B, int Hq, int Hkv, int64_t n_ctx, int splits,
             AffPlan* p) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || n_ctx < 1 || splits < 0) return TQ_ERR_ARG;
  const int G = Hq / Hkv;
  p->mx = aff_use_mx(c) ? 1 : 0;
  // matrix-core kernel: query heads x 2 x groups <= 16 product rows
  const int gmax = p->mx && c->d == 256 ? 2 : 4;
  p->gk = G % 4 == 0 && gmax >= 4 ? 4 : (G % 2 == 0 ? 2 : 1);
  p->chunks = G / p->gk;
  const int64_t units = int64_t(B) * Hkv * p->chunks;
  // tokens per workgroup round: 8 (matrix cores) or 4 waves of 64
  const int64_t round = p->mx ? 512 : int64_t(kAffWaves) * kAffTile;
  const int64_t max_s = std::min<int64_t>(kMaxSplitCount, (n_ctx + round - 1) / round);
  // default: one round of ~256 workgroups for the matrix-core kernel (one
  // per compute unit); ~2048 for the VALU kernel (8 per compute unit, two
  // resident at a time): measured fastest for long contexts
  int64_t S = splits > 0 ? splits : ((p->mx ? 256 : 2048) + units - 1) / units;
  S = std::max<int64_t>(1, std::min(S, max_s));
  int64_t tps = (n_ctx + S - 1) / S;
  tps = (tps + round - 1) / round * round;
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
  if (p.mx) {
    const dim3 blk(512);
    if (cfg->d == 128) {
      if (p.gk == 4) hipLaunchKernelGGL((k_affine_decode_mx<128, 4>), grid, blk, 0, stream, a);
      else if (p.gk == 2) hipLaunchKernelGGL((k_affine_decode_mx<128, 2>), grid, blk, 0, stream, a);
      else hipLaunchKernelGGL((k_affine_decode_mx<128, 1>), grid, blk, 0, stream, a);
    } else {
      return TQ_ERR_UNSUPPORTED;
    }
    st = aff_last_launch();
  } else {
    st = cfg->d == 128 ? launch_aff_decode<128>(cfg->bits_k, cfg->bits_v, p.gk, a, grid, stream)
                       : launch_aff_decode<256>(cfg->bits_k, cfg->bits_v, p.gk, a, grid, stream);
  }
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
