// Causal multi-query (prefill) attention over the packed cache on the
// matrix cores (gfx950, wave64). Instantiated by tq_inst_prefill.hip.
//
// A chunk of n_q new tokens has been appended to the cache; query i of the
// chunk sits at position n_ctx - n_q + i and attends to tokens 0 .. that
// position. With G query heads per KV head this is a dense contraction of
// (n_q * G) query rows against the dequantized cache, so both products run
// as v_mfma_f32_16x16x16_f16 on fp16 operands with fp32 accumulation.
//
// Workgroup: 4 waves, 64 query rows (row r = i * G + g of one KV head), wave
// w owns rows 16w .. 16w + 15. Per 64-token tile:
//   dequant  all 256 threads: thread (token t = tid / 4, part = tid % 4)
//            decodes coordinates [part * d/4, (part + 1) * d/4) of token t's
//            key (pair-table lookups, row-major fp16 tile) and value
//            (transposed fp16 tile), and the per-token scales.
//   scores   S^T = K_hat Q'^T per 16-token block: A = 4 coordinates of a
//            key row (8-byte LDS read), B = the lane's query row quad (held
//            in VGPRs). The output layout (lane (kq, col) holds tokens
//            4kq .. 4kq + 3 of query row col) is exactly the A layout of
//            P V_hat, so the weights never leave the registers.
//   softmax  online, in exp2 units, per query row over the 4 lanes that
//            hold it; tokens past the row's position are masked.
//   values   O += P V_hat: A = the lane's 4 weights (times the value norm),
//            B = 4 tokens of one coordinate from the transposed tile.
// Epilogue: O / l, staged per row in LDS, rotated back (R^T) with 16 lanes
// per row and stored as fp32.
#pragma once

#include "tq_device.h"

namespace tq {

struct PrefillArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const void* kn;
  const void* vn;
  const void* q;          // [B][Hq][n_q][D] queries of the chunk
  float* out;             // [B][Hq][n_q][D]
  int64_t capacity, n_ctx, n_q;
  int Hkv, Hq, G;
  int q_dtype;
  int norm_f16;
  float kscale;           // 1 / (sqrt(d) * alpha_k)
  float vscale;           // 1 / (sqrt(d) * alpha_v)
  float qmult;            // scale * log2(e)
  float cbk[16];          // alpha_k * key centroids
  float cbv[16];          // alpha_v * value centroids
  uint32_t sbits[8];      // rotation signs, bit i set when sign i is negative
};

typedef _Float16 pf_h4 __attribute__((ext_vector_type(4)));
typedef float pf_f4 __attribute__((ext_vector_type(4)));

constexpr int pf_max(int a, int b) { return a > b ? a : b; }

template <int D, int BK, int BV>
__global__ void __launch_bounds__(256) k_prefill(PrefillArgs a) {
  static_assert(D == 128 || D == 256, "prefill: d 128 or 256");
  constexpr int TT = 64;                   // tokens per tile
  constexpr int NS = D / 16;               // score k-steps = value coordinate tiles
  constexpr int KS = D + 8;                // key tile row stride (halves)
  constexpr int VS = TT + 8;               // transposed value tile row stride (halves)
  constexpr int CPT = D / 4;               // coordinates per dequant thread
  constexpr int KWD = CPT * BK / 32;       // code dwords per dequant thread
  constexpr int VWD = CPT * BV / 32;
  constexpr int KREC = D * BK / 8;
  constexpr int VREC = D * BV / 8;
  constexpr int KE = 1 << (2 * BK);
  constexpr int VE = 1 << BV;
  constexpr int E = D / 16;                // row elements per lane (16 lanes per row)
  constexpr int TILE_BYTES = TT * KS * 2 + D * VS * 2;
  constexpr int SMEM = pf_max(TILE_BYTES, 64 * D * 4);
  static_assert(64 * KS * 2 <= SMEM, "query staging fits");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ __attribute__((aligned(16))) float tks[TT];
  __shared__ __attribute__((aligned(16))) float tnv[TT];
  __shared__ uint32_t kpair[KE];
  __shared__ uint16_t vone[VE];
  _Float16* ktile = reinterpret_cast<_Float16*>(smem);
  _Float16* vtile = reinterpret_cast<_Float16*>(smem + TT * KS * 2);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = lane >> 4;
  const int col = lane & 15;
  const int unit = blockIdx.y;
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int64_t R = a.n_q * a.G;
  const int64_t r0 = int64_t(blockIdx.x) * 64;
  const int64_t rec0 = int64_t(unit) * a.capacity;
  const int64_t pos0 = a.n_ctx - a.n_q;

  for (int e = tid; e < KE; e += 256)
    kpair[e] = dev::pack_f16x2(a.cbk[e & ((1 << BK) - 1)], a.cbk[e >> BK]);
  for (int e = tid; e < VE; e += 256)
    vone[e] = __builtin_bit_cast(uint16_t, _Float16(a.cbv[e]));

  // ---------------- the wave's 16 query rows: R q * scale * log2(e), fp16
  _Float16* qst = reinterpret_cast<_Float16*>(smem);
  {
    const int l16 = lane & 15;
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
    const float mult = a.qmult / sqrtf(float(D));
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int m = 16 * wave + 4 * pass + (lane >> 4);
      const int64_t r = r0 + m;
      float v[E];
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = 0.f;
      if (r < R) {
        const int64_t qi = r / a.G, h = int64_t(kvh) * a.G + (r - qi * a.G);
        dev::load_row_part<E>(a.q, a.q_dtype,
                              ((int64_t(b) * a.Hq + h) * a.n_q + qi) * D + l16 * E, v);
      }
#pragma unroll
      for (int i = 0; i < E; ++i) if (smask >> i & 1) v[i] = -v[i];
      dev::fwht16<E, float>(v, l16);
#pragma unroll
      for (int i = 0; i < E; ++i) qst[m * KS + l16 * E + i] = _Float16(v[i] * mult);
    }
  }
  __syncthreads();
  pf_h4 qb[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qb[s] = *reinterpret_cast<const pf_h4*>(qst + (16 * wave + col) * KS + 16 * s + 4 * kq);

  // the lane's query row (score layout) and its position
  const int64_t my_r = r0 + 16 * wave + col;
  const int64_t my_pos = my_r < R ? pos0 + my_r / a.G : -1;
  const int64_t r_last = (r0 + 63 < R ? r0 + 63 : R - 1);
  const int64_t p_max = pos0 + r_last / a.G;
  const int ntiles = int(p_max / TT) + 1;

  // ---------------- dequant role: token t of the tile, coordinate part
  const int dt = tid >> 2, dpart = tid & 3;
  uint32_t kw[KWD], vw[VWD];
  uint32_t knb = 0, vnb = 0;
  auto fetch = [&](int n) {
    const int64_t tok = int64_t(n) * TT + dt;
    const bool ok = tok < a.n_ctx;
    const uint32_t* kp =
        reinterpret_cast<const uint32_t*>(a.kc + (rec0 + tok) * KREC) + dpart * KWD;
    const uint32_t* vp =
        reinterpret_cast<const uint32_t*>(a.vc + (rec0 + tok) * VREC) + dpart * VWD;
#pragma unroll
    for (int j = 0; j < KWD; ++j) kw[j] = 0u;
#pragma unroll
    for (int j = 0; j < VWD; ++j) vw[j] = 0u;
    knb = vnb = 0u;
    if (ok) {                            // rows past the context are never read
#pragma unroll
      for (int j = 0; j < KWD; ++j) kw[j] = kp[j];
#pragma unroll
      for (int j = 0; j < VWD; ++j) vw[j] = vp[j];
      if (dpart == 0) {
        if (a.norm_f16) {
          knb = static_cast<const uint16_t*>(a.kn)[rec0 + tok];
          vnb = static_cast<const uint16_t*>(a.vn)[rec0 + tok];
        } else {
          knb = static_cast<const uint32_t*>(a.kn)[rec0 + tok];
          vnb = static_cast<const uint32_t*>(a.vn)[rec0 + tok];
        }
      }
    }
  };

  float m_run = -1e30f, l_run = 0.f;
  pf_f4 o[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) o[j] = pf_f4{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  for (int n = 0; n < ntiles; ++n) {
    __syncthreads();                    // the previous tile (or q staging) is consumed
    {
      uint32_t pk[CPT / 2];
#pragma unroll
      for (int c = 0; c < CPT / 2; ++c) pk[c] = kpair[dev::field<2 * BK>(kw, c)];
      uint4* kd = reinterpret_cast<uint4*>(ktile + dt * KS + dpart * CPT);
#pragma unroll
      for (int c = 0; c < CPT / 8; ++c)
        kd[c] = make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]);
      uint16_t* vt = reinterpret_cast<uint16_t*>(vtile);
#pragma unroll
      for (int c = 0; c < CPT; ++c) vt[(dpart * CPT + c) * VS + dt] = vone[dev::field<BV>(vw, c)];
      if (dpart == 0) {
        tks[dt] = (a.norm_f16 ? dev::f16_to_f32(knb) : __uint_as_float(knb)) * a.kscale;
        tnv[dt] = (a.norm_f16 ? dev::f16_to_f32(vnb) : __uint_as_float(vnb)) * a.vscale;
      }
    }
    if (n + 1 < ntiles) fetch(n + 1);
    __syncthreads();

    // ---------------- scores S^T (tokens x rows), scaled and masked
    float sc[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      pf_f4 acc = pf_f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const pf_h4 ka =
            *reinterpret_cast<const pf_h4*>(ktile + (16 * tb + col) * KS + 16 * s + 4 * kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(ka, qb[s], acc, 0, 0, 0);
      }
      const float4 ks = *reinterpret_cast<const float4*>(tks + 16 * tb + 4 * kq);
      const float kss[4] = {ks.x, ks.y, ks.z, ks.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = int64_t(n) * TT + 16 * tb + 4 * kq + i;
        sc[tb][i] = tok <= my_pos ? acc[i] * kss[i] : -INFINITY;
        mt = fmaxf(mt, sc[tb][i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    pf_h4 pa[4];
    float ls = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float4 nv = *reinterpret_cast<const float4*>(tnv + 16 * tb + 4 * kq);
      const float nvs[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[tb][i] - m_new);
        ls += p;
        pa[tb][i] = _Float16(p * nvs[i]);
      }
    }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;

    // ---------------- O = O * alpha + P V_hat (rows 4kq + i of the wave)
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kq + i);
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[j][i] *= al[i];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const pf_h4 vb =
            *reinterpret_cast<const pf_h4*>(vtile + (16 * j + col) * VS + 16 * tb + 4 * kq);
        o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa[tb], vb, o[j], 0, 0, 0);
      }
    }
  }

  // ---------------- O / l, then R^T per row, fp32 out
  float il[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = __shfl(l_run, 4 * kq + i);
    il[i] = l > 0.f ? 1.f / l : 0.f;
  }
  __syncthreads();                      // the tiles are dead: stage rows there
  float* ost = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) ost[(16 * wave + 4 * kq + i) * D + 16 * j + col] = o[j][i] * il[i];
  __syncthreads();
  {
    const int l16 = lane & 15;
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
    const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int m = 16 * wave + 4 * pass + (lane >> 4);
      const int64_t r = r0 + m;
      float v[E];
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = ost[m * D + l16 * E + i];
      dev::fwht16<E, float>(v, l16);
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = (smask >> i & 1) ? -v[i] * nn : v[i] * nn;
      if (r < R) {
        const int64_t qi = r / a.G, h = int64_t(kvh) * a.G + (r - qi * a.G);
        float4* dst = reinterpret_cast<float4*>(
            a.out + ((int64_t(b) * a.Hq + h) * a.n_q + qi) * D + l16 * E);
#pragma unroll
        for (int k = 0; k < E / 4; ++k)
          dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
      }
    }
  }
}

}  // namespace tq
