// Causal multi-query (prefill) attention over the packed cache on the
// matrix cores (gfx950, wave64). Instantiated by tq_inst_prefill.hip.
//
// A chunk of n_q new tokens has been appended to the cache; query i of the
// chunk sits at position n_ctx - n_q + i and attends to tokens 0 .. that
// position. With G query heads per KV head this is a dense contraction of
// (n_q * G) query rows against the dequantized cache, so both products run
// as v_mfma_f32_16x16x32_f16 on fp16 operands with fp32 accumulation (lane
// (kq, r) of an operand holds k-values 8kq .. 8kq + 7 of row/column r; the
// output lane (kq, c) holds rows 4kq .. 4kq + 3 of column c).
//
// Workgroup: W waves (8 at d = 128, 4 at d = 256), each owning RB blocks of
// 16 query rows (RB = 2 at d = 128, 1 at d = 256; row r = i * G + g of one
// KV head; wave w owns rows 16 RB w .. 16 RB (w + 1) - 1), so every
// dequantized tile serves 16 RB W rows and each operand read serves RB
// blocks. Per
// 64-token tile, double-buffered in LDS so that the next tile's dequant
// overlaps this tile's products (one barrier per tile):
//   dequant  lane = token; a wave decodes one quarter of the coordinates
//            of every token's key (pair-table lookups, row-major fp16 tile)
//            or value (transposed fp16 tile, one row store per coordinate),
//            and the per-token scales. With 8 waves, waves 0-3 take the
//            keys and 4-7 the values; with 4, each wave both.
//   scores   S^T = K_hat Q'^T per 16-token block: A = 8 coordinates of a key
//            row (16-byte LDS read), B = the lane's query row (VGPRs). The
//            output lane (kq, col) holds tokens 4kq .. 4kq + 3 of the block
//            for query row col.
//   softmax  online, in exp2 units, per query row over the 4 lanes that
//            hold it; tokens past the row's position are masked.
//   values   O += P V_hat per 32 tokens: the lane's 8 weights (times the
//            value norm) of blocks 2b and 2b + 1 are the A operand as they
//            are; the value tile stores its token columns in that order
//            (token 32b + 16h + 4q + i at column 32b + 8q + 4h + i), so the
//            B operand is one 16-byte read.
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
  const uint32_t* kq;     // QJL sign plane (d/32 words per record), QJL only
  const uint16_t* kr;     // QJL residual norms (fp16), QJL only
  float qjl_c;            // sqrt(pi / (2 d))
  uint32_t qsbits[8];     // QJL rotation signs, same layout
};

typedef _Float16 pf_h8 __attribute__((ext_vector_type(8)));
typedef float pf_f4 __attribute__((ext_vector_type(4)));

constexpr int pf_max(int a, int b) { return a > b ? a : b; }

constexpr int pf_waves(int d) { return d == 128 ? 8 : 4; }
constexpr int pf_row_blocks(int d, bool qjl) { return d == 128 && !qjl ? 2 : 1; }
constexpr int pf_rows(int d, bool qjl) { return 16 * pf_waves(d) * pf_row_blocks(d, qjl); }

// QJL: the sign dot sum_i q''_i sigma_i of every (row, token) is a second
// score product of the same shape, A = the key's signs as fp16 +-1 (a third
// LDS tile written with the keys), B = the row's q'' = R_2 q'; the score is
// ks_t * S + rho_t * S_qjl with rho_t = ||r_t|| sqrt(pi / (2d)).
template <int D, int BK, int BV, bool QJL>
__global__ void __launch_bounds__(64 * pf_waves(D)) k_prefill(PrefillArgs a) {
  static_assert(D == 128 || D == 256, "prefill: d 128 or 256");
  constexpr int W = pf_waves(D);           // waves
  constexpr int RB = pf_row_blocks(D, QJL);  // blocks of 16 query rows per wave
  constexpr int NR = pf_rows(D, QJL);      // query rows per workgroup
  constexpr int NT = 64 * W;
  constexpr int TT = 64;                   // tokens per tile
  constexpr int NS = D / 16;               // value coordinate tiles of 16
  constexpr int NK = D / 32;               // score k-steps of 32 coordinates
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
  constexpr int KT_BYTES = TT * KS * 2;
  constexpr int VT_BYTES = D * VS * 2;
  constexpr int TILE_BYTES = KT_BYTES + VT_BYTES + (QJL ? KT_BYTES : 0);
  constexpr int QST_BYTES = NR * KS * 2 * (QJL ? 2 : 1);
  // two tile buffers (the next tile is decoded while this one is used)
  // where they fit, else one with a barrier on each side of the decode
  constexpr int NBUF = 2 * TILE_BYTES + 4096 <= 152 * 1024 ? 2 : 1;
  constexpr int SMEM = pf_max(NBUF * TILE_BYTES, pf_max(NR * D * 4, QST_BYTES));
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ __attribute__((aligned(16))) float tks[2][TT];
  __shared__ __attribute__((aligned(16))) float tnv[2][TT];
  __shared__ __attribute__((aligned(16))) float trho[QJL ? 2 : 1][TT];
  __shared__ uint32_t kpair[KE];
  __shared__ uint16_t vone[VE];
  auto ktile = [&](int buf) { return reinterpret_cast<_Float16*>(smem + buf * TILE_BYTES); };
  auto vtile = [&](int buf) {
    return reinterpret_cast<_Float16*>(smem + buf * TILE_BYTES + KT_BYTES);
  };
  auto stile = [&](int buf) {
    return reinterpret_cast<_Float16*>(smem + buf * TILE_BYTES + KT_BYTES + VT_BYTES);
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = lane >> 4;
  const int col = lane & 15;
  const int unit = blockIdx.y;
  const int b = unit / a.Hkv;
  const int kvh = unit - b * a.Hkv;
  const int64_t R = a.n_q * a.G;
  const int64_t r0 = int64_t(blockIdx.x) * NR;
  const int64_t rec0 = int64_t(unit) * a.capacity;
  const int64_t pos0 = a.n_ctx - a.n_q;

  for (int e = tid; e < KE; e += NT)
    kpair[e] = dev::pack_f16x2(a.cbk[e & ((1 << BK) - 1)], a.cbk[e >> BK]);
  for (int e = tid; e < VE; e += NT)
    vone[e] = __builtin_bit_cast(uint16_t, _Float16(a.cbv[e]));

  // ---------------- the wave's 16 query rows: R q * scale * log2(e), fp16.
  // A first pass finds the largest element of the wave's rows (q' and q''),
  // the second stores them scaled by one power of two 2^-qe that puts it
  // near 2^10 (no fp16 overflow or subnormals); the scores undo it in fp32.
  _Float16* qst = reinterpret_cast<_Float16*>(smem);
  int qe = 0;
  {
    const int l16 = lane & 15;
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
    const float mult = a.qmult / sqrtf(float(D));
    auto row = [&](int pass, float (&v)[E], float (&v2)[E]) {
      const int64_t r = r0 + 16 * RB * wave + 4 * pass + (lane >> 4);
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
      for (int i = 0; i < E; ++i) v[i] *= mult;
      if constexpr (QJL) {
        // q'' = R_2 q' from the fp32 q'
        const uint32_t qmask = dev::bitmap_bits(a.qsbits, l16 * E, E);
#pragma unroll
        for (int i = 0; i < E; ++i) v2[i] = (qmask >> i & 1) ? -v[i] : v[i];
        dev::fwht16<E, float>(v2, l16);
        const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
        for (int i = 0; i < E; ++i) v2[i] *= nn;
      }
    };
    float vmax = 0.f;
#pragma unroll 1
    for (int pass = 0; pass < 4 * RB; ++pass) {
      float v[E], v2[E];
      row(pass, v, v2);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        vmax = fmaxf(vmax, fabsf(v[i]));
        if constexpr (QJL) vmax = fmaxf(vmax, fabsf(v2[i]));
      }
    }
    vmax = dev::wave_max(vmax);
    qe = vmax > 0.f ? ilogbf(vmax) - 10 : 0;
#pragma unroll 1
    for (int pass = 0; pass < 4 * RB; ++pass) {
      const int m = 16 * RB * wave + 4 * pass + (lane >> 4);
      float v[E], v2[E];
      row(pass, v, v2);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        qst[m * KS + l16 * E + i] = _Float16(ldexpf(v[i], -qe));
        if constexpr (QJL) qst[(NR + m) * KS + l16 * E + i] = _Float16(ldexpf(v2[i], -qe));
      }
    }
  }
  const float qsc = ldexpf(1.f, qe);     // undoes the query rows' power of two
  __syncthreads();
  pf_h8 qb[RB][NK];
  pf_h8 qb2[QJL ? RB : 1][QJL ? NK : 1];
  int64_t my_pos[RB];                   // the lane's query rows (score layout)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = 16 * (RB * wave + rb) + col;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      qb[rb][s] = *reinterpret_cast<const pf_h8*>(qst + m * KS + 32 * s + 8 * kq);
      if constexpr (QJL)
        qb2[rb][s] = *reinterpret_cast<const pf_h8*>(qst + (NR + m) * KS + 32 * s + 8 * kq);
    }
    my_pos[rb] = r0 + m < R ? pos0 + (r0 + m) / a.G : -1;
  }
  const int64_t r_last = (r0 + NR - 1 < R ? r0 + NR - 1 : R - 1);
  const int64_t p_max = pos0 + r_last / a.G;
  const int64_t p_min = pos0 + r0 / a.G;  // tiles wholly at or before it need no mask
  const int ntiles = int(p_max / TT) + 1;

  // ---------------- dequant role: lane = token of the tile, wave = quarter
  // of the coordinates (of the keys, the values, or both)
  const int dt = lane;
  const int dpart = W == 8 ? (wave & 3) : wave;
  const bool do_k = W == 4 || wave < 4;
  const bool do_v = W == 4 || wave >= 4;     // wave-uniform
  constexpr int SWD = QJL ? CPT / 32 : 1;   // QJL sign words per dequant lane
  uint32_t kw[KWD], vw[VWD], sw[SWD];
  uint32_t knb = 0, vnb = 0, rnb = 0;
  auto fetch = [&](int n) {
    const int64_t tok = int64_t(n) * TT + dt;
    const bool ok = tok < a.n_ctx;
#pragma unroll
    for (int j = 0; j < KWD; ++j) kw[j] = 0u;
#pragma unroll
    for (int j = 0; j < VWD; ++j) vw[j] = 0u;
#pragma unroll
    for (int j = 0; j < SWD; ++j) sw[j] = 0u;
    knb = vnb = rnb = 0u;
    if (!ok) return;                     // rows past the context are never read
    if (do_k) {
      const uint32_t* kp =
          reinterpret_cast<const uint32_t*>(a.kc + (rec0 + tok) * KREC) + dpart * KWD;
#pragma unroll
      for (int j = 0; j < KWD; ++j) kw[j] = kp[j];
      if (dpart == 0)
        knb = a.norm_f16 ? uint32_t(static_cast<const uint16_t*>(a.kn)[rec0 + tok])
                         : static_cast<const uint32_t*>(a.kn)[rec0 + tok];
      if constexpr (QJL) {
        const uint32_t* sp = a.kq + (rec0 + tok) * (D / 32) + dpart * SWD;
#pragma unroll
        for (int j = 0; j < SWD; ++j) sw[j] = sp[j];
        if (dpart == 0) rnb = a.kr[rec0 + tok];
      }
    }
    if (do_v) {
      const uint32_t* vp =
          reinterpret_cast<const uint32_t*>(a.vc + (rec0 + tok) * VREC) + dpart * VWD;
#pragma unroll
      for (int j = 0; j < VWD; ++j) vw[j] = vp[j];
      if (dpart == 0)
        vnb = a.norm_f16 ? uint32_t(static_cast<const uint16_t*>(a.vn)[rec0 + tok])
                         : static_cast<const uint32_t*>(a.vn)[rec0 + tok];
    }
  };

  float m_run[RB], l_run[RB];
  int vexp = 0;                         // value norms carry 2^-vexp (below)
  pf_f4 o[RB][NS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -1e30f;
    l_run[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) o[rb][j] = pf_f4{0.f, 0.f, 0.f, 0.f};
  }

  // dequantized tile of the fetched words into LDS buffer `buf`
  auto put = [&](int buf) {
    if (do_k) {
      uint32_t pk[CPT / 2];
#pragma unroll
      for (int c = 0; c < CPT / 2; ++c) pk[c] = kpair[dev::field<2 * BK>(kw, c)];
      uint4* kd = reinterpret_cast<uint4*>(ktile(buf) + dt * KS + dpart * CPT);
#pragma unroll
      for (int c = 0; c < CPT / 8; ++c)
        kd[c] = make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]);
      if (dpart == 0)
        tks[buf][dt] = (a.norm_f16 ? dev::f16_to_f32(knb) : __uint_as_float(knb)) * a.kscale;
      if constexpr (QJL) {
        // sign bit set -> -1: the fp16 pair 0x3C00 | bit << 15 per coordinate
        uint32_t ps[CPT / 2];
#pragma unroll
        for (int c = 0; c < CPT / 2; ++c) {
          const uint32_t two = (sw[c >> 4] >> (2 * (c & 15))) & 3u;
          ps[c] = 0x3C003C00u | (two & 1u) << 15 | (two & 2u) << 30;
        }
        uint4* sd = reinterpret_cast<uint4*>(stile(buf) + dt * KS + dpart * CPT);
#pragma unroll
        for (int c = 0; c < CPT / 8; ++c)
          sd[c] = make_uint4(ps[4 * c], ps[4 * c + 1], ps[4 * c + 2], ps[4 * c + 3]);
        if (dpart == 0) trho[buf][dt] = dev::f16_to_f32(rnb) * a.qjl_c;
      }
    }
    if (do_v) {
      uint16_t* vt = reinterpret_cast<uint16_t*>(vtile(buf));
      const int vcol = (dt & 32) | ((dt >> 2) & 3) << 3 | ((dt >> 4) & 1) << 2 | (dt & 3);
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        vt[(dpart * CPT + c) * VS + vcol] = vone[dev::field<BV>(vw, c)];
      if (dpart == 0)
        tnv[buf][dt] = (a.norm_f16 ? dev::f16_to_f32(vnb) : __uint_as_float(vnb)) * a.vscale;
    }
  };

  fetch(0);
  __syncthreads();                      // every wave has its query rows: staging is free
  put(0);
  if (ntiles > 1) fetch(1);
  __syncthreads();                      // tile 0 is in place
  for (int n = 0; n < ntiles; ++n) {
    const int buf = NBUF == 2 ? (n & 1) : 0;
    // the next tile goes to the other buffer, whose last readers finished
    // before the barrier that ended the previous iteration
    if (NBUF == 2 && n + 1 < ntiles) {
      put(buf ^ 1);
      if (n + 2 < ntiles) fetch(n + 2);
    }
    const _Float16* kt = ktile(buf);
    const _Float16* vtl = vtile(buf);
    const _Float16* stl = stile(buf);

    // ---------------- scores S^T (tokens x rows), scaled (exp2 units) and
    // masked on the tiles that reach past the workgroup's lowest row position
    const bool masked = int64_t(n) * TT + TT - 1 > p_min;   // workgroup-uniform
    float sc[RB][4][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      pf_f4 acc[RB], acq[QJL ? RB : 1];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb] = pf_f4{0.f, 0.f, 0.f, 0.f};
        if constexpr (QJL) acq[rb] = pf_f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const pf_h8 ka =
            *reinterpret_cast<const pf_h8*>(kt + (16 * tb + col) * KS + 32 * s + 8 * kq);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[rb][s], acc[rb], 0, 0, 0);
        if constexpr (QJL) {
          const pf_h8 sa =
              *reinterpret_cast<const pf_h8*>(stl + (16 * tb + col) * KS + 32 * s + 8 * kq);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acq[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, qb2[rb][s], acq[rb], 0, 0, 0);
        }
      }
      const float4 ks = *reinterpret_cast<const float4*>(&tks[buf][16 * tb + 4 * kq]);
      const float kss[4] = {ks.x * qsc, ks.y * qsc, ks.z * qsc, ks.w * qsc};
      float rhs[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (QJL) {
        const float4 rh = *reinterpret_cast<const float4*>(&trho[buf][16 * tb + 4 * kq]);
        rhs[0] = rh.x * qsc; rhs[1] = rh.y * qsc; rhs[2] = rh.z * qsc; rhs[3] = rh.w * qsc;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[rb][i] * kss[i];
          if constexpr (QJL) v = fmaf(acq[rb][i], rhs[i], v);
          sc[rb][tb][i] = v;
        }
    }
    if (masked) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t tok = int64_t(n) * TT + 16 * tb + 4 * kq + i;
            if (tok > my_pos[rb]) sc[rb][tb][i] = -INFINITY;
          }
    }
    // The running max (per row, the same on its 4 lanes) is raised only when
    // a score exceeds it by more than 2^8 (weights stay <= 2^8, which with
    // the value-norm band below keeps the fp16 operands finite): then the
    // tile's row maxima are taken and the accumulators rescaled. The branch
    // is wave-uniform; it always runs on the first tile (m_run = -1e30, so
    // alpha = 0), and a row masked on every token keeps m_run and weight 0.
    pf_h8 pa[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float lim = m_run[rb] + 8.f;
      bool up = false;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) up |= sc[rb][tb][i] > lim;
      if (__ballot(up)) {
        float mt = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[rb][tb][i]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run[rb], mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        m_run[rb] = m_new;
        l_run[rb] *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kq + i);
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rb][j][i] *= al[i];
      }
    }
    float ls[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ls[rb] = 0.f;
    // the weights p * nv (p <= 1) go to fp16: nv carries a workgroup-uniform
    // power of two 2^-vexp that keeps the tile's largest value norm within
    // [2^-6, 2^6], moved (with the accumulators) only when a tile leaves it
    float nvt[4][4];
    float nvmax = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float4 nv = *reinterpret_cast<const float4*>(&tnv[buf][16 * tb + 4 * kq]);
      nvt[tb][0] = ldexpf(nv.x, -vexp);
      nvt[tb][1] = ldexpf(nv.y, -vexp);
      nvt[tb][2] = ldexpf(nv.z, -vexp);
      nvt[tb][3] = ldexpf(nv.w, -vexp);
#pragma unroll
      for (int i = 0; i < 4; ++i) nvmax = fmaxf(nvmax, nvt[tb][i]);
    }
    nvmax = fmaxf(nvmax, __shfl_xor(nvmax, 16));
    nvmax = fmaxf(nvmax, __shfl_xor(nvmax, 32));
    if (nvmax > 64.f || (nvmax > 0.f && nvmax < 0.015625f)) {   // uniform, rare
      const int sh = ilogbf(nvmax) - 4;
      vexp += sh;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) nvt[tb][i] = ldexpf(nvt[tb][i], -sh);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rb][j][i] = ldexpf(o[rb][j][i], -sh);
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float (&nvs)[4] = nvt[tb];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sc[rb][tb][i] - m_run[rb]);
          ls[rb] += p;
          pa[rb][tb >> 1][4 * (tb & 1) + i] = _Float16(p * nvs[i]);
        }
    }
    // the lane's partial row sums (its 16 tokens); the 4 lanes of a row are
    // added once, after the loop
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_run[rb] += ls[rb];

    // ---------------- O += P V_hat (rows 4kq + i of each block)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const pf_h8 vb =
            *reinterpret_cast<const pf_h8*>(vtl + (16 * j + col) * VS + 32 * hb + 8 * kq);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rb][hb], vb, o[rb][j], 0, 0, 0);
      }
    }
    __syncthreads();
    if (NBUF == 1 && n + 1 < ntiles) {  // one buffer: decode between two barriers
      put(0);
      if (n + 2 < ntiles) fetch(n + 2);
      __syncthreads();
    }
  }

  // ---------------- O / l, then R^T per row, fp32 out
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16);
    l_run[rb] += __shfl_xor(l_run[rb], 32);
  }
  __syncthreads();                      // the tiles are dead: stage rows there
  float* ost = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float il[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = __shfl(l_run[rb], 4 * kq + i);
      il[i] = l > 0.f ? ldexpf(1.f / l, vexp) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ost[(16 * (RB * wave + rb) + 4 * kq + i) * D + 16 * j + col] = o[rb][j][i] * il[i];
  }
  __syncthreads();
  {
    const int l16 = lane & 15;
    const uint32_t smask = dev::bitmap_bits(a.sbits, l16 * E, E);
    const float nn = 1.0f / sqrtf(float(D));
#pragma unroll
    for (int pass = 0; pass < 4 * RB; ++pass) {
      const int m = 16 * RB * wave + 4 * pass + (lane >> 4);
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
