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
//   dequant  keys: lane = token, a wave decodes one quarter of every
//            token's coordinates (pair-table lookups, 16-byte row stores
//            into a row-major fp16 tile). Values: lane = 4 consecutive
//            tokens x 8 coordinates (one octet of their codes); a lookup in
//            a table of fp16 pairs indexed by the codes of two tokens gives
//            two tokens' values of one coordinate, so each coordinate of the
//            4 tokens is one 8-byte store into the transposed tile. Each
//            value enters the tile times its token's norm (and a per-tile
//            power of two), each key scale carries the query rows' power of
//            two. With 8 waves, waves 0-3 take the keys and 4-7 the values;
//            with 4, each wave both.
//   scores   S^T = K_hat Q'^T per 16-token block: A = 8 coordinates of a key
//            row (16-byte LDS read), B = the lane's query row (VGPRs). The
//            output lane (kq, col) holds tokens 4kq .. 4kq + 3 of the block
//            for query row col.
//   softmax  online, in exp2 units, per query row over the 4 lanes that
//            hold it: one fma gives score minus running max, tokens past
//            the row's position are masked, the max is raised lazily, and
//            the fp16 weights 2^t also feed the row sums (dot2).
//   values   O += P V_hat per 32 tokens: the lane's 8 weights of blocks 2b
//            and 2b + 1 are the A operand as they are; the value tile
//            stores its token columns in that order
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
  static_assert(BV >= 2 && BV <= 4, "prefill: 2 to 4 value bits");
  constexpr int W = pf_waves(D);           // waves
  constexpr int RB = pf_row_blocks(D, QJL);  // blocks of 16 query rows per wave
  constexpr int NR = pf_rows(D, QJL);      // query rows per workgroup
  constexpr int NT = 64 * W;
  constexpr int TT = 64;                   // tokens per tile
  constexpr int NS = D / 16;               // value coordinate tiles of 16
  constexpr int NK = D / 32;               // score k-steps of 32 coordinates
  constexpr int KS = D + 8;                // key tile row stride (halves)
  constexpr int VS = TT + 8;               // transposed value tile row stride (halves)
  constexpr int CPT = D / 4;               // key coordinates per dequant lane
  constexpr int KWD = CPT * BK / 32;       // key code dwords per dequant lane
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
  __shared__ __attribute__((aligned(16))) float tks[2][TT];     // key scale per token
  __shared__ __attribute__((aligned(16))) float trho[QJL ? 2 : 1][TT];
  __shared__ int texp[2];                  // the value tile's power of two
  __shared__ float wmax[W];
  __shared__ uint32_t kpair[KE];
  // fp16 values of codes (e & (VE - 1), e >> BV) as one pair, token order
  __shared__ __attribute__((aligned(16))) uint32_t vpair[VE * VE];
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
  for (int e = tid; e < VE * VE; e += NT)
    vpair[e] = dev::pack_f16x2(a.cbv[e & (VE - 1)], a.cbv[e >> BV]);

  // ---------------- the wave's 16 RB query rows: R q * scale * log2(e),
  // fp16. A first pass finds the largest element of the workgroup's rows
  // (q' and q''); the second stores them scaled by one power of two 2^-qe
  // that puts it near 2^10 (no fp16 overflow or subnormals). The key scales
  // carry 2^qe back in fp32.
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
    if (lane == 0) wmax[wave] = vmax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < W; ++w) vmax = fmaxf(vmax, wmax[w]);
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

  // ---------------- dequant roles. Keys: lane = token of the tile, wave =
  // quarter of the coordinates. Values: value lane vl (0 .. 255 over the
  // value waves) takes tokens 4 vq .. 4 vq + 3 and the coordinate octets
  // vo, vo + 16, ... Tokens past the context load the last token's record
  // (in bounds; every score they enter is masked).
  const int dt = lane;
  const int dpart = W == 8 ? (wave & 3) : wave;
  const bool do_k = W == 4 || wave < 4;
  const bool do_v = W == 4 || wave >= 4;     // wave-uniform
  constexpr int SWD = QJL ? CPT / 32 : 1;   // QJL sign words per dequant lane
  constexpr int VO = D / 128;               // value octets per lane
  constexpr int VXW = BV == 3 ? 2 : 1;      // code dwords per (octet, token)
  const int vl = (wave & 3) * 64 + lane;
  const int vq = vl & 15, vo = vl >> 4;
  const int last = int(a.n_ctx - 1);
  const uint8_t* kbase = a.kc + rec0 * KREC + dpart * KWD * 4;
  const uint8_t* vbase = a.vc + rec0 * VREC;
  uint32_t kw[KWD], sw[SWD], vx[VO][4][VXW];
  uint32_t knb = 0, rnb = 0, vnb[4];
  auto norm_at = [&](const void* np, int t) -> uint32_t {
    return a.norm_f16 ? uint32_t(static_cast<const uint16_t*>(np)[rec0 + t])
                      : static_cast<const uint32_t*>(np)[rec0 + t];
  };
  auto fetch = [&](int n) {
    if (do_k) {
      const int t = min(n * TT + dt, last);
      const uint32_t* kp = reinterpret_cast<const uint32_t*>(kbase + int64_t(t) * KREC);
#pragma unroll
      for (int j = 0; j < KWD; ++j) kw[j] = kp[j];
      if (dpart == 0) knb = norm_at(a.kn, t);
      if constexpr (QJL) {
        const uint32_t* sp = a.kq + (rec0 + t) * (D / 32) + dpart * SWD;
#pragma unroll
        for (int j = 0; j < SWD; ++j) sw[j] = sp[j];
        if (dpart == 0) rnb = a.kr[rec0 + t];
      }
    }
    if (do_v) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = min(n * TT + 4 * vq + u, last);
        const uint32_t* rp = reinterpret_cast<const uint32_t*>(vbase + int64_t(t) * VREC);
#pragma unroll
        for (int o = 0; o < VO; ++o) {
          const int oct = vo + 16 * o;
          if constexpr (BV == 3) {
            // bits 24 oct .. 24 oct + 23: dword i, and i + 1 when they
            // straddle (i + 1 stays inside the record then)
            const int i = (3 * oct) >> 2;
            vx[o][u][0] = rp[i];
            vx[o][u][1] = rp[i + 1 < VREC / 4 ? i + 1 : i];
          } else {
            vx[o][u][0] = rp[BV == 4 ? oct : oct >> 1];
          }
        }
        vnb[u] = norm_at(a.vn, t);
      }
    }
  };

  float m_run[RB], l_run[RB];
  int vexp = 0;                         // accumulators carry 2^-vexp (value tiles)
  int vexp_d = 0;                       // the value waves' running choice of it
  float vmul = a.vscale;                // vscale * 2^-vexp_d
  pf_f4 o[RB][NS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = 0.f;                    // set by the first tile
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
        tks[buf][dt] =
            (a.norm_f16 ? dev::f16_to_f32(knb) : __uint_as_float(knb)) * (a.kscale * qsc);
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
        if (dpart == 0) trho[buf][dt] = dev::f16_to_f32(rnb) * (a.qjl_c * qsc);
      }
    }
    if (do_v) {
      // Values enter the tile times their norm: nv * vscale * 2^-vexp_d,
      // with one power of two per tile that keeps the tile's largest norm
      // within [2^-6, 2^6] (moved only when a tile leaves that band: a norm
      // above it, or all below). Every value wave holds all 64 tokens, so
      // each takes the same decision.
      float ns[4];
      bool above = false, inside = false;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float nv = a.norm_f16 ? dev::f16_to_f32(vnb[u]) : __uint_as_float(vnb[u]);
        ns[u] = nv * vmul;
        above |= ns[u] > 64.f;
        inside |= ns[u] >= 0.015625f;
      }
      if (__ballot(above) || !__ballot(inside)) {     // wave-uniform, rare
        float mx = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) mx = fmaxf(mx, ldexpf(ns[u], vexp_d));
        mx = dev::dpp_wave_max(mx);
        if (mx > 0.f) {
          const int nexp = ilogbf(mx) - 4;
#pragma unroll
          for (int u = 0; u < 4; ++u) ns[u] = ldexpf(ns[u], vexp_d - nexp);
          vexp_d = nexp;
          vmul = ldexpf(a.vscale, -vexp_d);
        }
      }
      if (vl == 0) texp[buf] = vexp_d;
      const dev::half2_t sc01 = {_Float16(ns[0]), _Float16(ns[1])};
      const dev::half2_t sc23 = {_Float16(ns[2]), _Float16(ns[3])};
      // token t sits at column vcol(t); the quad's 4 tokens are adjacent
      const int t0 = 4 * vq;
      const int vcol = (t0 & 32) | ((t0 >> 2) & 3) << 3 | ((t0 >> 4) & 1) << 2;
      // even coordinates 2j: group j (2 BV bits) of ze holds the codes of
      // the pair's two tokens as one index; odd ones in zo
      constexpr uint32_t M = BV == 4 ? 0x0F0F0F0Fu : BV == 3 ? 0x71C71C7u : 0x33333333u;
      const char* vpb = reinterpret_cast<const char*>(vpair);
#pragma unroll
      for (int o = 0; o < VO; ++o) {
        const int oct = vo + 16 * o;
        uint32_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          x[u] = BV == 3   ? __builtin_amdgcn_alignbit(vx[o][u][1], vx[o][u][0],
                                                       uint32_t(8 * ((3 * oct) & 3)))
                 : BV == 2 ? vx[o][u][0] >> (16 * (oct & 1))
                           : vx[o][u][0];
        uint32_t pv[2][8];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t ze[1] = {(x[2 * p] & M) | ((x[2 * p + 1] << BV) & ~M)};
          const uint32_t zo[1] = {((x[2 * p] >> BV) & M) | (x[2 * p + 1] & ~M)};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pv[p][2 * j] = *reinterpret_cast<const uint32_t*>(
                vpb + dev::bits_at<2 * BV, 2>(ze, 2 * BV * j));
            pv[p][2 * j + 1] = *reinterpret_cast<const uint32_t*>(
                vpb + dev::bits_at<2 * BV, 2>(zo, 2 * BV * j));
          }
        }
        uint2* vt = reinterpret_cast<uint2*>(vtile(buf) + 8 * oct * VS + vcol);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const dev::half2_t v01 = __builtin_bit_cast(dev::half2_t, pv[0][k]) * sc01;
          const dev::half2_t v23 = __builtin_bit_cast(dev::half2_t, pv[1][k]) * sc23;
          vt[k * (VS / 4)] =
              make_uint2(__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23));
        }
      }
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

    // ---------------- scores S^T (tokens x rows) in exp2 units, less the
    // running max: t = ks_t * S (+ rho_t * S_qjl) - m, masked on the tiles
    // that reach past the workgroup's lowest row position
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
      const float kss[4] = {ks.x, ks.y, ks.z, ks.w};
      float rhs[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (QJL) {
        const float4 rh = *reinterpret_cast<const float4*>(&trho[buf][16 * tb + 4 * kq]);
        rhs[0] = rh.x; rhs[1] = rh.y; rhs[2] = rh.z; rhs[3] = rh.w;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t = fmaf(acc[rb][i], kss[i], -m_run[rb]);
          if constexpr (QJL) t = fmaf(acq[rb][i], rhs[i], t);
          sc[rb][tb][i] = t;
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
    // a score exceeds it by more than 2^8, so the weights stay <= 2^8; then
    // the tile's row maxima are taken and the accumulators rescaled. The
    // branch is wave-uniform. The first tile always takes it and sets the
    // max (token 0 is visible to every row; rows past the chunk, masked
    // everywhere, get a finite max and weight 0).
    const bool first = n == 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tm = sc[rb][0][0];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tm = fmaxf(tm, sc[rb][tb][i]);
      if (__ballot(first || tm > 8.f)) {
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        const float delta = fmaxf(tm, first ? -3.0e38f : 0.f);
        const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-delta);
        m_run[rb] += delta;
        l_run[rb] *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * kq + i);
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rb][j][i] *= al[i];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[rb][tb][i] -= delta;
      }
    }
    // the value tile's power of two (the same on every lane)
    const int te = texp[buf];
    if (te != vexp) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[rb][j][i] = ldexpf(o[rb][j][i], vexp - te);
      vexp = te;
    }
    // weights p = 2^t as fp16 (p <= 2^8); the row sums add the same fp16
    // weights (2 per dot), the lane's 16 tokens here and its 4 lanes once
    // after the loop
    pf_h8 pa[RB][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pa[rb][tb >> 1][4 * (tb & 1) + i] = _Float16(__builtin_amdgcn_exp2f(sc[rb][tb][i]));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 w4 = __builtin_bit_cast(uint4, pa[rb][h]);
        l_run[rb] = dev::dot2(w4.x, 0x3C003C00u, l_run[rb]);
        l_run[rb] = dev::dot2(w4.y, 0x3C003C00u, l_run[rb]);
        l_run[rb] = dev::dot2(w4.z, 0x3C003C00u, l_run[rb]);
        l_run[rb] = dev::dot2(w4.w, 0x3C003C00u, l_run[rb]);
      }

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
