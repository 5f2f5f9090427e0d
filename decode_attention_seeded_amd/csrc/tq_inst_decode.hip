// Instantiates the split-K decode kernel for one (D, key bits) pair, chosen
// at compile time with -DTQ_D=... -DTQ_BK=... (BK = 16: dense bf16 baseline),
// and exposes one launcher that dispatches over value bits, heads per
// workgroup, QJL and the matrix-core variant.
#include "tq_internal.h"
#include "tq_kernels.h"

#ifndef TQ_D
#error "TQ_D must be defined"
#endif
#ifndef TQ_BK
#error "TQ_BK must be defined"
#endif

#define TQ_CAT2(a, b, c, d) a##b##c##d
#define TQ_CAT(a, b, c, d) TQ_CAT2(a, b, c, d)
#define TQ_LAUNCHER TQ_CAT(launch_decode_d, TQ_D, _k, TQ_BK)

namespace tq {

template <int BV, int GK, bool QJL>
static int go(int mx, const DecodeArgs& a, dim3 grid, hipStream_t st) {
#if TQ_BK == 16
  if (mx) return TQ_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((k_decode<TQ_D, TQ_BK, BV, GK, QJL>), grid, dim3(TQ_D / 32 * 64), 0, st,
                     a, a.qp, a.qq);
#else
  if (mx) {
    const dim3 block(64 * mx_waves(TQ_D));
    if constexpr (!QJL) {
      if (a.append == 2) {              // chunked append: its own instantiation
        if (a.norm_f16)
          hipLaunchKernelGGL((k_decode_mx<TQ_D, TQ_BK, BV, GK, false, true, true>), grid, block,
                             0, st, a);
        else
          hipLaunchKernelGGL((k_decode_mx<TQ_D, TQ_BK, BV, GK, false, false, true>), grid,
                             block, 0, st, a);
        return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
      }
    }
    if (a.norm_f16)
      hipLaunchKernelGGL((k_decode_mx<TQ_D, TQ_BK, BV, GK, QJL, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_mx<TQ_D, TQ_BK, BV, GK, QJL, false>), grid, block, 0, st, a);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
  }
  hipLaunchKernelGGL((k_decode_pk<TQ_D, TQ_BK, BV, GK, QJL>), grid, dim3(TQ_D / 32 * 64), 0,
                     st, a, reinterpret_cast<const uint32_t*>(a.qp), a.qq);
#endif
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int BV, int GK>
static int go_q(int qjl, int mx, const DecodeArgs& a, dim3 grid, hipStream_t st) {
#if TQ_BK == 16
  (void)qjl;
  return go<BV, GK, false>(mx, a, grid, st);
#else
  return qjl ? go<BV, GK, true>(mx, a, grid, st) : go<BV, GK, false>(mx, a, grid, st);
#endif
}

template <int BV>
static int go_g(int gk, int qjl, int mx, const DecodeArgs& a, dim3 grid, hipStream_t st) {
  switch (gk) {
    case 1: return go_q<BV, 1>(qjl, mx, a, grid, st);
    case 2: return go_q<BV, 2>(qjl, mx, a, grid, st);
    case 4: return go_q<BV, 4>(qjl, mx, a, grid, st);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

int TQ_LAUNCHER(int bv, int gk, int qjl, int mx, const DecodeArgs& a, dim3 grid,
                hipStream_t st) {
#if TQ_BK == 16
  return bv == 16 ? go_g<16>(gk, 0, mx, a, grid, st) : TQ_ERR_UNSUPPORTED;
#else
  switch (bv) {
    case 2: return go_g<2>(gk, qjl, mx, a, grid, st);
    case 3: return go_g<3>(gk, qjl, mx, a, grid, st);
    case 4: return go_g<4>(gk, qjl, mx, a, grid, st);
    default: return TQ_ERR_UNSUPPORTED;
  }
#endif
}

}  // namespace tq
