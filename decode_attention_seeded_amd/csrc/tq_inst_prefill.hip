// Instantiates the causal prefill kernel for one head dimension, chosen at
// compile time with -DTQ_D=..., and exposes one launcher that dispatches
// over the key and value bit widths.
#include "tq_internal.h"
#include "tq_prefill.h"

#ifndef TQ_D
#error "TQ_D must be defined"
#endif

#define TQ_PCAT2(a, b) a##b
#define TQ_PCAT(a, b) TQ_PCAT2(a, b)
#define TQ_PLAUNCHER TQ_PCAT(launch_prefill_d, TQ_D)

namespace tq {

template <int BK, int BV>
static int go(int qjl, const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if (qjl)
    hipLaunchKernelGGL((k_prefill<TQ_D, BK, BV, true>), grid, dim3(64 * pf_waves(TQ_D)), 0, st,
                       a);
  else
    hipLaunchKernelGGL((k_prefill<TQ_D, BK, BV, false>), grid, dim3(64 * pf_waves(TQ_D)), 0, st,
                       a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int BK>
static int go_v(int bv, int qjl, const PrefillArgs& a, dim3 grid, hipStream_t st) {
  switch (bv) {
    case 2: return go<BK, 2>(qjl, a, grid, st);
    case 3: return go<BK, 3>(qjl, a, grid, st);
    case 4: return go<BK, 4>(qjl, a, grid, st);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

int TQ_PLAUNCHER(int bk, int bv, int qjl, const PrefillArgs& a, dim3 grid, hipStream_t st) {
  switch (bk) {
    case 2: return go_v<2>(bv, qjl, a, grid, st);
    case 3: return go_v<3>(bv, qjl, a, grid, st);
    case 4: return go_v<4>(bv, qjl, a, grid, st);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

}  // namespace tq
