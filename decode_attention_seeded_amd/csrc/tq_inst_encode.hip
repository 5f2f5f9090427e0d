// Instantiates the persistent K/V encode kernel for one (D, key bits) pair,
// chosen at compile time with -DTQ_D=... -DTQ_BK=..., and exposes one
// launcher that dispatches over value bits, QJL and the input dtype.
#include <algorithm>

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
#define TQ_LAUNCHER TQ_CAT(launch_encode_d, TQ_D, _k, TQ_BK)

namespace tq {

namespace {

constexpr int kEncodeBlock = 256;

// Workgroups of `kern` that fit on the whole device at once (occupancy per
// CU from the kernel's register and LDS use, times the CU count).
int resident_blocks(const void* kern) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kEncodeBlock, 0) !=
      hipSuccess)
    return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

template <int BV, bool QJL, int DT>
int go(const EncodeArgs& a, hipStream_t st) {
  constexpr int IW = DT == 0 ? 4 : 2;
  constexpr int P = TQ_D / 32;
  constexpr int64_t RPW = 64 / P;
  constexpr int WPB = kEncodeBlock / 64;
  auto kern = k_encode<TQ_D, TQ_BK, BV, QJL, DT>;
  static const int resident = resident_blocks(reinterpret_cast<const void*>(kern));
  if (resident <= 0) return TQ_ERR_HIP;

  // work items are numbered in 32 bits: split the (batch, head) range so
  // that one launch has fewer than 2^30 of them
  const int64_t groups = (a.n_new + RPW - 1) / RPW;
  if (2 * groups >= (int64_t(1) << 30)) return TQ_ERR_ARG;
  const int64_t bh_per_launch = std::max<int64_t>(1, (int64_t(1) << 29) / groups);
  const int64_t es = IW;
  for (int64_t bh0 = 0; bh0 < a.BH; bh0 += bh_per_launch) {
    EncodeArgs c = a;
    const int64_t nb = std::min<int64_t>(bh_per_launch, a.BH - bh0);
    c.BH = int(nb);
    const int64_t bits[2] = {TQ_BK, BV};
    const int64_t nbytes = a.norm_f16 ? 2 : 4;
    for (int z = 0; z < 2; ++z) {
      c.x[z] = static_cast<const uint8_t*>(a.x[z]) + bh0 * a.n_new * TQ_D * es;
      c.codes[z] = a.codes[z] + bh0 * a.capacity * (TQ_D * bits[z] / 8);
      c.norms[z] = static_cast<uint8_t*>(a.norms[z]) + bh0 * a.capacity * nbytes;
    }
    if (QJL) {
      c.qbits = a.qbits + bh0 * a.capacity * (TQ_D / 8);
      c.rnorm = a.rnorm + bh0 * a.capacity;
    }
    const int64_t items = 2 * nb * groups;
    const int64_t want = (items + WPB - 1) / WPB;
    const unsigned blocks = unsigned(std::min<int64_t>(want, resident));
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kEncodeBlock), 0, st, c);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  }
  return TQ_OK;
}

template <int BV, bool QJL>
int go_w(const EncodeArgs& a, hipStream_t st) {
  switch (a.in_dtype) {
    case 0: return go<BV, QJL, 0>(a, st);
    case 1: return go<BV, QJL, 1>(a, st);
    default: return go<BV, QJL, 2>(a, st);
  }
}

template <int BV>
int go_q(bool qjl, const EncodeArgs& a, hipStream_t st) {
  return qjl ? go_w<BV, true>(a, st) : go_w<BV, false>(a, st);
}

}  // namespace

int TQ_LAUNCHER(int bv, bool qjl, const EncodeArgs& a, hipStream_t st) {
  switch (bv) {
    case 2: return go_q<2>(qjl, a, st);
    case 3: return go_q<3>(qjl, a, st);
    case 4: return go_q<4>(qjl, a, st);
    default: return TQ_ERR_UNSUPPORTED;
  }
}

}  // namespace tq
