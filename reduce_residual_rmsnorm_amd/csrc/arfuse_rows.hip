// Row-kernel instances for one rank count ARFUSE_N (set by the build):
// every VPT in {1, 2, 4, 8} x {plain, LL} x epilogue mask.

#include "arfuse_device.hpp"

#ifndef ARFUSE_N
#error "build with -DARFUSE_N=<1..8>"
#endif

#define ARFUSE_CAT2(a, b) a##b
#define ARFUSE_CAT(a, b) ARFUSE_CAT2(a, b)

namespace arfuse_detail {
namespace {

template <int N, int VPT, bool LL>
RowFn by_epi(int epi) {
  switch (epi) {
    case 0: return row_kernel<N, VPT, LL, 0>;
    case ARFUSE_EPI_BF16: return row_kernel<N, VPT, LL, ARFUSE_EPI_BF16>;
    case ARFUSE_EPI_FP4: return row_kernel<N, VPT, LL, ARFUSE_EPI_FP4>;
    case ARFUSE_EPI_BF16 | ARFUSE_EPI_FP4: return row_kernel<N, VPT, LL, ARFUSE_EPI_BF16 | ARFUSE_EPI_FP4>;
    case ARFUSE_EPI_FP8: return row_kernel<N, VPT, LL, ARFUSE_EPI_FP8>;
    case ARFUSE_EPI_BF16 | ARFUSE_EPI_FP8: return row_kernel<N, VPT, LL, ARFUSE_EPI_BF16 | ARFUSE_EPI_FP8>;
  }
  return nullptr;
}

template <int N, int VPT>
RowFn by_layout(bool ll, int epi) {
  return ll ? by_epi<N, VPT, true>(epi) : by_epi<N, VPT, false>(epi);
}

template <int N>
RowFn by_vpt(int vpt, bool ll, int epi) {
  switch (vpt) {
    case 1: return by_layout<N, 1>(ll, epi);
    case 2: return by_layout<N, 2>(ll, epi);
    case 4: return by_layout<N, 4>(ll, epi);
    case 8: return by_layout<N, 8>(ll, epi);
  }
  return nullptr;
}

}  // namespace

RowFn ARFUSE_CAT(select_row_kernel_n, ARFUSE_N)(int vpt, bool ll, int epi) {
  return by_vpt<ARFUSE_N>(vpt, ll, epi);
}

}  // namespace arfuse_detail
