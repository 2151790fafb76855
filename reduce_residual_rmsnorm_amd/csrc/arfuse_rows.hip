// Row-kernel instances for one rank count ARFUSE_N (set by the build):
// every VPT in {1, 2, 4, 8} x {plain, LL, sentinel} x epilogue mask, and the
// split-row instances for VPT 1 and 2.

#include "arfuse_device.hpp"

#ifndef ARFUSE_N
#error "build with -DARFUSE_N=<1..8>"
#endif

#define ARFUSE_CAT2(a, b) a##b
#define ARFUSE_CAT(a, b) ARFUSE_CAT2(a, b)

namespace arfuse_detail {
namespace {

template <int N, int VPT, bool LL, bool SENT, bool SPLIT>
RowFn by_epi(int epi) {
  constexpr int B = ARFUSE_EPI_BF16, F4 = ARFUSE_EPI_FP4, F8 = ARFUSE_EPI_FP8;
  switch (epi) {
    case 0: return row_kernel<N, VPT, LL, SENT, 0, SPLIT>;
    case B: return row_kernel<N, VPT, LL, SENT, B, SPLIT>;
    case F4: return row_kernel<N, VPT, LL, SENT, F4, SPLIT>;
    case B | F4: return row_kernel<N, VPT, LL, SENT, B | F4, SPLIT>;
    case F8: return row_kernel<N, VPT, LL, SENT, F8, SPLIT>;
    case B | F8: return row_kernel<N, VPT, LL, SENT, B | F8, SPLIT>;
  }
  return nullptr;
}

template <int N, int VPT, bool SPLIT>
RowFn by_layout(int layout, int epi) {
  switch (layout) {
    case ARFUSE_LAYOUT_PLAIN: return by_epi<N, VPT, false, false, SPLIT>(epi);
    case ARFUSE_LAYOUT_LL: return by_epi<N, VPT, true, false, SPLIT>(epi);
    case ARFUSE_LAYOUT_SENTINEL: return by_epi<N, VPT, false, true, SPLIT>(epi);
  }
  return nullptr;
}

template <int N>
RowFn by_vpt(int vpt, int layout, int epi, bool split) {
  if (split) {
    switch (vpt) {
      case 1: return by_layout<N, 1, true>(layout, epi);
      case 2: return by_layout<N, 2, true>(layout, epi);
    }
    return nullptr;
  }
  switch (vpt) {
    case 1: return by_layout<N, 1, false>(layout, epi);
    case 2: return by_layout<N, 2, false>(layout, epi);
    case 4: return by_layout<N, 4, false>(layout, epi);
    case 8: return by_layout<N, 8, false>(layout, epi);
  }
  return nullptr;
}

}  // namespace

RowFn ARFUSE_CAT(select_row_kernel_n, ARFUSE_N)(int vpt, int layout, int epi, bool split) {
  return by_vpt<ARFUSE_N>(vpt, layout, epi, split);
}

}  // namespace arfuse_detail
