// Row-kernel instances for one rank count ARFUSE_N (set by the build):
// every VPT in {1, 2, 4, 8} x {plain, LL, sentinel} x epilogue mask, the
// split-row instances for VPT 1 and 2, and the streaming-store instances for
// every VPT in the plain and sentinel layouts (LL rows are decode-sized).

#include "arfuse_device.hpp"

#ifndef ARFUSE_N
#error "build with -DARFUSE_N=<1..8>"
#endif

#define ARFUSE_CAT2(a, b) a##b
#define ARFUSE_CAT(a, b) ARFUSE_CAT2(a, b)

namespace arfuse_detail {
namespace {

template <int N, int VPT, bool LL, bool SENT, int KIND>
RowFn by_epi(int epi) {
  constexpr int B = ARFUSE_EPI_BF16, F4 = ARFUSE_EPI_FP4, F8 = ARFUSE_EPI_FP8;
  switch (epi) {
    case 0: return row_kernel<N, VPT, LL, SENT, 0, KIND>;
    case B: return row_kernel<N, VPT, LL, SENT, B, KIND>;
    case F4: return row_kernel<N, VPT, LL, SENT, F4, KIND>;
    case B | F4: return row_kernel<N, VPT, LL, SENT, B | F4, KIND>;
    case F8: return row_kernel<N, VPT, LL, SENT, F8, KIND>;
    case B | F8: return row_kernel<N, VPT, LL, SENT, B | F8, KIND>;
  }
  return nullptr;
}

template <int N, int VPT, int KIND>
RowFn by_layout(int layout, int epi) {
  switch (layout) {
    case ARFUSE_LAYOUT_PLAIN: return by_epi<N, VPT, false, false, KIND>(epi);
    case ARFUSE_LAYOUT_LL:
      if constexpr (KIND == kRowStream) return nullptr;
      else return by_epi<N, VPT, true, false, KIND>(epi);
    case ARFUSE_LAYOUT_SENTINEL: return by_epi<N, VPT, false, true, KIND>(epi);
  }
  return nullptr;
}

template <int N, int KIND>
RowFn by_vpt_kind(int vpt, int layout, int epi) {
  switch (vpt) {
    case 1: return by_layout<N, 1, KIND>(layout, epi);
    case 2: return by_layout<N, 2, KIND>(layout, epi);
    case 4:
      if constexpr (KIND == kRowSplit) return nullptr;
      else return by_layout<N, 4, KIND>(layout, epi);
    case 8:
      if constexpr (KIND == kRowSplit) return nullptr;
      else return by_layout<N, 8, KIND>(layout, epi);
  }
  return nullptr;
}

template <int N>
RowFn by_vpt(int vpt, int layout, int epi, int kind) {
  switch (kind) {
    case kRowWhole: return by_vpt_kind<N, kRowWhole>(vpt, layout, epi);
    case kRowSplit: return by_vpt_kind<N, kRowSplit>(vpt, layout, epi);
    case kRowStream: return by_vpt_kind<N, kRowStream>(vpt, layout, epi);
  }
  return nullptr;
}

}  // namespace

RowFn ARFUSE_CAT(select_row_kernel_n, ARFUSE_N)(int vpt, int layout, int epi, int kind) {
  return by_vpt<ARFUSE_N>(vpt, layout, epi, kind);
}

}  // namespace arfuse_detail
