// The 64 x 64 NT kernel for small outputs, every format and scale mode.
#include "kernels.hpp"

namespace mxg {
namespace {
template <int FA, int FB>
dense_fn pick_small_fmt(bool mx, bool psb, bool fuse) {
  if (mx) {
    if (fuse) return psb ? dense_small_kernel<FA, FB, SM_MX, true, true> : dense_small_kernel<FA, FB, SM_MX, false, true>;
    return psb ? dense_small_kernel<FA, FB, SM_MX, true, false> : dense_small_kernel<FA, FB, SM_MX, false, false>;
  }
  if constexpr (FA != F_E2M1 && FB != F_E2M1) {
    if (fuse)
      return psb ? dense_small_kernel<FA, FB, SM_TENSOR, true, true> : dense_small_kernel<FA, FB, SM_TENSOR, false, true>;
    return psb ? dense_small_kernel<FA, FB, SM_TENSOR, true, false> : dense_small_kernel<FA, FB, SM_TENSOR, false, false>;
  }
  return nullptr;
}
}  // namespace

dense_fn pick_small(int ea, int eb, bool mx, bool psb, bool fuse) {
  if (ea == F_E2M1 && eb == F_E2M1) return pick_small_fmt<F_E2M1, F_E2M1>(mx, psb, fuse);
  if (ea == F_E4M3 && eb == F_E4M3) return pick_small_fmt<F_E4M3, F_E4M3>(mx, psb, fuse);
  if (ea == F_E4M3 && eb == F_E5M2) return pick_small_fmt<F_E4M3, F_E5M2>(mx, psb, fuse);
  if (ea == F_E5M2 && eb == F_E4M3) return pick_small_fmt<F_E5M2, F_E4M3>(mx, psb, fuse);
  if (ea == F_E5M2 && eb == F_E5M2) return pick_small_fmt<F_E5M2, F_E5M2>(mx, psb, fuse);
  return nullptr;
}
}  // namespace mxg
