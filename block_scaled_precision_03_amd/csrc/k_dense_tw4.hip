// Dense kernels: tensor-wise FP8 with A in E4M3 (B in E4M3 or E5M2).
#include "kernels.hpp"

namespace mxg {
dense_fn pick_dense_tw_a4(int eb, int layout, bool psb, bool fuse) {
  if (eb == F_E4M3) return pick_big<F_E4M3, F_E4M3, SM_TENSOR>(layout, psb, fuse);
  if (eb == F_E5M2) return pick_big<F_E4M3, F_E5M2, SM_TENSOR>(layout, psb, fuse);
  return nullptr;
}
}  // namespace mxg
