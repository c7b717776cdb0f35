// Dense kernels: MXFP4 (E2M1 x E2M1 with E8M0 scales).
#include "kernels.hpp"

namespace mxg {
dense_fn pick_dense_fp4(int layout, bool psb, bool fuse) {
  return pick_big<F_E2M1, F_E2M1, SM_MX>(layout, psb, fuse);
}
}  // namespace mxg
