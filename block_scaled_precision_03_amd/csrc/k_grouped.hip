// The grouped groupwise FP8 kernels.
#include "kernels.hpp"

namespace mxg {
dense_fn pick_grouped_dense(bool psb) {
  return psb ? grouped_dense_kernel<true> : grouped_dense_kernel<false>;
}

grouped_fn pick_grouped_stream(int bm, bool psb) {
  if (bm == 64) return psb ? grouped_stream_kernel<true, 64, 64, 2, 2> : grouped_stream_kernel<false, 64, 64, 2, 2>;
  if (bm == 128) return psb ? grouped_stream_kernel<true, 128, 128, 1, 2> : grouped_stream_kernel<false, 128, 128, 1, 2>;
  return nullptr;
}

dense_fn pick_grouped_bf16(bool psb) {
  return psb ? grouped_dense_kernel<true, F_BF16> : grouped_dense_kernel<false, F_BF16>;
}

grouped_fn pick_grouped_stream_bf16(int bm, int bn, bool psb) {
  if (bm == 64 && bn == 64)
    return psb ? grouped_stream_kernel<true, 64, 64, 2, 2, false, F_BF16> : grouped_stream_kernel<false, 64, 64, 2, 2, false, F_BF16>;
  if (bm == 128 && bn == 128)
    return psb ? grouped_stream_kernel<true, 128, 128, 1, 2, false, F_BF16> : grouped_stream_kernel<false, 128, 128, 1, 2, false, F_BF16>;
  if (bm == 128 && bn == 64)
    return psb ? grouped_stream_kernel<true, 128, 64, 1, 2, false, F_BF16> : grouped_stream_kernel<false, 128, 64, 1, 2, false, F_BF16>;
  return nullptr;
}

grouped_fn pick_grouped_tail_bf16(bool psb) {
  return psb ? grouped_stream_kernel<true, 128, 64, 2, 2, true, F_BF16> : grouped_stream_kernel<false, 128, 64, 2, 2, true, F_BF16>;
}

grouped_fn pick_grouped_tail(bool psb) {
  return psb ? grouped_stream_kernel<true, 128, 64, 2, 2, true> : grouped_stream_kernel<false, 128, 64, 2, 2, true>;
}
}  // namespace mxg
