// The kernel instantiations of the library, by translation unit, as host
// pointers to their launch stubs.  Each k_*.hip file instantiates one share
// of the templates (so that the shares compile in parallel) and returns the
// kernel that a call with these static arguments launches, or nullptr for
// a combination that is not built.
#pragma once
#include "grouped.hpp"
#include "small.hpp"

namespace mxg {

typedef void (*dense_fn)(DenseArgs);
typedef void (*grouped_fn)(GroupedArgs);

// Persistent 256 x 256 dense kernel of one scale mode (SM_MX, SM_TENSOR),
// NT/NN/TN; `fuse`: the bias/activation epilogue (NT only).
template <int FA, int FB, int SMODE>
dense_fn pick_big(int layout, bool psb, bool fuse) {
  constexpr int NT = 0, NN = 1, TN = 2;          // the header's layout codes
  if (fuse) {
    if (layout != NT) return nullptr;
    return psb ? dense_kernel<FA, FB, SMODE, false, false, true, true>
               : dense_kernel<FA, FB, SMODE, false, false, false, true>;
  }
  {
    // MX scales are blocked along K whatever the code layout, so the
    // transposed variants load them exactly as NT does
    switch (layout) {
      case NT: return psb ? dense_kernel<FA, FB, SMODE, false, false, true> : dense_kernel<FA, FB, SMODE, false, false, false>;
      case NN: return psb ? nullptr : dense_kernel<FA, FB, SMODE, false, true, false>;
      case TN: return psb ? nullptr : dense_kernel<FA, FB, SMODE, true, true, false>;
      default: return nullptr;
    }
  }
}

// k_dense_mx4.hip / k_dense_mx5.hip: MX FP8 with A in E4M3 / E5M2.
dense_fn pick_dense_mx_a4(int eb, int layout, bool psb, bool fuse);
dense_fn pick_dense_mx_a5(int eb, int layout, bool psb, bool fuse);
// k_dense_tw4.hip / k_dense_tw5.hip: tensor-wise FP8 with A in E4M3 / E5M2.
dense_fn pick_dense_tw_a4(int eb, int layout, bool psb, bool fuse);
dense_fn pick_dense_tw_a5(int eb, int layout, bool psb, bool fuse);
// k_dense_fp4.hip: MXFP4.
dense_fn pick_dense_fp4(int layout, bool psb, bool fuse);
// k_small.hip: the 64 x 64 NT kernel, every format.
dense_fn pick_small(int ea, int eb, bool mx, bool psb, bool fuse);
// k_grouped.hip: the grouped kernels (256 x 256 dense pipeline; persistent
// streaming with BM-row tiles; the streaming kernel on the dense pipeline's
// tail pieces).
dense_fn pick_grouped_dense(bool psb);
grouped_fn pick_grouped_stream(int bm, bool psb);
grouped_fn pick_grouped_tail(bool psb);
// The BF16 grouped GEMM on the same three kernels.
dense_fn pick_grouped_bf16(bool psb);
grouped_fn pick_grouped_stream_bf16(int bm, int bn, bool psb);
grouped_fn pick_grouped_tail_bf16(bool psb);

}  // namespace mxg
