// Measurement aids (not part of the GEMM path): the throughput the scaled
// matrix-core instruction reaches with nothing else running, and the shader
// clock while it runs, so that a kernel's fraction of the published peak can
// be read against what the chip sustains.
#pragma once
#include "common.hpp"

namespace mxg {

// Eight waves per workgroup (two per SIMD, as the dense kernel), each running
// 32 independent accumulator chains of v_mfma_scale_f32_16x16x128_f8f6f4 on
// finite codes that vary by lane (E4M3 codes with exponent field <= 14, or
// any E2M1 nibbles), neutral scales.  Wave 0 of workgroup 0 reads the shader
// clock counter (s_memtime) and the 100 MHz reference (s_memrealtime) around
// the loop and writes both deltas to clk[0], clk[1].
template <int FMT>
__global__ __launch_bounds__(512, 1) void mfma_ceiling_kernel(int64_t iters, uint64_t *clk) {
  const int lane = threadIdx.x & 63;
  const uint32_t mask = 0x77777777u;   // E4M3: exponent field <= 14 (finite)
  v8i x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (int)((0x9E3779B9u * (uint32_t)(lane * 8 + i + 1)) & mask);
    y[i] = (int)((0x85EBCA6Bu * (uint32_t)(lane * 8 + i + 7)) & mask);
  }
  v4f acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = mfma_scaled<FMT, FMT>(x, y, acc[i], E8M0_ONE_X4, E8M0_ONE_X4);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s += acc[i].x + acc[i].y + acc[i].z + acc[i].w;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
  if (s == 1234.5f) clk[2] = (uint64_t)threadIdx.x;   // keeps the chains live
}

}  // namespace mxg
