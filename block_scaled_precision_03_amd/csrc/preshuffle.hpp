// One-time re-layout kernels: B operand codes and E8M0 scales into the order
// in which the gfx950 scaled matrix-core K-loop consumes them.  Callers run
// them once per weight at load time ("Add FlyDSL grouped groupwise FP8 GEMM
// for ROCm", PR body: weights pre-swizzled into the MFMA B layout once, the
// GEMM call does no shuffling).  Byte moves only: HBM-bound.
//
// FP8 B layout: fragment (n-tile t of 16 rows, k-step ks of 128 K) occupies
// 2048 contiguous bytes at (t*nks + ks)*2048: half h (0/1) at +1024*h, lane l
// at +16*l, holding row 16t + l%16, k = 128ks + 64h + 16(l/16) + j, j=0..15.
// FP4 B layout: fragment (t, ks) occupies 1024 bytes at (t*nks + ks)*1024:
// lane l at +16*l holds packed bytes 64ks + 16(l/16) + j of row 16t + l%16
// (K values 128ks + 32(l/16) + [0, 32)).
// E8M0 scale layout: word ((rt*ngrp + g)*64 + l) of 4 bytes, byte t =
// scale of row 16rt + l%16, 32-K block 16g + 4t + l/16 (four k-steps per word).
#pragma once
#include "common.hpp"

namespace mxg {

// One thread per 16-byte output chunk.
template <bool FP4, bool TB>
__global__ __launch_bounds__(256) void preshuffle_b_kernel(const uint8_t *__restrict__ B,
                                                           uint8_t *__restrict__ out,
                                                           int64_t N, int64_t K,
                                                           int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t nks = K / 128;
  const int lane = (int)(c & 63);
  int64_t frag, h;
  if (FP4) { frag = c >> 6; h = 0; }
  else { frag = c >> 7; h = (c >> 6) & 1; }
  const int64_t t = frag / nks, ks = frag % nks;
  const int64_t n = 16 * t + (lane & 15);
  uint8_t v[16];
  if (FP4) {
    const int64_t b0 = 64 * ks + 16 * (lane >> 4);   // packed byte offset in row n
    if (n < N) {
      const u4v x = *(const u4v *)(B + n * (K / 2) + b0);
      *(u4v *)v = x;
    } else {
      *(u4v *)v = (u4v){0u, 0u, 0u, 0u};
    }
  } else {
    const int64_t k0 = 128 * ks + 64 * h + 16 * (lane >> 4);
    if (n >= N) {
      *(u4v *)v = (u4v){0u, 0u, 0u, 0u};
    } else if (!TB) {
      *(u4v *)v = *(const u4v *)(B + n * K + k0);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = B[(k0 + j) * N + n];
    }
  }
  *(u4v *)(out + c * 16) = *(u4v *)v;
}

// One thread per output 32-bit word.
__global__ __launch_bounds__(256) void preshuffle_scales_kernel(const uint8_t *__restrict__ s,
                                                                uint32_t *__restrict__ out,
                                                                int64_t rows, int64_t K,
                                                                int64_t nwords) {
  const int64_t wi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (wi >= nwords) return;
  const int64_t sk = K / 32, ngrp = (K + 511) / 512;
  const int lane = (int)(wi & 63);
  const int64_t rg = wi >> 6;
  const int64_t rt = rg / ngrp, g = rg % ngrp;
  const int64_t row = 16 * rt + (lane & 15);
  uint32_t word = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t blk = 16 * g + 4 * t + (lane >> 4);
    uint32_t b = 127u;
    if (row < rows && blk < sk) b = s[row * sk + blk];
    word |= b << (8 * t);
  }
  out[wi] = word;
}

}  // namespace mxg
