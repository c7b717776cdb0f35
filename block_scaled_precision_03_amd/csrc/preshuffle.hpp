// One-time re-layout kernels: B operand codes and E8M0 scales into the order
// in which the gfx950 scaled matrix-core K-loop consumes them.  Callers run
// them once per weight at load time ("Add FlyDSL grouped groupwise FP8 GEMM
// for ROCm", PR body: weights pre-swizzled into the MFMA B layout once, the
// GEMM call does no shuffling).  Byte moves only: HBM-bound.
//
// Layouts (column group cg = 64 rows of B, k-step ks = 128 K values; rows
// past N are zero):
// FP8 B: chunk (cg, ks) of 8 KiB at (cg*nks + ks)*8192; within it, n-tile t
//   (16 rows) at +2048t, K half h at +1024h, lane l at +16l holds row
//   64cg + 16t + l%16, k = 128ks + 64h + 16(l/16) + j, j = 0..15.
// FP4 B: chunk (cg, ks) of 4 KiB at (cg*nks + ks)*4096; lane l of n-tile t
//   at +1024t + 16l holds packed bytes 64ks + 16(l/16) + j of row
//   64cg + 16t + l%16 (K values 128ks + 32(l/16) + [0, 32)).
// E8M0 scales: 32-bit word ((cg*ngrp + g)*4 + t)*64 + l (ngrp = ceil(K/512)),
//   byte j = scale of row 64cg + 16t + l%16, 32-K block 16g + 4j + l/16;
//   padding reads as 127 (2^0).  A column group's words for one group of
//   four K steps are 1 KiB in (subtile, lane) order, so a wave reads the
//   words of one subtile as 64 consecutive words.
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
  constexpr int PER_CHUNK = FP4 ? 256 : 512;       // 16-byte pieces per (cg, ks)
  const int64_t cgks = c / PER_CHUNK;
  const int r2 = (int)(c % PER_CHUNK);
  const int64_t cg = cgks / nks, ks = cgks % nks;
  int t, h, lane;
  if (FP4) { t = r2 >> 6; h = 0; lane = r2 & 63; }
  else { t = r2 >> 7; h = (r2 >> 6) & 1; lane = r2 & 63; }
  const int64_t n = 64 * cg + 16 * t + (lane & 15);
  u4v v = (u4v){0u, 0u, 0u, 0u};
  if (n < N) {
    if (FP4) {
      v = *(const u4v *)(B + n * (K / 2) + 64 * ks + 16 * (lane >> 4));
    } else {
      const int64_t k0 = 128 * ks + 64 * h + 16 * (lane >> 4);
      if (!TB) {
        v = *(const u4v *)(B + n * K + k0);
      } else {
        uint8_t b[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) b[j] = B[(k0 + j) * N + n];
        v = *(const u4v *)b;
      }
    }
  }
  *(u4v *)(out + c * 16) = v;
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
  const int t = (int)((wi >> 6) & 3);
  const int64_t cgg = wi >> 8;
  const int64_t cg = cgg / ngrp, g = cgg % ngrp;
  const int64_t row = 64 * cg + 16 * t + (lane & 15);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t blk = 16 * g + 4 * j + (lane >> 4);
    uint32_t b = 127u;
    if (row < rows && blk < sk) b = s[row * sk + blk];
    word |= b << (8 * j);
  }
  out[wi] = word;
}

}  // namespace mxg
