// Dense NT GEMM for small outputs: 64 x 64 tiles, one workgroup per tile.
//
// A 256 x 256 tile of the persistent kernel needs 256 rows and 256 columns
// of output to keep one compute unit busy; a GEMM with a few such tiles
// leaves most compute units idle (a 256^3 GEMM is one tile on one of 256).
// This kernel cuts the output into 64 x 64 tiles (sixteen times as many),
// four waves per workgroup in a 2 x 2 grid, each a 32 x 32 block of 2 x 2
// matrix-core tiles.  There is no LDS staging: every wave loads its own
// fragments from global memory straight into registers in the scaled
// matrix-core instruction's operand order, three 128-element K steps ahead
// of the one it computes, through range-checked buffer loads (rows past M
// or N read zeros).  Preshuffled B (and its E8M0 scales) is read in the
// layout of preshuffle.hpp, where a lane's fragment is one contiguous 16
// bytes.  Per output element the instruction sequence over K is the
// persistent kernel's, so the two give identical bits.
//
// MX operands feed their E8M0 scales to the instruction ("PyTorch on AMD
// GPUs gains a FlyDSL backend", Interpretation); tensor-wise operands use
// the neutral scale and sA*sB in the epilogue ("Experimental FlyDSL GEMM
// backend for TE PyTorch", Supported Data Types).  The fused epilogue adds
// the BF16 bias and applies the activation as mxgemm_run_fused specifies.
#pragma once
#include "dense.hpp"

namespace mxg {

constexpr int SBM = 64, SBN = 64;

template <int FA, int FB, int SMODE, bool PSB, bool FUSE>
__global__ __launch_bounds__(256) void dense_small_kernel(DenseArgs p) {
  constexpr bool FP4 = (FA == F_E2M1);
  constexpr bool MX = (SMODE == SM_MX);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int i16 = lane & 15, q = lane >> 4;
  const int tm = (int)blockIdx.x / p.tiles_n, tn = (int)blockIdx.x % p.tiles_n;
  const int64_t m0 = (int64_t)tm * SBM + wm * 32, n0 = (int64_t)tn * SBN + wn * 32;
  const int64_t KB = FP4 ? p.K / 2 : p.K;          // bytes of K per row
  const int nst = (int)(p.K / 128);
  const int64_t sk = p.K / 32;                     // E8M0 scales per row
  const int64_t nks = p.K / 128, ngrp = (p.K + 511) / 512;

  // Operand resources from the wave's first row / column (rows past the
  // operand's end read zeros).
  const int64_t abase = m0 * KB;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + abase, clamp_records(p.a_bytes - abase));
  int64_t bbase;
  if constexpr (PSB) bbase = ((tn * SBN) / 64) * nks * (FP4 ? 4096 : 8192);
  else bbase = n0 * KB;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + bbase, clamp_records(p.b_bytes - bbase));
  __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.A, 0), rsb = make_rsrc(p.A, 0);
  if constexpr (MX) {
    const int64_t sab = m0 * sk;
    rsa = make_rsrc((const uint8_t *)p.sA + sab, clamp_records(p.sa_bytes - sab));
    int64_t sbb;
    if constexpr (PSB) sbb = ((tn * SBN) / 64) * ngrp * 1024;
    else sbb = n0 * sk;
    rsb = make_rsrc((const uint8_t *)p.sB + sbb, clamp_records(p.sb_bytes - sbb));
  }

  // Per-lane byte offsets (fragment t = 0, 1 of the wave's 2 x 2 tiles).
  // K-contiguous FP8 row r: bytes 16q and 64 + 16q of the 128-byte step;
  // FP4: bytes 16q of the 64-byte step.  Preshuffled: subtile s of the
  // column group at 2048 s (FP8; 1024 s for FP4), then lane * 16 (+ 1024 for
  // the second FP8 half).
  const int ps = FP4 ? 64 : 128;                   // bytes per K step and row
  auto frag_a = [&](int st, int a) -> v8i {
    const uint32_t o = (uint32_t)((16 * a + i16) * KB + (int64_t)st * ps + 16 * q);
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)o, 0, 0);
    if constexpr (FP4) return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(o + 64), 0, 0);
    return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  auto frag_b = [&](int st, int b) -> v8i {
    uint32_t o;
    if constexpr (PSB) {
      const int s = wn * 2 + b;
      o = FP4 ? (uint32_t)(st * 4096 + s * 1024 + lane * 16) : (uint32_t)(st * 8192 + s * 2048 + lane * 16);
    } else {
      o = (uint32_t)((16 * b + i16) * KB + (int64_t)st * ps + 16 * q);
    }
    const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)o, 0, 0);
    if constexpr (FP4) return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
    const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(o + (PSB ? 1024 : 64)), 0, 0);
    return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  // E8M0 scales: lane (i, q) uses 32-K block q of its row in K step st.
  auto scale_a = [&](int st, int a) -> int {
    if constexpr (!MX) return E8M0_ONE_X4;
    const uint32_t wd = buf_load_u32(rsa, (uint32_t)((16 * a + i16) * sk + 4 * st));
    return (int)(wd >> (8 * q));
  };
  auto scale_b = [&](int st, int b) -> int {
    if constexpr (!MX) return E8M0_ONE_X4;
    if constexpr (PSB) {
      const int s = wn * 2 + b;
      const uint32_t wd = buf_load_u32(rsb, (uint32_t)((((st >> 2) * 4 + s) * 64 + lane) * 4));
      return (int)(wd >> (8 * (st & 3)));
    } else {
      const uint32_t wd = buf_load_u32(rsb, (uint32_t)((16 * b + i16) * sk + 4 * st));
      return (int)(wd >> (8 * q));
    }
  };

  v4f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

  // A ring of SD register sets: the loads of K step st + SD - 1 are issued
  // before step st is computed, so SD - 1 steps of loads are in flight (one
  // workgroup per tile leaves few waves per compute unit to cover a load's
  // latency otherwise).
  constexpr int SD = 4;
  v8i fa[SD][2], fb[SD][2];
  int sa[SD][2], sb[SD][2];
  auto load = [&](int st, auto slot) {
    constexpr int sl = decltype(slot)::value;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      fa[sl][x] = frag_a(st, x);
      fb[sl][x] = frag_b(st, x);
      sa[sl][x] = scale_a(st, x);
      sb[sl][x] = scale_b(st, x);
    }
  };
  static_for<0, SD - 1>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (j < nst) load(j, std::integral_constant<int, j>{});
  });
  for (int st0 = 0; st0 < nst; st0 += SD) {
    static_for<0, SD>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int st = st0 + j;
      if (st < nst) {
        if (st + SD - 1 < nst) load(st + SD - 1, std::integral_constant<int, (j + SD - 1) % SD>{});
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            // first operand = B tile: the result lane holds 4 consecutive n
            acc[a][b] = mfma_scaled<FB, FA>(fb[j][b], fa[j][a], acc[a][b], sb[j][b], sa[j][a]);
      }
    });
  }

  // Epilogue: lane (i, q) of tile (a, b) holds row m0 + 16a + i, columns
  // n0 + 16b + 4q .. +3.
  float alpha = 1.0f;
  if constexpr (SMODE == SM_TENSOR) alpha = *(const float *)p.sA * *(const float *)p.sB;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t r = m0 + 16 * a + i16;
    if (r >= p.M) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + 16 * b + 4 * q;
      v4f v = acc[a][b];
      if constexpr (SMODE == SM_TENSOR) v = v * alpha;
      if constexpr (FUSE) {
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (col + k < p.N) bias[k] = __uint_as_float((uint32_t)p.bias[col + k] << 16);
        }
        v.x = activate(p.act, v.x + bias[0]);
        v.y = activate(p.act, v.y + bias[1]);
        v.z = activate(p.act, v.z + bias[2]);
        v.w = activate(p.act, v.w + bias[3]);
      }
      const uint32_t u[2] = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
      uint16_t *dst = p.D + r * p.N + col;
      if (col + 4 <= p.N && (p.N & 3) == 0) {
        *(v2i *)dst = (v2i){(int)u[0], (int)u[1]};
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (col + k < p.N) dst[k] = (uint16_t)(u[k >> 1] >> (16 * (k & 1)));
      }
    }
  }
}

}  // namespace mxg
