// Grouped groupwise FP8 GEMM for gfx950 ("Add FlyDSL grouped groupwise FP8
// GEMM for ROCm"): for each group g of rows (an expert),
//   D[r, n] = sum_k dec(XQ[r,k]) xs(r, k/128) * dec(WQ[g,n,k]) ws[g, n/128, k/128].
//
// * Tile scheduling: the grid is derived from static shapes only --
//   (ceil(totM/BM) + G - 1) M-tiles x N/BN N-tiles -- and each workgroup
//   resolves its group by walking m_sizes on the device (Tile selection;
//   commit on in-kernel group resolution).  A tile never spans two groups;
//   tiles past the last group exit.  Every group is clamped to [0, totM) so a
//   violated sum(m_sizes) == totM precondition cannot reach memory outside D.
// * Software scaling (Architecture support): each 128-K step runs the scaled
//   matrix-core instruction with the neutral E8M0 scale into a zeroed
//   accumulator, then adds that partial times xs(row, kb) * ws(g, n/128, kb)
//   in FP32.
// * Activation scales are read in the per-group block layout (commit on the
//   scale_a layout): group g's block begins at start_g*(K/128); (local row i,
//   k-block kb) sits at i + kb*M_g.
// * B is either plain [G, N, K] (staged through XOR-swizzled LDS like A) or
//   preshuffled per group (copied linearly into LDS).
#pragma once
#include "dense.hpp"

namespace mxg {

struct GroupedArgs {
  const int64_t *m_sizes;
  const uint8_t *XQ, *WQ;
  const float *xs, *ws;
  uint16_t *D;
  int64_t totM, N, K;
  int G, tiles_n;
};

template <int BM, int BN, bool PSB>
__global__ __launch_bounds__(256, 1) void grouped_kernel(GroupedArgs p) {
  constexpr int FM = BM / 32, FN = BN / 32;     // 2x2 waves
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
  const int wm = w >> 1, wn = w & 1;
  const int i16 = lane & 15;
  const int tm_flat = blockIdx.x / p.tiles_n;
  const int tn = blockIdx.x % p.tiles_n;

  // ---- group resolution (uniform across the workgroup)
  int64_t start = 0, seen = 0, mg = 0, tl = -1;
  int g = -1;
  for (int gg = 0; gg < p.G; ++gg) {
    int64_t s = p.m_sizes[gg];
    const int64_t room = p.totM - start;
    s = s < 0 ? 0 : (s > room ? room : s);
    const int64_t t = (s + BM - 1) / BM;
    if (tm_flat < seen + t) {
      g = gg;
      mg = s;
      tl = tm_flat - seen;
      break;
    }
    seen += t;
    start += s;
  }
  if (g < 0) return;
  const int64_t row0 = start + tl * BM;
  const int64_t row_lim = start + mg;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t K = p.K, N = p.N;
  const int nst = (int)(K / 128);
  const int64_t kb_n = K / 128;
  const uint8_t *Wg = p.WQ + (int64_t)g * N * K;
  const int64_t wbytes = N * K;

  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(p.xs, clamp_records(p.totM * kb_n * 4));
  const float *wsg = p.ws + (int64_t)g * (N / 128) * kb_n + ((n0 + wn * (BN / 2)) / 128) * kb_n;

  v4f acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

  float xs_n[FM], ws_n = 0.f;
  auto load_scales = [&](int st) {
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      const int64_t local = row0 + wm * (BM / 2) + a * 16 + i16 - start;
      const int64_t idx = start * kb_n + local + (int64_t)st * mg;
      xs_n[a] = __uint_as_float(buf_load_u32(rxs, (uint32_t)(idx * 4)));
    }
    ws_n = wsg[st];
  };
  auto load_stage = [&](int st, uint8_t *buf) {
    load_nt<BM, 4>(p.XQ, p.totM * K, row0, K, st, buf, w, lane);
    if constexpr (PSB) load_ps<BN, 4>(Wg, wbytes, n0 / 64, kb_n, st, buf + BM * 128, w, lane);
    else load_nt<BN, 4>(Wg, wbytes, n0, K, st, buf + BM * 128, w, lane);
  };

  if (nst > 0) {
    load_stage(0, smem);
    load_scales(0);
  }
  wait_vmem();
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const uint8_t *la = smem + (st & 1) * STAGE;
    const uint8_t *lb = la + BM * 128;
    float xs_c[FM];
#pragma unroll
    for (int a = 0; a < FM; ++a) xs_c[a] = xs_n[a];
    const float ws_c = ws_n;
    v8i bf[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      if constexpr (PSB) bf[b] = frag_ps8(lb, wn * (BN / 32) + b, lane);
      else bf[b] = frag_nt8(lb, wn * (BN / 2) + b * 16, lane);
    }
    if (st + 1 < nst) {
      load_stage(st + 1, smem + ((st + 1) & 1) * STAGE);
      load_scales(st + 1);
    }
    v8i af = frag_nt8(la, wm * (BM / 2), lane);
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      v8i af_next;
      if (a + 1 < FM) af_next = frag_nt8(la, wm * (BM / 2) + (a + 1) * 16, lane);
      const float sc = xs_c[a] * ws_c;
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const v4f part = mfma_scaled<F_E4M3, F_E4M3>(bf[b], af, (v4f){0.f, 0.f, 0.f, 0.f},
                                                      E8M0_ONE_X4, E8M0_ONE_X4);
        acc[a][b] += part * sc;
      }
      if (a + 1 < FM) af = af_next;
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem();
    __syncthreads();
  }

  store_tile<BM, BN, FM, FN>(acc, 1.0f, smem, p.D, row0, n0, row_lim, N, wm, wn);
}

}  // namespace mxg
