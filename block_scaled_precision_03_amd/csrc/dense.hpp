// Dense block-scaled GEMM kernel for gfx950:
//   D[m,n] = sum_k a(m,k) b(n,k), FP32 accumulation on the scaled matrix
//   cores (v_mfma_scale_f32_16x16x128_f8f6f4), BF16 output.
//
// MX operands feed their E8M0 block scales straight into the instruction
// (one scale per 32 K values: "PyTorch on AMD GPUs gains a FlyDSL backend",
// Interpretation).  Tensor-wise operands use the neutral scale 2^0 in the
// instruction and multiply by sA*sB in the epilogue ("Experimental FlyDSL GEMM
// backend for TE PyTorch", Supported Data Types: tensor-wise and mixed
// E4M3/E5M2 FP8).
//
// Block tile 256x256, four waves in a 2x2 grid (128x128 per wave, 8x8
// matrix-core tiles of 16x16).  Each stage holds 128 bytes of K per row of A
// and B (one 128-element K step for FP8, two for FP4) in LDS, double
// buffered (2 x 64 KiB of the 160 KiB).  Operands travel global -> LDS by
// buffer-load-to-LDS DMA, 16 bytes per lane, into XOR-swizzled rows so that
// the fragment reads are free of bank conflicts.  Transposed operands (the
// 'T' side of NN/TN) are kept in LDS k-major and read with the transposing
// ds_read_b64_tr_b8.  The epilogue stages the BF16 tile through the same LDS
// and writes 16-byte coalesced rows.
#pragma once
#include "common.hpp"

namespace mxg {

enum : int { SM_MX = 0, SM_TENSOR = 1 };

struct DenseArgs {
  const uint8_t *A, *B;
  const void *sA, *sB;
  uint16_t *D;
  int64_t M, N, K;
  int64_t a_bytes, b_bytes, sa_bytes, sb_bytes;
  int tiles_m, tiles_n;
};

constexpr int DBM = 256, DBN = 256, DNW = 4;
constexpr int DSTAGE = (DBM + DBN) * 128;

// ---------------------------------------------------------------------------
// Global -> LDS stage loaders.  Each issues R*128/1024 wave-wide 1 KiB DMAs.

// K-contiguous operand rows [r0, r0+R) x bytes [128*st, 128*st+128).
// LDS row r (128 B) holds 16-byte piece p at position p ^ f(r),
// f(r) = (r%8) ^ ((r/8)%2).
template <int R, int NW = DNW>
__device__ inline void load_nt(const uint8_t *X, int64_t total, int64_t r0, int64_t KB,
                               int st, uint8_t *lds, int w, int lane) {
  const int64_t base = r0 * KB + (int64_t)st * 128;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(X + base, clamp_records(total - base));
  constexpr int PER_W = R / 8 / NW;
#pragma unroll
  for (int j = 0; j < PER_W; ++j) {
    const int blk = w * PER_W + j;
    const int r = blk * 8 + (lane >> 3);
    const int f = (r & 7) ^ ((r >> 3) & 1);
    const uint32_t voff = (uint32_t)r * (uint32_t)KB + (uint32_t)(((lane & 7) ^ f) << 4);
    dma16(rs, lds + blk * 1024, voff);
  }
}

// Transposed operand stored [K, Rtot] (rows contiguous): LDS holds 128 k-rows
// of R bytes; 16-byte column chunk c of k-row kk sits at position c ^ (kk%8).
template <int R, int NW = DNW>
__device__ inline void load_t(const uint8_t *X, int64_t total, int64_t c0, int64_t Rtot,
                              int st, uint8_t *lds, int w, int lane) {
  const int64_t base = (int64_t)st * 128 * Rtot + c0;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(X + base, clamp_records(total - base));
  constexpr int LPR = R / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int PER_W = 128 / RPI / NW;
#pragma unroll
  for (int j = 0; j < PER_W; ++j) {
    const int blk = w * PER_W + j;
    const int kk = blk * RPI + lane / LPR;
    const int chunk = (lane % LPR) ^ (kk & 7);
    const uint32_t voff = (uint32_t)kk * (uint32_t)Rtot + (uint32_t)(chunk << 4);
    dma16(rs, lds + blk * 1024, voff);
  }
}

// Preshuffled B: fragment (n-tile t, k-step ks) is contiguous (FP8: two 1 KiB
// halves, FP4: one 1 KiB block) in lane order; copied linearly.
template <bool FP4, int R = DBN, int NW = DNW>
__device__ inline void load_ps(const uint8_t *X, int64_t total, int64_t nt0, int64_t nks,
                               int st, uint8_t *lds, int w, int lane) {
  constexpr int FRAG = FP4 ? 1024 : 2048;
  const int64_t ks0 = FP4 ? 2 * (int64_t)st : (int64_t)st;
  const int64_t base = (nt0 * nks + ks0) * FRAG;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(X + base, clamp_records(total - base));
  constexpr int PER_W = (R / 16) * 2 / NW;
#pragma unroll
  for (int j = 0; j < PER_W; ++j) {
    const int idx = w * PER_W + j;
    const int t = idx >> 1, sub = idx & 1;
    const uint32_t voff = (uint32_t)(t * nks) * FRAG + sub * 1024 + lane * 16;
    dma16(rs, lds + idx * 1024, voff);
  }
}

// ---------------------------------------------------------------------------
// LDS -> register fragments for one 16-row tile and one 128-element K step.
// Matrix-core operand order (gfx950, 8-bit): lane (i = row, q = lane/16) holds
// k in [16q, 16q+16) then [64+16q, 64+16q+16); 4-bit: k in [32q, 32q+32).
// The lane's E8M0 scale covers 32-K block q of its row.

__device__ inline v8i frag_nt8(const uint8_t *region, int rloc, int lane) {
  const int i = lane & 15, q = lane >> 4;
  const int f = (i & 7) ^ (i >> 3);
  const uint8_t *row = region + (rloc + i) * 128;
  const v4i lo = lds_read16(row + ((q ^ f) << 4));
  const v4i hi = lds_read16(row + (((q + 4) ^ f) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__device__ inline v4i frag_nt4(const uint8_t *region, int rloc, int s, int lane) {
  const int i = lane & 15, q = lane >> 4;
  const int f = (i & 7) ^ (i >> 3);
  return lds_read16(region + (rloc + i) * 128 + (((4 * s + q) ^ f) << 4));
}

template <int R>
__device__ inline v8i frag_t8(const uint8_t *region, int cb, int lane) {
  const int i = lane & 15, q = lane >> 4;
  v2i p[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kk = 16 * q + 8 * (t & 1) + 64 * (t >> 1) + (i >> 1);
    p[t] = lds_read_tr8(region + kk * R + ((((cb >> 4) ^ (kk & 7))) << 4) + ((i & 1) << 3));
  }
  return (v8i){p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

__device__ inline v8i frag_ps8(const uint8_t *region, int t, int lane) {
  const v4i lo = lds_read16(region + t * 2048 + lane * 16);
  const v4i hi = lds_read16(region + t * 2048 + 1024 + lane * 16);
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__device__ inline v4i frag_ps4(const uint8_t *region, int t, int s, int lane) {
  return lds_read16(region + (t * 2 + s) * 1024 + lane * 16);
}

__device__ inline v8i widen(const v4i &v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// ---------------------------------------------------------------------------
// Epilogue: FP32 accumulators -> BF16 (RNE) -> LDS -> 16-byte row stores.
// Wave (wm, wn) owns rows [wm*BM/2, +BM/2) and columns [wn*BN/2, +BN/2) of the
// block tile; lane (i16, q) holds D[16a + i16][16b + 4q + r], r = 0..3 (the
// matrix-core result with the B tile as first operand).  In LDS, row m is
// BN*2 bytes and its 8-byte chunk c sits at position c ^ (m % 16).  Rows at
// or beyond row_lim and columns at or beyond N are not written.
template <int BM, int BN, int FM, int FN>
__device__ inline void store_tile(const v4f (&acc)[FM][FN], float alpha, uint8_t *cs,
                                  uint16_t *D, int64_t m0, int64_t n0, int64_t row_lim,
                                  int64_t N, int wm, int wn) {
  constexpr int ROWB = BN * 2;
  const int lane = threadIdx.x & 63, i16 = lane & 15, q = lane >> 4;
  __syncthreads();
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int m = wm * (BM / 2) + a * 16 + i16;
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int c = (wn * (BN / 2) + b * 16 + 4 * q) >> 2;
      const v4f v = acc[a][b];
      const uint32_t lo = pack_bf16x2(v.x * alpha, v.y * alpha);
      const uint32_t hi = pack_bf16x2(v.z * alpha, v.w * alpha);
      *(__attribute__((address_space(3))) v2i *)(__attribute__((address_space(3))) char *)(uintptr_t)(
          cs + m * ROWB + ((c ^ (m & 15)) << 3)) = (v2i){(int)lo, (int)hi};
    }
  }
  __syncthreads();
  constexpr int PAIRS = BN / 8;                 // 16-byte pairs per row
  constexpr int RPP = 256 / PAIRS;              // rows per pass (256 threads)
  const bool vec_ok = (N & 7) == 0;
#pragma unroll 4
  for (int it = 0; it < BM / RPP; ++it) {
    const int m = it * RPP + (int)threadIdx.x / PAIRS;
    const int j = (int)threadIdx.x % PAIRS;
    const int64_t gm = m0 + m, gn = n0 + 8 * j;
    const int pos = j ^ ((m & 15) >> 1);
    v4i v = lds_read16(cs + m * ROWB + (pos << 4));
    if (m & 1) v = (v4i){v.z, v.w, v.x, v.y};
    if (gm < row_lim) {
      uint16_t *dst = D + gm * N + gn;
      if (vec_ok && gn + 8 <= N) {
        *(v4i *)dst = v;
      } else {
        const uint32_t u[4] = {(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gn + e < N) dst[e] = (uint16_t)(u[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Block -> output tile.  Consecutive workgroups land on different XCDs
// (round-robin over 8); remap so that each XCD works on a compact band of
// tiles, then walk tiles in groups of 8 tile-rows for L2 reuse.
__device__ inline void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nb = tiles_m * tiles_n;
  int b = bid;
  if ((nb & 7) == 0) b = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int g = b / per_group;
  const int first = g * GM;
  const int rows = min(GM, tiles_m - first);
  const int in = b - g * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

template <int FA, int FB, int SMODE, bool TA, bool TB, bool PSB>
__global__ __launch_bounds__(256, 1) void dense_kernel(DenseArgs p) {
  constexpr bool FP4 = (FA == F_E2M1);
  constexpr int KS = FP4 ? 2 : 1;          // 128-element K steps per stage
  constexpr int FM = 8, FN = 8;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * DSTAGE];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int i16 = lane & 15, q = lane >> 4;
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * DBM, n0 = (int64_t)tn * DBN;
  const int64_t KB = FP4 ? p.K / 2 : p.K;   // bytes of K per row
  const int nst = (int)(KB / 128);
  const int64_t nks = p.K / 128;            // 128-element K steps

  v4f acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Scale sources (MX only): plain [rows, K/32] bytes, or preshuffled B.
  __amdgpu_buffer_rsrc_t rsa, rsb;
  if constexpr (SMODE == SM_MX) {
    rsa = make_rsrc(p.sA, clamp_records(p.sa_bytes));
    rsb = make_rsrc(p.sB, clamp_records(p.sb_bytes));
  }
  const int64_t sk32 = p.K / 32;
  const int64_t ngrp = (p.K + 511) / 512;
  uint32_t sa_n[FM][KS], sb_n[FN][KS];

  auto load_scales = [&](int st) {
    if constexpr (SMODE == SM_MX) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int64_t ks = (int64_t)st * KS + s;
#pragma unroll
        for (int a = 0; a < FM; ++a) {
          const int64_t row = m0 + wm * 128 + a * 16 + i16;
          sa_n[a][s] = buf_load_u32(rsa, (uint32_t)(row * sk32 + 4 * ks));
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          if constexpr (PSB) {
            const int64_t rt = (n0 + wn * 128) / 16 + b;
            sb_n[b][s] = buf_load_u32(rsb, (uint32_t)(((rt * ngrp + ks / 4) * 64 + lane) * 4));
          } else {
            const int64_t row = n0 + wn * 128 + b * 16 + i16;
            sb_n[b][s] = buf_load_u32(rsb, (uint32_t)(row * sk32 + 4 * ks));
          }
        }
      }
    }
  };

  auto load_stage = [&](int st, uint8_t *buf) {
    uint8_t *la = buf, *lb = buf + DBM * 128;
    if constexpr (TA) load_t<DBM>(p.A, p.a_bytes, m0, p.M, st, la, w, lane);
    else load_nt<DBM>(p.A, p.a_bytes, m0, KB, st, la, w, lane);
    if constexpr (PSB) load_ps<FP4>(p.B, p.b_bytes, n0 / 16, nks, st, lb, w, lane);
    else if constexpr (TB) load_t<DBN>(p.B, p.b_bytes, n0, p.N, st, lb, w, lane);
    else load_nt<DBN>(p.B, p.b_bytes, n0, KB, st, lb, w, lane);
  };

  if (nst > 0) {
    load_stage(0, smem);
    load_scales(0);
  }
  wait_vmem();
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    uint8_t *buf = smem + (st & 1) * DSTAGE;
    const uint8_t *la = buf, *lb = buf + DBM * 128;
    uint32_t sa_c[FM][KS], sb_c[FN][KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int a = 0; a < FM; ++a) sa_c[a][s] = sa_n[a][s];
#pragma unroll
      for (int b = 0; b < FN; ++b) sb_c[b][s] = sb_n[b][s];
    }
    // B fragments of this stage first; A fragments are read one 16-row tile
    // ahead of the matrix-core instructions that consume them.
    auto read_a = [&](int s, int a) -> v8i {
      if constexpr (FP4) return widen(frag_nt4(la, wm * 128 + a * 16, s, lane));
      else if constexpr (TA) return frag_t8<DBM>(la, wm * 128 + a * 16, lane);
      else return frag_nt8(la, wm * 128 + a * 16, lane);
    };
    auto read_b = [&](int s, int b) -> v8i {
      if constexpr (PSB) {
        if constexpr (FP4) return widen(frag_ps4(lb, wn * 8 + b, s, lane));
        else return frag_ps8(lb, wn * 8 + b, lane);
      } else if constexpr (FP4) return widen(frag_nt4(lb, wn * 128 + b * 16, s, lane));
      else if constexpr (TB) return frag_t8<DBN>(lb, wn * 128 + b * 16, lane);
      else return frag_nt8(lb, wn * 128 + b * 16, lane);
    };
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      v8i bf[FN];
#pragma unroll
      for (int b = 0; b < FN; ++b) bf[b] = read_b(s, b);
      if (s == 0 && st + 1 < nst) {
        load_stage(st + 1, smem + ((st + 1) & 1) * DSTAGE);
        load_scales(st + 1);
      }
      v8i af = read_a(s, 0);
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        v8i af_next;
        if (a + 1 < FM) af_next = read_a(s, a + 1);
        int sa = E8M0_ONE_X4;
        if constexpr (SMODE == SM_MX) sa = (int)(sa_c[a][s] >> (8 * q));
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          int sb = E8M0_ONE_X4;
          if constexpr (SMODE == SM_MX) {
            if constexpr (PSB) sb = (int)(sb_c[b][s] >> (8 * ((st * KS + s) & 3)));
            else sb = (int)(sb_c[b][s] >> (8 * q));
          }
          // First operand = B tile: the result lane holds 4 consecutive n.
          acc[a][b] = mfma_scaled<FB, FA>(bf[b], af, acc[a][b], sb, sa);
        }
        if (a + 1 < FM) af = af_next;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue
  float alpha = 1.0f;
  if constexpr (SMODE == SM_TENSOR) alpha = *(const float *)p.sA * *(const float *)p.sB;
  store_tile<DBM, DBN, FM, FN>(acc, alpha, smem, p.D, m0, n0, p.M, p.N, wm, wn);
}

}  // namespace mxg
