// Dense NT GEMM with a preshuffled B operand: the fast path for weights.
//
//   D[m,n] = sum_k a(m,k) b(n,k) on v_mfma_scale_f32_16x16x128_f8f6f4, FP32
//   accumulation, BF16 output.  MX operands pass their E8M0 block scales to
//   the instruction; tensor-wise operands use the neutral scale and the
//   epilogue multiplies by sA*sB.
//
// Why this shape: a 256x256 block tile needs ~32 bytes of operand per clock
// per CU at the matrix-core rate, and first touches of a tile come from the
// Infinity Cache/HBM with microseconds of latency, so about three K steps of
// operands must be in flight per CU -- more than LDS can hold for both
// operands.  So only A goes through LDS (a 4-deep ring of 32 KiB stages fed
// by buffer-load-to-LDS DMA), and B, preshuffled once into per-lane order,
// streams straight from global memory into registers three K steps ahead:
// the register file is B's staging buffer.  The four waves split the block
// tile by columns (each wave owns 256 rows x 64 columns), so no B fragment is
// loaded twice; every wave reads the whole A stage from LDS (64 B/clk/CU at
// the matrix-core rate).  One barrier per K step.
//
// Preshuffled B ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm": weights
// swizzled once into the MFMA B layout): column group cg = 64 rows of B, k
// step ks = 128 K values; chunk (cg, ks) is contiguous at (cg*nks + ks)*CGB:
//   FP8 (CGB = 8 KiB): + t*2048 + h*1024 + lane*16 holds row 64cg + 16t +
//       lane%16, k = 128ks + 64h + 16(lane/16) + [0,16)
//   FP4 (CGB = 4 KiB): + t*1024 + lane*16 holds packed bytes 64ks +
//       16(lane/16) + [0,16) of row 64cg + 16t + lane%16
// Preshuffled E8M0 scales of B: 32-bit word ((cg*ngrp + g)*64 + lane)*4 + t,
// byte j = scale of row 64cg + 16t + lane%16, 32-K block 16g + 4j + lane/16.
#pragma once
#include "dense.hpp"

namespace mxg {


// Epilogue for a wave tile of FM x FN 16x16 tiles at (row_off, col_off) of a
// BM x BN block tile; same LDS staging as store_tile.
template <int BM, int BN, int FM, int FN>
__device__ inline void store_tile_at(const v4f (&acc)[FM][FN], float alpha, uint8_t *cs,
                                     uint16_t *D, int64_t m0, int64_t n0, int64_t row_lim,
                                     int64_t N, int row_off, int col_off) {
  constexpr int ROWB = BN * 2;
  const int lane = threadIdx.x & 63, i16 = lane & 15, q = lane >> 4;
  __syncthreads();
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int m = row_off + a * 16 + i16;
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int c = (col_off + b * 16 + 4 * q) >> 2;
      const v4f v = acc[a][b];
      const uint32_t lo = pack_bf16x2(v.x * alpha, v.y * alpha);
      const uint32_t hi = pack_bf16x2(v.z * alpha, v.w * alpha);
      *(__attribute__((address_space(3))) v2i *)(__attribute__((address_space(3))) char *)(uintptr_t)(
          cs + m * ROWB + ((c ^ (m & 15)) << 3)) = (v2i){(int)lo, (int)hi};
    }
  }
  __syncthreads();
  constexpr int PAIRS = BN / 8;
  constexpr int RPP = 256 / PAIRS;
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

// vmcnt(n) with expcnt/lgkmcnt left alone (n <= 63).
template <int N>
__device__ inline void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The K loop.  Every LDS access of the loop goes through one restrict
// pointer per ring slot, so the compiler can prove that the DMA filling one
// slot does not alias the reads of another and does not stall those reads on
// it; reads of a slot still wait for that slot's own DMA.
template <int FA, int FB, int SMODE>
struct FastLoop {
  static constexpr bool FP4 = (FA == F_E2M1);
  static constexpr bool MX = (SMODE == SM_MX);
  static constexpr int KS = FP4 ? 2 : 1;       // 128-element K steps per stage
  static constexpr int PD = 2;                 // stages in flight ahead of use
  static constexpr int NS = PD + 1;            // ring slots (LDS for A, registers for B)
  static constexpr int FM = 16, FN = 4;        // wave tile 256 x 64
  static constexpr int ASTAGE = 256 * 128;
  // per slot: A scales [KS][256 rows][4 B], then B scales [4 waves][64 lanes][16 B]
  static constexpr int SA_BYTES = 256 * 4 * KS;
  static constexpr int SSTAGE = MX ? SA_BYTES + 4096 : 16;
  static constexpr int CGB = FP4 ? 4096 : 8192;
  // Vector-memory instructions each wave issues per stage: A DMA 8 (+ KS
  // A-scale DMAs), B fragments 8 (+ 1 B-scale load).  Every K step issues
  // exactly one stage (past the last stage against empty ranges, which read
  // nothing), so the number of loads newer than stage st is a constant.
  static constexpr int VM_STAGE = 8 + (MX ? KS : 0) + 8 + (MX ? 1 : 0);
  static constexpr int VM_NEWER = (PD - 1) * VM_STAGE;
  static_assert(VM_NEWER < 64, "vmcnt range");
  typedef typename std::conditional<FP4, v4i, v8i>::type bfrag_t;

  struct Ctx {
    const DenseArgs *p;
    int lane, w, q, nst;
    int64_t m0, KB, sk32;
    // Loop-invariant buffer resources (A rows from m0, this wave's B column
    // group, scales) and per-lane byte offsets; each load adds a uniform
    // offset, so the loop needs no per-load address registers.
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb, rzero;
    uint32_t vo_a[2];      // A piece offsets for even / odd 8-row blocks
    uint32_t vo_sa;        // A-scale row offset
    uint32_t vo_lane;      // lane * 16
  };

  __device__ static inline void issue(const Ctx &c, int st, uint8_t *__restrict__ ring,
                                      uint8_t *__restrict__ scl, bfrag_t (&bdst)[KS][FN]) {
    const bool real = st < c.nst;
    // A: rows m0 + [0, 256), bytes [128 st, 128 st + 128): 8 DMAs of 8 rows.
    const __amdgpu_buffer_rsrc_t ra = real ? c.ra : c.rzero;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = c.w * 8 + j;
      const uint32_t soff = (uint32_t)blk * 8u * (uint32_t)c.KB + (uint32_t)st * 128u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(ring + blk * 1024), 16,
                                               (int)c.vo_a[j & 1], (int)soff, 0, 0);
    }
    if constexpr (MX) {
      const __amdgpu_buffer_rsrc_t rsa = real ? c.rsa : c.rzero;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint32_t soff = (uint32_t)(((int64_t)st * KS + s) * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void *)(scl + s * 1024 + c.w * 256), 4,
                                                 (int)c.vo_sa, (int)soff, 0, 0);
      }
    }
    const __amdgpu_buffer_rsrc_t rb = real ? c.rb : c.rzero;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t kso = (uint32_t)(((int64_t)st * KS + s) * CGB);
#pragma unroll
      for (int t = 0; t < FN; ++t) {
        if constexpr (FP4) {
          bdst[s][t] = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rb, (int)c.vo_lane, (int)(kso + t * 1024), 0);
        } else {
          const v4i lo = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rb, (int)c.vo_lane, (int)(kso + t * 2048), 0);
          const v4i hi = (v4i)__builtin_amdgcn_raw_buffer_load_b128(rb, (int)c.vo_lane, (int)(kso + t * 2048 + 1024), 0);
          bdst[s][t] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
      }
    }
    if constexpr (MX) {
      const uint32_t soff = (uint32_t)((((int64_t)st * KS) / 4) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(real ? c.rsb : c.rzero,
                                               (lds_void *)(scl + SA_BYTES + c.w * 1024), 16,
                                               (int)c.vo_lane, (int)soff, 0, 0);
    }
  }

  __device__ static inline void compute(const Ctx &c, int st, const uint8_t *__restrict__ la,
                                        const uint8_t *__restrict__ ls,
                                        const bfrag_t (&bq)[KS][FN], v4f (&acc)[FM][FN]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      int sb[FN];
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        sb[b] = E8M0_ONE_X4;
        if constexpr (MX) {
          const uint32_t word = *(const __attribute__((address_space(3))) uint32_t *)(
              (const __attribute__((address_space(3))) char *)(uintptr_t)(ls + SA_BYTES + c.w * 1024 + c.lane * 16 + b * 4));
          sb[b] = (int)(word >> (8 * ((st * KS + s) & 3)));
        }
      }
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        v8i af;
        if constexpr (FP4) af = widen(frag_nt4(la, a * 16, s, c.lane));
        else af = frag_nt8(la, a * 16, c.lane);
        int sa = E8M0_ONE_X4;
        if constexpr (MX) {
          const uint32_t word = *(const __attribute__((address_space(3))) uint32_t *)(
              (const __attribute__((address_space(3))) char *)(uintptr_t)(ls + s * 1024 + (a * 16 + (c.lane & 15)) * 4));
          sa = (int)(word >> (8 * c.q));
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          v8i bfv;
          if constexpr (FP4) bfv = widen(bq[s][b]);
          else bfv = bq[s][b];
          acc[a][b] = mfma_scaled<FB, FA>(bfv, af, acc[a][b], sb[b], sa);
        }
      }
    }
  }

  // One K step: stage st is consumed from slot (ring_c, scl_c, bq_c); stage
  // st + PD is issued into the slot freed by step st - 1.
  __device__ static inline void step(const Ctx &c, int st, const uint8_t *__restrict__ ring_c,
                                     const uint8_t *__restrict__ scl_c, const bfrag_t (&bq_c)[KS][FN],
                                     uint8_t *__restrict__ ring_n, uint8_t *__restrict__ scl_n,
                                     bfrag_t (&bq_n)[KS][FN], v4f (&acc)[FM][FN]) {
    // Stage st has landed (this wave's part) once only the newer stages'
    // loads are outstanding; the barrier publishes every wave's DMA and
    // retires every wave's reads of the slot about to be refilled.
    wait_vmem_le<VM_NEWER>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    issue(c, st + PD, ring_n, scl_n, bq_n);
    compute(c, st, ring_c, scl_c, bq_c, acc);
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ static inline void run(const Ctx &c, v4f (&acc)[FM][FN],
                                    uint8_t *__restrict__ r0, uint8_t *__restrict__ r1,
                                    uint8_t *__restrict__ r2, uint8_t *__restrict__ s0,
                                    uint8_t *__restrict__ s1, uint8_t *__restrict__ s2) {
    static_assert(NS == 3, "three slots");
    bfrag_t b0[KS][FN], b1[KS][FN], b2[KS][FN];
    issue(c, 0, r0, s0, b0);
    issue(c, 1, r1, s1, b1);
    for (int st = 0; st < c.nst; st += NS) {
      step(c, st, r0, s0, b0, r2, s2, b2, acc);
      if (st + 1 < c.nst) step(c, st + 1, r1, s1, b1, r0, s0, b0, acc);
      if (st + 2 < c.nst) step(c, st + 2, r2, s2, b2, r1, s1, b1, acc);
    }
    wait_vmem_le<0>();
  }
};

template <int FA, int FB, int SMODE>
__global__ __launch_bounds__(256, 1) void dense_fast_kernel(DenseArgs p) {
  typedef FastLoop<FA, FB, SMODE> L;
  constexpr int ASTAGE = L::ASTAGE, SSTAGE = L::SSTAGE;
  // 128 KiB: the three-slot A ring uses 96 KiB; the epilogue uses it all.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * ASTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscl[L::NS * SSTAGE];

  typename L::Ctx c;
  c.p = &p;
  c.lane = threadIdx.x & 63;
  c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
  c.q = c.lane >> 4;
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  c.m0 = (int64_t)tm * 256;
  const int64_t n0 = (int64_t)tn * 256;
  c.KB = L::FP4 ? p.K / 2 : p.K;
  c.nst = (int)(c.KB / 128);
  c.sk32 = p.K / 32;
  const int64_t nks = p.K / 128;
  const int64_t cg = n0 / 64 + c.w;            // this wave's column group of B
  const int64_t bbase = cg * nks * L::CGB;
  const int64_t abase = c.m0 * c.KB;
  c.ra = make_rsrc(p.A + abase, clamp_records(p.a_bytes - abase));
  c.rb = make_rsrc(p.B + bbase, clamp_records(p.b_bytes - bbase));
  c.rzero = make_rsrc(p.B, 0);
  c.rsa = c.rzero;
  c.rsb = c.rzero;
  {
    const uint32_t r8 = (uint32_t)(c.lane >> 3), p8 = (uint32_t)(c.lane & 7);
    c.vo_a[0] = r8 * (uint32_t)c.KB + ((p8 ^ r8) << 4);
    c.vo_a[1] = r8 * (uint32_t)c.KB + ((p8 ^ r8 ^ 1u) << 4);
  }
  c.vo_lane = (uint32_t)c.lane * 16u;
  c.vo_sa = 0;
  if constexpr (L::MX) {
    const int64_t ngrp = (p.K + 511) / 512;
    const int64_t sabase = (c.m0 + 64 * c.w) * c.sk32;
    c.rsa = make_rsrc((const uint8_t *)p.sA + sabase, clamp_records(p.sa_bytes - sabase));
    c.vo_sa = (uint32_t)(c.lane * c.sk32);
    const int64_t sbase = cg * ngrp * 1024;
    c.rsb = make_rsrc((const uint8_t *)p.sB + sbase, clamp_records(p.sb_bytes - sbase));
  }

  v4f acc[L::FM][L::FN];
#pragma unroll
  for (int a = 0; a < L::FM; ++a)
#pragma unroll
    for (int b = 0; b < L::FN; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

  L::run(c, acc, smem, smem + ASTAGE, smem + 2 * ASTAGE, sscl, sscl + SSTAGE, sscl + 2 * SSTAGE);

  float alpha = 1.0f;
  if constexpr (SMODE == SM_TENSOR) alpha = *(const float *)p.sA * *(const float *)p.sB;
  store_tile_at<256, 256, L::FM, L::FN>(acc, alpha, smem, p.D, c.m0, n0, p.M, p.N, 0, c.w * 64);
}

}  // namespace mxg
