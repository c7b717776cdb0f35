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
// Block tile 256x256, eight waves (two per SIMD) in a 2x4 grid (128x64 per
// wave, 8x4 matrix-core tiles of 16x16).  Each stage holds 128 bytes of K per
// row of A and B (one 128-element K step for FP8, two for FP4) in LDS, double
// buffered, plus the MX scales of a group of four K steps.  Operands travel
// global -> LDS by buffer-load-to-LDS DMA, 16 bytes per lane, issued from
// inline assembly with explicit waits, into XOR-swizzled rows so that the
// fragment reads are free of bank conflicts.  Transposed operands (the 'T'
// side of NN/TN) are kept in LDS k-major and read with the transposing
// ds_read_b64_tr_b8 (packed E2M1: ds_read_b64_tr_b4).  The grid is persistent (one workgroup per compute
// unit): the tiles of a workgroup share one K pipeline, the next tile's first
// stage streams in during the current tile's last K step, and a finished
// tile is stored from registers (BF16, 16-byte rows after a cross-lane
// exchange) during the next tile's first K step.
#pragma once
#include "common.hpp"

namespace mxg {

// Scale modes: MX (E8M0 per 32 K values, applied by the matrix-core
// instruction), tensor-wise (one FP32 per operand, applied in the epilogue),
// groupwise (the grouped GEMM: FP32 per row and 128-K block of A, per 128 x
// 128 block of each group's B, applied in software after every 128-K step),
// and none with the grouped GEMM's addressing (the BF16 grouped GEMM).
enum : int { SM_MX = 0, SM_TENSOR = 1, SM_GROUP = 2, SM_GNONE = 3 };

struct DenseArgs {
  const uint8_t *A, *B;
  const void *sA, *sB;            // groupwise: x_scale and w_scale (FP32)
  uint16_t *D;
  int64_t M, N, K;                // groupwise: M = totM, N and K per group
  int64_t a_bytes, b_bytes, sa_bytes, sb_bytes;
  int tiles_m, tiles_n;
  const int64_t *m_sizes;         // groupwise only
  int G;                          // groupwise only
  int tail_grid, tail_rounds;     // groupwise only: see grouped_split_end
  const uint16_t *bias;           // fused epilogue: BF16 [N] or null
  int act;                        // fused epilogue: ACT_*
};

// One output tile: origin, the row limit of its stores (M, or the end of its
// group) and, for the grouped GEMM, its group (index, first row, rows).
struct TileId {
  int64_t m0, n0, lim, start, mg;
  int g;
};

constexpr int DBM = 256, DBN = 256;
constexpr int DNW8 = 8;           // waves of the pipelined dense kernel

// LDS placement of staged tiles, chosen for gfx950's LDS, which serves a
// wave's read in phases over 64 four-byte banks (256 B):
// - ds_read_b128 in four phases of 16 lanes: {0-3, 12-15, 20-23, 24-27},
//   {4-11, 16-19, 28-31} and the same two sets plus 32;
// - ds_read_b64 and ds_read_b64_tr_b8 in two phases, lanes 0-31 and 32-63.
// K-contiguous tile rows are 128 B: 16-byte piece p of row r sits at position
// p ^ kswz(r).  A fragment read gives lane (i, q) piece q or q + 4 of row i
// (rows 128 B apart, so row parity picks the bank half); every phase pairs
// rows {0-3, 12-15} with {4-11} at pieces differing in bit 0, and r & 6 gives
// each parity class of either set four distinct even XOR values, so the
// phase's 16 lanes land on 16 distinct 16-byte bank groups.
__device__ constexpr int kswz(int r) { return r & 6; }

// Transposed tiles (k-rows of 256 B): 16-byte chunk c of k-row kk sits at
// c ^ tswz(kk).  A transposing fragment read has the 32 lanes of a phase read
// k-rows kk0 + 16 q' + j (q' = 0, 1; j < 8; kk0 a multiple of 8 with bit 4
// clear) at 8-byte offset i % 2; a 4-bit XOR of j and q' spreads them over
// all 32 eight-byte bank groups.
__device__ constexpr int tswz(int kk) { return (kk & 7) | ((kk & 16) >> 1); }

// Transposed packed E2M1 tiles (k-rows of 128 B: 256 columns, two per
// byte): 16-byte piece p of k-row kk sits at p ^ fswz(kk).  A fragment read
// (ds_read_b64_tr_b4) has the 32 lanes of a phase read 8 bytes from k-rows
// k0 + i (lanes 0-15) and k0 + 32 + i (lanes 16-31), i < 16.  Rows 128 B
// apart fall in the two bank halves by parity, and fswz gives the 8 rows of
// one parity in each run of 16 eight distinct pieces; the two lane groups
// read the two 8-byte halves of a piece (the column chunks of two adjacent
// tiles, see rdt4_pair), so the phase's 32 reads hit 32 distinct bank pairs.
__device__ constexpr int fswz(int kk) { return (kk >> 1) & 7; }

// ---------------------------------------------------------------------------
// Matrix-core operand order (gfx950) of a 16-row tile and a 128-element K
// step: 8-bit, lane (i = row, q = lane/16) holds k in [16q, 16q+16) then
// [64+16q, 64+16q+16); 4-bit, k in [32q, 32q+32) in the low half of the
// operand register (widen).  The lane's E8M0 scale covers 32-K block q of its
// row.
__device__ inline v8i widen(const v4i &v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// vmcnt(n) with expcnt/lgkmcnt left alone (n <= 63).
template <int N>
__device__ inline void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The dense kernel: block tile 256 x 256, eight waves in a 2 x 4 grid (wave
// tile 128 x 64, 8 x 4 matrix-core tiles, 128 accumulators), two waves per
// SIMD so that one wave's LDS or barrier stall is covered by the other's
// matrix work.  Two LDS stages of 128 bytes of K per row for A and B (plus
// MX scales) are double buffered; every K step streams the next stage in by
// DMA while the current one feeds the matrix cores.
//
// The kernel is persistent: one workgroup per compute unit walks a list of
// output tiles, and the K steps of consecutive tiles form one unbroken
// pipeline.  The stage after a tile's last K step is the first stage of the
// next tile, and the finished tile's accumulators go out as BF16 straight
// from registers while that stage streams in, so no compute unit idles on an
// epilogue, a workgroup launch or a cold first stage between tiles.
//
template <int FA, int FB, int SMODE, bool TA, bool TB, bool PSB, bool FUSE = false>
struct DenseLoop {
  static constexpr bool FP4 = (FA == F_E2M1);
  static constexpr bool MX = (SMODE == SM_MX);
  static constexpr bool GROUP = (SMODE == SM_GROUP);
  static constexpr bool GROUPED = GROUP || SMODE == SM_GNONE;   // B of group g at rows g N
  static constexpr bool BF = (FA == F_BF16);    // BF16: a 128-byte K chunk is 64 elements
  static_assert(BF == (FB == F_BF16) && (!BF || (SMODE == SM_GNONE && !TA && !TB)), "BF16 operands");
  static constexpr bool SCALED = MX || GROUP;    // scales staged through LDS
  static constexpr int NW = DNW8;
  static constexpr int KS = FP4 ? 2 : 1;        // 128-element K steps per stage
  static constexpr int FM = 8, FN = 4;          // wave tile 128 x 64
  static constexpr int AB = DBM * 128;          // A bytes per stage
  static constexpr int STAGE = (DBM + DBN) * 128;
  // MX scales arrive in groups of four K steps (16 bytes per row): A rows
  // at SA_OFF + 16 row, B rows (or, preshuffled, B column groups of 1 KiB)
  // at SB_OFF.  Groupwise scales in the same groups of four K steps: the
  // tile's 256 activation scales of K step j at SA_OFF + 1024 j + 4 row,
  // the weight block scales of its two 128-column blocks c at SB_OFF +
  // 16 c + 4 j.  Two group slots.
  static constexpr int SA_OFF = 0, SB_OFF = 4096;
  static constexpr int SGROUP = SCALED ? 8192 : 0;
  // LDS: [A slot 0][A slot 1][B slot 0][B slot 1][scales slot 0][slot 1].
  // A read offset within either slot then fits the 16-bit offset field of a
  // DS instruction on top of one per-lane base register per operand.
  static constexpr int B_REG = 2 * AB, S_REG = 4 * AB;
  // Fused epilogue: the BF16 bias of a tile's 256 columns, two slots by the
  // parity of the tile's index (tile t's bias is read while tile t + 1's
  // first K step stores tile t, and replaced by tile t + 2's).
  static constexpr int BIAS_OFF = S_REG + 2 * SGROUP, BIAS_SLOT = DBN * 2;
  static constexpr int LDS_BYTES = BIAS_OFF + (FUSE ? 2 * BIAS_SLOT : 0);
  static constexpr int CGB = FP4 ? 4096 : 8192;
  // Operand tile kinds in LDS: K-contiguous rows, transposed 8-bit k-rows,
  // transposed packed E2M1 k-rows.
  static constexpr int OP_K = 0, OP_T8 = 1, OP_T4 = 2;
  static constexpr int OPA = TA ? (FP4 ? OP_T4 : OP_T8) : OP_K;
  static constexpr int OPB = TB ? (FP4 ? OP_T4 : OP_T8) : OP_K;
  static constexpr bool PIN = FP4 || (!TA && !TB && (PSB || !MX));

  // Loop-invariant state.  Every global load of the loop is one buffer
  // instruction: a resource fixed for the tile, a per-lane offset fixed for
  // the kernel (VGPR) and a uniform per-stage offset (SGPR).
  struct Ctx {
    const DenseArgs *p;
    int lane, w, wm, wn, i16, q, nst;
    int64_t KB, sk32, nks, ngrp;
    uint32_t vo_a[2], vo_b[2];     // operand DMA offsets (by block parity)
    uint32_t vo_s;                 // scale DMA offset
    uint32_t lds0;                 // LDS address of the kernel's LDS block (uniform)
  };


  // Per-kernel state of a workgroup: wave and lane indices, the per-lane
  // DMA offsets, the LDS block.
  __device__ static inline void init(Ctx &c, const DenseArgs &p, uint8_t *smem) {
    c.p = &p;
    c.lane = threadIdx.x & 63;
    c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    c.wm = c.w >> 2;
    c.wn = c.w & 3;
    c.i16 = c.lane & 15;
    c.q = c.lane >> 4;
    c.KB = BF ? 2 * p.K : (FP4 ? p.K / 2 : p.K);
    c.nst = (int)(c.KB / 128);
    c.sk32 = p.K / 32;
    c.nks = BF ? c.KB / 128 : p.K / 128;
    c.ngrp = (p.K + 511) / 512;
    dma_offsets(OPA, c.lane, c.w, c.KB, p.M, c.vo_a);
    dma_offsets(OPB, c.lane, c.w, c.KB, p.N, c.vo_b);
    c.vo_s = 0;
    if constexpr (MX) {
      if (c.w < 4 || !PSB) c.vo_s = (uint32_t)(c.lane * c.sk32);
      else c.vo_s = (uint32_t)(c.lane * 16);
    } else if constexpr (GROUP) {
      // waves 0-3: one activation scale per lane; wave 4: lane l reads the
      // weight block scale of column block (l / 4) % 2, K step l % 4
      if (c.w < 4) c.vo_s = (uint32_t)(c.lane * 4);
      else c.vo_s = (uint32_t)(((c.lane >> 2) & 1) * c.nks * 4 + (c.lane & 3) * 4);
    }
    c.lds0 = lds_addr(smem);
  }

  // The DMA sources of one output tile (uniform).
  struct Tile {
    int64_t m0, n0, lim;
    u32x4 ra, rb, rs;              // rs: this wave's scale source
    uint32_t soff, mg4;            // groupwise: this wave's scale offset, 4 * group rows
    int bslot;                     // fused epilogue: bias slot of the tile
  };

  __device__ static inline void set_tile(const Ctx &c, const TileId &id, Tile &t) {
    const DenseArgs &p = *c.p;
    const int64_t m0 = id.m0, n0 = id.n0;
    t.m0 = m0;
    t.n0 = n0;
    t.lim = id.lim;
    // A: rows m0.. (K-contiguous) or columns m0.. of [K, M] (packed E2M1:
    // byte m0 / 2 of each k-row); B likewise.
    const int64_t abase = TA ? (FP4 ? m0 / 2 : m0) : m0 * c.KB;
    t.ra = rsrc4(p.A + abase, clamp_records(p.a_bytes - abase));
    // Preshuffled B: the whole buffer (it holds every column group of every
    // 256-column tile, padding included); the offsets below stay inside it.
    // Grouped: group g's weights are rows [g N, g N + N) of one [G N, K]
    // operand; the resource starts at the tile's first row (plain) or column
    // group (preshuffled), and every offset from there is range-checked.
    int64_t bbase;
    if constexpr (GROUPED) bbase = PSB ? ((int64_t)id.g * p.N + n0) / 64 * c.nks * CGB : ((int64_t)id.g * p.N + n0) * c.KB;
    else if constexpr (PSB) bbase = 0;
    else bbase = TB ? (FP4 ? n0 / 2 : n0) : n0 * c.KB;
    t.rb = rsrc4(p.B + bbase, clamp_records(p.b_bytes - bbase));
    t.rs = (u32x4){0u, 0u, 0u, 0u};
    t.soff = 0;
    t.mg4 = 0;
    t.bslot = 0;
    if constexpr (GROUP) {
      // waves 0-3: activation scales, per-group block layout (row r of the
      // group at start*nkb + (r - start) + kb*mg); wave 4: the weight block
      // scales of group g, [G, N/128, K/128]
      if (c.w < 4) {
        t.rs = rsrc4(p.sA, clamp_records(p.sa_bytes));
        t.soff = (uint32_t)((id.start * c.nks + (m0 - id.start)) * 4);
        t.mg4 = (uint32_t)(id.mg * 4);
      } else {
        t.rs = rsrc4(p.sB, clamp_records(p.sb_bytes));
        t.soff = (uint32_t)((((int64_t)id.g * (p.N / 128) + n0 / 128) * c.nks) * 4);
      }
    }
    if constexpr (MX) {
      if (c.w < 4) {
        const int64_t b = (m0 + 64 * c.w) * c.sk32;
        t.rs = rsrc4((const uint8_t *)p.sA + b, clamp_records(p.sa_bytes - b));
      } else if constexpr (PSB) {
        const int64_t b = (n0 / 64 + (c.w - 4)) * c.ngrp * 1024;
        t.rs = rsrc4((const uint8_t *)p.sB + b, clamp_records(p.sb_bytes - b));
      } else {
        const int64_t b = (n0 + 64 * (c.w - 4)) * c.sk32;
        t.rs = rsrc4((const uint8_t *)p.sB + b, clamp_records(p.sb_bytes - b));
      }
    }
  }

  // Per-lane offsets of the 1 KiB wave DMAs of an operand tile.
  //  K-contiguous rows (256 rows x 128 B): DMA block blk covers rows
  //    8blk + lane/8; LDS position p of row r holds 16-byte piece
  //    p ^ kswz(r), so the lane reads piece (lane%8) ^ kswz(lane/8).
  //    Uniform part of the offset: blk*8*KB + 128*st.
  //  transposed (128 k-rows x 256 B): DMA block blk = 4w + j covers k-rows
  //    4blk + lane/16; position c of k-row kk holds column chunk c ^ tswz(kk),
  //    so the lane reads chunk (lane%16) ^ tswz(4blk + lane/16), which
  //    depends on j%2 (vo[j%2]) and w%2.  Uniform part: (4blk + 128 st) * Rtot.
  //  transposed packed E2M1 (256 k-rows x 128 B, Rtot/2 bytes per k-row in
  //    memory): DMA block blk covers k-rows 8blk + lane/8; position p of
  //    k-row kk holds piece p ^ fswz(kk), which depends on blk%2 (vo[j%2]).
  //    Uniform part: (8blk + 256 st) * Rtot/2.
  __device__ static inline void dma_offsets(int kind, int lane, int w, int64_t KB, int64_t Rtot,
                                            uint32_t (&vo)[2]) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      if (kind == OP_T4) {
        const int r8 = lane >> 3;
        vo[par] = (uint32_t)(r8 * (Rtot / 2)) + (uint32_t)(((lane & 7) ^ fswz(8 * par + r8)) << 4);
      } else if (kind == OP_T8) {
        // DMA j of wave w covers k-rows 16w + 4j .. +3 of the stage
        const int kk = 16 * (w & 1) + par * 4 + (lane >> 4);
        vo[par] = (uint32_t)((lane >> 4) * Rtot) + (uint32_t)(((lane & 15) ^ tswz(kk)) << 4);
      } else {
        const int r8 = lane >> 3;
        vo[par] = (uint32_t)(r8 * KB) + (uint32_t)(((lane & 7) ^ kswz(r8)) << 4);
      }
    }
  }

  // 1 KiB DMAs J0 .. J1-1 (of four) of this wave into the tile at LDS
  // address `tile`.  The whole offset goes through the range check (the
  // resource ends where the operand ends), so rows past M (N), and columns
  // past the end of a transposed operand's last k-row, read zeros.
  template <int KIND, int J0, int J1>
  __device__ static inline void load_tile(const Ctx &c, const u32x4 &r, const uint32_t (&vo)[2],
                                          int64_t KB, int64_t Rtot, int st, uint32_t tile) {
    const uint32_t base = tile + (uint32_t)c.w * 4096u;
    auto add = [&](int blk) {
      if constexpr (KIND == OP_T4) return (uint32_t)((8 * blk + 256 * (int64_t)st) * (Rtot / 2));
      else if constexpr (KIND == OP_T8) return (uint32_t)((4 * blk + 128 * (int64_t)st) * Rtot);
      else return (uint32_t)(blk * 8 * KB + 128 * (int64_t)st);
    };
    static_for<J0, J1>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      dma_asm_v<16, j * 1024>(base, r, vo[j & 1], add(c.w * 4 + j));
    });
  }

  // DMA of stage st of tile t (operands and MX scales) into ring slot si
  // (operands) and scale slot gs.  PART selects a part of it (0, 1: the A
  // tile's first and second halves; 2: B's first half; 3: B's second half
  // and the scales; 4: the scales alone); -1 issues everything.
  template <int PART = -1>
  __device__ static inline void issue(const Ctx &c, const Tile &t, int st, int si, int gs) {
    const DenseArgs &p = *c.p;
    const uint32_t slot = c.lds0 + (uint32_t)si * AB;
    constexpr bool ALL = PART < 0;
    if constexpr (ALL || PART == 0) load_tile<OPA, 0, 2>(c, t.ra, c.vo_a, c.KB, p.M, st, slot);
    if constexpr (ALL || PART == 1) load_tile<OPA, 2, 4>(c, t.ra, c.vo_a, c.KB, p.M, st, slot);
    if constexpr (ALL || PART == 2 || PART == 3) {
      constexpr int J0 = (PART == 3) ? 2 : 0, J1 = (PART == 2) ? 2 : 4;
      if constexpr (PSB && GROUPED) {
        // column group (4w + j)/8 = w/2, KiB (4w + j)%8 = 4(w%2) + j, from
        // the tile's first column group, range-checked
        const uint32_t add0 = (uint32_t)(((c.w >> 1) * c.nks + st) * CGB) + (uint32_t)(c.w & 1) * 4096u;
        const uint32_t base = slot + B_REG + (uint32_t)c.w * 4096u;
        static_for<J0, J1>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          dma_asm_v<16, j * 1024>(base, t.rb, (uint32_t)(c.lane * 16), add0 + j * 1024);
        });
      } else if constexpr (PSB) {
        // column group (4w + j)/8 = w/2, KiB (4w + j)%8 = 4(w%2) + j
        const uint32_t soff0 = (uint32_t)((t.n0 / 64 * c.nks + (FP4 ? 2 * (int64_t)st : st)) * CGB) +
                               (uint32_t)((c.w >> 1) * c.nks * CGB) + (uint32_t)(c.w & 1) * 4096u;
        const uint32_t base = slot + B_REG + (uint32_t)c.w * 4096u;
        const u32x4 rb = t.rb;
        static_for<J0, J1>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          dma_asm<16, j * 1024>(base, rb, (uint32_t)(c.lane * 16), soff0 + j * 1024);
        });
      } else {
        load_tile<OPB, J0, J1>(c, t.rb, c.vo_b, c.KB, p.N, st, slot + B_REG);
      }
    }
    if constexpr (FUSE && (ALL || PART == 3 || PART == 4)) {
      // with the tile's first stage: its 256 BF16 bias values (two 256-byte
      // DMAs by wave 3; columns past N read zeros).  Without a bias (an
      // activation alone) the resource is empty: the DMAs write zeros and
      // read no memory.
      if (st == 0 && c.w == 3) {
        const u32x4 rb = p.bias ? rsrc4(p.bias + t.n0, clamp_records(2 * (p.N - t.n0)))
                                : rsrc4(p.D, 0u);
        const uint32_t dst = c.lds0 + BIAS_OFF + (uint32_t)t.bslot * BIAS_SLOT;
        dma_asm_v<4, 0>(dst, rb, (uint32_t)(c.lane * 4), 0u);
        dma_asm_v<4, 256>(dst, rb, (uint32_t)(c.lane * 4), 256u);
      }
    }
    if constexpr (GROUP && (ALL || PART == 3 || PART == 4)) {
      // With the first stage of each group of four K steps: waves 0-3 the
      // 256 activation scales of K step 4 grp + w (four 256-byte DMAs of
      // 64 rows), wave 4 the 2 x 4 weight block scales (lane l: column
      // block (l / 4) % 2, K step l % 4).  Offsets past the last K block or
      // the buffer read zeros or scales no output uses.
      if ((st & 3) == 0) {
        const uint32_t grp = (uint32_t)(st / 4);
        const uint32_t dst = c.lds0 + S_REG + (uint32_t)gs * SGROUP;
        if (c.w < 4) {
          const uint32_t add = t.soff + (4u * grp + (uint32_t)c.w) * t.mg4;
          static_for<0, 4>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            dma_asm_v<4, j * 256>(dst + SA_OFF + (uint32_t)c.w * 1024u, t.rs, c.vo_s, add + j * 256);
          });
        } else if (c.w == 4) {
          dma_asm_v<4>(dst + SB_OFF, t.rs, c.vo_s, t.soff + grp * 16u);
        }
      }
    }
    if constexpr (MX && (ALL || PART == 3 || PART == 4)) {
      // With the first stage of each group of four K steps, scale slot gs
      // receives the group's scales: waves 0-3 the A rows 64w.. (16 bytes
      // each), waves 4-7 the B rows 64(w-4).. or, preshuffled, column group
      // w-4 (1 KiB: four 16-row subtiles x 64 lanes x one word).
      if (((st * KS) & 3) == 0) {
        const uint32_t grp = (uint32_t)(st * KS / 4);
        const uint32_t dst = c.lds0 + S_REG + (uint32_t)gs * SGROUP + (c.w < 4 ? SA_OFF : SB_OFF) +
                             (uint32_t)(c.w & 3) * 1024u;
        const uint32_t soff = (PSB && c.w >= 4) ? grp * 1024u : grp * 16u;
        dma_asm<16>(dst, t.rs, c.vo_s, soff);
      }
    }
  }

  // The same stage DMA with the operand tiles issued by waves 4-7 alone
  // (K-contiguous operands): wave 4 + v takes A blocks 8v .. 8v + 7 and, of
  // B, blocks 8v .. 8v + 7 or preshuffled column group v.  The MX scales stay
  // one DMA per wave.  Each SIMD runs one wave of each half of the
  // workgroup, so one of its two waves reaches its first matrix-core
  // instruction right after the barrier while the other queues the ~16
  // DMAs of 1 KiB whose issue the address path paces.
  __device__ static inline void issue_hi(const Ctx &c, const Tile &t, int st, int si, int gs) {
    static_assert(!TA && !TB, "K-contiguous operands");
    const uint32_t slot = c.lds0 + (uint32_t)si * AB;
    if (c.w >= 4) {
      const int v = c.w - 4;
      const uint32_t abase = slot + (uint32_t)v * 8192u;
      static_for<0, 8>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        dma_asm_v<16, j * 1024>(abase, t.ra, c.vo_a[0], (uint32_t)((v * 8 + j) * 8 * c.KB + 128 * (int64_t)st));
      });
      const uint32_t bbase = slot + B_REG + (uint32_t)v * 8192u;
      if constexpr (PSB && GROUPED) {
        // column group v of the tile, range-checked (the last tile of the
        // stack may have fewer than four)
        const uint32_t add0 = (uint32_t)((v * c.nks + st) * CGB);
        static_for<0, 8>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          dma_asm_v<16, j * 1024>(bbase, t.rb, (uint32_t)(c.lane * 16), add0 + j * 1024);
        });
      } else if constexpr (PSB) {
        const uint32_t soff0 = (uint32_t)(((t.n0 / 64 + v) * c.nks + (FP4 ? 2 * (int64_t)st : st)) * CGB);
        const u32x4 rb = t.rb;
        static_for<0, 8>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          dma_asm<16, j * 1024>(bbase, rb, (uint32_t)(c.lane * 16), soff0 + j * 1024);
        });
      } else {
        static_for<0, 8>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          dma_asm_v<16, j * 1024>(bbase, t.rb, c.vo_b[0], (uint32_t)((v * 8 + j) * 8 * c.KB + 128 * (int64_t)st));
        });
      }
    }
    issue<4>(c, t, st, si, gs);               // the MX scales only
  }

  __device__ static inline uint32_t lds_u32(const uint8_t *p) { return lds_load_u32(p); }

  // Per-lane LDS byte offsets of the fragment reads, fixed for the kernel.
  // Each read is then lane offset + a compile-time constant (slot, tile,
  // half), which the compiler folds into the 16-bit offset field of the DS
  // instruction (the lane offsets are masked so that it knows they are
  // small and non-negative), instead of keeping one address register per
  // fragment and slot.
  static constexpr uint32_t LMASK = 0x3FFFFu;
  struct Lanes {
    uint32_t a[2], b[2];           // FP8 K-contiguous / preshuffled: the two 16-byte halves;
                                   // FP4: the two k steps of the stage
    uint32_t at, bt;               // transposed: 8-byte piece 0 of tile 0 (packed E2M1:
                                   // k-row 32q + i, column chunk of tile 0)
    uint32_t sa, sb;               // scale words
  };

  __device__ static inline void lane_offsets(const Ctx &c, Lanes &L) {
    const int i = c.i16, q = c.q;
    const int f = kswz(i);
    // K-contiguous tile rows: row r at r*128, piece p at (p ^ kswz(r))*16.
    // FP8: halves h hold pieces q and q+4; FP4: k step h holds piece 4h+q.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = FP4 ? 4 * h + q : q + 4 * h;
      L.a[h] = ((uint32_t)((c.wm * 128 + i) * 128 + ((piece ^ f) << 4))) & LMASK;
      if constexpr (PSB) L.b[h] = ((uint32_t)(B_REG + c.wn * 8192 + (FP4 ? 0 : h * 1024) + c.lane * 16)) & LMASK;
      else L.b[h] = ((uint32_t)(B_REG + (c.wn * 64 + i) * 128 + ((piece ^ f) << 4))) & LMASK;
    }
    // Transposed tiles (256 B per k-row): piece 0 of tile 0.  Piece t sits
    // in k-row kk + 8 (t & 1) + 64 (t >> 1), whose swizzle tswz is that of kk
    // (neither step reaches bits 0-2 or bit 4 of kk = 16 q + i / 2), so it is
    // 0, 2048, 16384 or 18432 bytes further (rdt).  Tile x sits x 16-byte
    // chunks further; the
    // chunk index is XOR-swizzled by tswz(kk) and the wave's first chunk (8wm
    // or 4wn) is aligned to the tile count, so its offset is the tile-0
    // offset ^ (x << 4), and XOR on bits 4-6 commutes with adding those
    // distances (multiples of 2048).
    if constexpr (FP4) {
      // Packed E2M1 k-rows (128 B): tile x of the wave covers 16 columns, the
      // 8-byte chunk c0 + x (A: c0 = 8 wm, B: c0 = 4 wn), half x % 2 of
      // 16-byte piece (c0 + x) / 2.  Lane (i, q) reads k-row 32 q + i (+ 16
      // for the second half of its 32 K values, + 128 for the stage's second
      // K step), whose swizzle fswz is i / 2 in all of them; c0 / 2 has bits
      // 0-1 clear, so piece (c0/2 + x/2) ^ (i/2) = (c0/2 ^ i/2) ^ x/2.  Lanes
      // of odd q start at the other half (bit 3), see rdt4_pair.
      const int kk = 32 * q + i;
      const int half = (q & 1) << 3;
      L.at = ((uint32_t)(kk * 128 + (((c.wm * 4) ^ fswz(kk)) << 4) + half)) & LMASK;
      L.bt = ((uint32_t)(B_REG + kk * 128 + (((c.wn * 2) ^ fswz(kk)) << 4) + half)) & LMASK;
    } else {
      const int kk = 16 * q + (i >> 1);
      const int ca = c.wm * 8, cb = c.wn * 4;
      L.at = ((uint32_t)(kk * 256 + ((ca ^ tswz(kk)) << 4) + ((i & 1) << 3))) & LMASK;
      L.bt = ((uint32_t)(B_REG + kk * 256 + ((cb ^ tswz(kk)) << 4) + ((i & 1) << 3))) & LMASK;
    }
    if constexpr (GROUP) {
      // activation scale of row wm*128 + 16a + i (K step j at +1024 j), the
      // weight block scale of the wave's 64 columns (block wn/2; +4 j)
      L.sa = ((uint32_t)(S_REG + SA_OFF + (c.wm * 128 + i) * 4)) & LMASK;
      L.sb = ((uint32_t)(S_REG + SB_OFF + (c.wn >> 1) * 16)) & LMASK;
      return;
    }
    L.sa = ((uint32_t)(S_REG + SA_OFF + (c.wm * 128 + i) * 16)) & LMASK;
    if constexpr (PSB) L.sb = ((uint32_t)(S_REG + SB_OFF + c.wn * 1024 + c.lane * 4)) & LMASK;
    else L.sb = ((uint32_t)(S_REG + SB_OFF + (c.wn * 64 + i) * 16)) & LMASK;
  }

  __device__ static inline v8i rd8(const uint8_t *base, uint32_t lo, uint32_t hi, int imm) {
    const v4i x = lds_read16(base + lo + imm);
    const v4i y = lds_read16(base + hi + imm);
    return (v8i){x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
  }

  // The four 8-byte pieces t of a transposed fragment: k-rows 8 (t & 1) +
  // 64 (t >> 1) after the lane's first, at fixed distances from it.
  __device__ static inline v8i rdt(const uint8_t *base, uint32_t off) {
    v2i p0 = lds_read_tr8(base + off);
    v2i p1 = lds_read_tr8(base + off + 2048);
    v2i p2 = lds_read_tr8(base + off + 16384);
    v2i p3 = lds_read_tr8(base + off + 18432);
    return (v8i){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  }

  // Transposed packed E2M1 fragments of tiles x and x + 1 (x even) in K
  // step s of the stage.  Each fragment is two 16 x 16 nibble transposes
  // (k-rows 32q + i, then 32q + 16 + i): lane (i, q) receives column i at
  // k = 32q .. 32q + 15, then 32q + 16 .. 32q + 31, the matrix-core operand
  // order of a 4-bit fragment.  The two tiles' chunks are the two halves of
  // one 16-byte piece; lanes of even q read tile x's half in the first pair
  // of reads and tile x + 1's in the second, lanes of odd q the reverse (so
  // that every read's phase covers both halves, free of bank conflicts), and
  // a per-lane select puts each tile's data in its fragment.
  __device__ static inline void rdt4_pair(const uint8_t *base, uint32_t off, int x, int s, v8i &f0, v8i &f1) {
    const uint32_t o0 = (off ^ ((uint32_t)(x >> 1) << 4)) + (uint32_t)s * 16384u;
    const uint32_t o1 = (off ^ (((uint32_t)(x >> 1) << 4) | 8u)) + (uint32_t)s * 16384u;
    const v2i a0 = lds_read_tr4(base + o0), a1 = lds_read_tr4(base + o0 + 2048);
    const v2i b0 = lds_read_tr4(base + o1), b1 = lds_read_tr4(base + o1 + 2048);
    const v4i u = (v4i){a0.x, a0.y, a1.x, a1.y}, v = (v4i){b0.x, b0.y, b1.x, b1.y};
    const bool odd = ((__lane_id() >> 4) & 1) != 0;
    f0 = widen(odd ? v : u);
    f1 = widen(odd ? u : v);
  }

  // Epilogue of one finished tile: its accumulators (times alpha) as BF16.
  // Lane (i, q) of matrix-core tile (a, b) holds row wm*128 + 16a + i,
  // columns wn*64 + 16b + 4q .. +3.  For full tiles two neighbouring tiles
  // (b = 2p, 2p+1) are recombined across lanes l and l^16 (ds_bpermute) so
  // that every lane holds 8 consecutive columns: lanes with q even get
  // columns 8(q/2) .. +7 of tile 2p, lanes with q odd those of tile 2p+1.  One
  // 16-byte store per lane then covers 64 contiguous bytes of 16 rows.  Edge
  // tiles (and N not a multiple of 8) store element by element with masks.
  struct Epi {
    u32x4 rd;                    // full tiles: D from the tile's origin
    uint32_t voff;               // full tiles: this lane's byte offset in the tile
    uint32_t rowstride;          // bytes of 16 rows of D
    int m0, n0, lim;             // tile origin and row limit (edge tiles)
    float alpha;
    bool full, on;
    int bslot, act;              // fused epilogue
  };
  static constexpr int EPI_STORES = FM * FN / 2;   // store instructions per full tile

  __device__ static inline void make_epi(const Ctx &c, int64_t m0, int64_t n0, int64_t lim, float alpha,
                                         bool on, Epi &e, int bslot = 0) {
    const DenseArgs &p = *c.p;
    e.m0 = (int)m0;
    e.n0 = (int)n0;
    e.lim = (int)lim;
    e.bslot = bslot;
    e.act = FUSE ? p.act : ACT_NONE;
    e.alpha = alpha;
    e.on = on;
    // Full tiles store through the range-checked vector offset (at most
    // 2 (255 N + 255) bytes from the tile's origin), which must stay below
    // the resource's clamped size of 2^31 - 16 bytes; wider D takes the
    // element-wise path.
    e.full = m0 + DBM <= lim && n0 + DBN <= p.N && (p.N & 7) == 0 && p.N <= (1 << 22);
    const int64_t org = m0 * p.N + n0;
    e.rd = rsrc4(p.D + org, clamp_records(2 * (p.M * p.N - org)));
    e.rowstride = (uint32_t)(32 * p.N);
    const int lane = (int)__lane_id(), i = lane & 15, q = lane >> 4;
    e.voff = (uint32_t)(2 * ((c.wm * (FM * 16) + i) * p.N + c.wn * (FN * 16) + 16 * (q & 1) + 8 * (q >> 1)));
  }

  __device__ static inline void store_rows(const Ctx &c, const Epi &e, int a, const v4f (&row_in)[FN]) {
    const float al = e.alpha;
    // alpha is 1 unless the operands are tensor-wise: no multiply
    v4f row[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) row[b] = (SMODE != SM_TENSOR) ? row_in[b] : row_in[b] * al;
    // Fused epilogue: + bias[n] (BF16 from the tile's bias slot), then the
    // activation, both in FP32 before the one rounding to BF16; applied to
    // one matrix-core tile at a time, right before it is packed.
    auto finish = [&](v4f v, int b) -> v4f {
      if constexpr (FUSE) {
        const int lane = (int)__lane_id();
        const uint32_t bs = c.lds0 + BIAS_OFF + (uint32_t)e.bslot * BIAS_SLOT + (c.wn * 64 + 4 * (lane >> 4)) * 2;
        const v2i w = *(const lds_v2i *)(uintptr_t)(bs + b * 32);
        v.x += __uint_as_float((uint32_t)w.x << 16);
        v.y += __uint_as_float((uint32_t)w.x & 0xFFFF0000u);
        v.z += __uint_as_float((uint32_t)w.y << 16);
        v.w += __uint_as_float((uint32_t)w.y & 0xFFFF0000u);
        const int act = e.act;
        if (act != ACT_NONE) {
          v.x = activate(act, v.x);
          v.y = activate(act, v.y);
          v.z = activate(act, v.z);
          v.w = activate(act, v.w);
        }
      }
      return v;
    };
    if (e.full) {
      // computed here, not hoisted into a register per row tile
      uint32_t rs = e.rowstride;
      asm volatile("" : "+s"(rs));
      const int lane = (int)__lane_id();
      const bool odd = ((lane >> 4) & 1) != 0;
      const int partner = (lane ^ 16) << 2;
#pragma unroll
      for (int pr = 0; pr < FN / 2; ++pr) {
        const v4f x = finish(row[2 * pr], 2 * pr), y = finish(row[2 * pr + 1], 2 * pr + 1);
        const uint32_t xlo = pack_bf16x2(x.x, x.y), xhi = pack_bf16x2(x.z, x.w);
        const uint32_t ylo = pack_bf16x2(y.x, y.y), yhi = pack_bf16x2(y.z, y.w);
        // q even keeps its tile-2p chunk and takes the partner's; q odd the
        // same with tile 2p+1
        const uint32_t rlo = (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)(odd ? xlo : ylo));
        const uint32_t rhi = (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)(odd ? xhi : yhi));
        const v4i v = odd ? (v4i){(int)rlo, (int)rhi, (int)ylo, (int)yhi}
                          : (v4i){(int)xlo, (int)xhi, (int)rlo, (int)rhi};
        store16_asm(v, e.rd, e.voff, (uint32_t)a * rs + 64u * pr);
      }
    } else {
      // edge tiles: lane position recomputed here rather than kept live
      const DenseArgs &p = *c.p;
      const int lane = (int)__lane_id(), i = lane & 15, q = lane >> 4;
      const int64_t r = (int64_t)e.m0 + c.wm * (FM * 16) + a * 16 + i;
      if (r < e.lim) {
        uint16_t *dst = p.D + r * p.N;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          const v4f v = finish(row[b], b);
          const uint32_t u[2] = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
          const int64_t col = (int64_t)e.n0 + c.wn * (FN * 16) + b * 16 + 4 * q;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (col + k < p.N) dst[col + k] = (uint16_t)(u[k >> 1] >> (16 * (k & 1)));
        }
      }
    }
  }

  // One K step from ring slot si (scale slot gs).  With EPI the step is the
  // first of a tile: each accumulator row a-tile is first handed to the
  // epilogue `e` (the previous tile's result, stored while the matrix cores
  // run) and then restarted from zero.
  template <bool EPI>
  __device__ static inline void compute(const Ctx &c, const Lanes &L, int st,
                                        const uint8_t *smem, int si, int gs, v4f (&acc)[FM][FN],
                                        const struct Epi &e) {
    // The B and scale lane offsets include their regions' bases.
    const uint8_t *la = smem + si * AB, *lb = smem + si * AB, *ls = smem + gs * SGROUP;
    auto read_a = [&](int s, int a) -> v8i {
      if constexpr (FP4) return widen(lds_read16(la + L.a[s] + a * 2048));
      else if constexpr (TA) {
        // MX: the tile's base offset formed here from an opaque copy, not
        // kept in a register per tile through the loop (with the scale words
        // beside them, eight of those pushed accumulators into scratch inside
        // the K loop, each reload waiting on the stage's DMAs)
        uint32_t o = L.at;
        if constexpr (MX) asm volatile("" : "+v"(o));
        return rdt(la, o ^ ((uint32_t)a << 4));
      } else return rd8(la, L.a[0], L.a[1], a * 2048);
    };
    auto read_b = [&](int s, int b) -> v8i {
      if constexpr (PSB) {
        if constexpr (FP4) return widen(lds_read16(lb + L.b[0] + s * 4096 + b * 1024));
        else return rd8(lb, L.b[0], L.b[1], b * 2048);
      } else if constexpr (FP4) {
        return widen(lds_read16(lb + L.b[s] + b * 2048));
      } else if constexpr (TB) {
        uint32_t o = L.bt;
        if constexpr (MX) asm volatile("" : "+v"(o));
        return rdt(lb, o ^ ((uint32_t)b << 4));
      } else return rd8(lb, L.b[0], L.b[1], b * 2048);
    };
    auto b_scale = [&](int s, int b) -> int {
      if constexpr (MX) {
        const int j = (st * KS + s) & 3;        // K step within the scale group
        if constexpr (PSB) {
          const uint32_t word = lds_u32(ls + L.sb + b * 256);
          return (int)(word >> (8 * j));
        } else {
          const uint32_t word = lds_u32(ls + L.sb + b * 256 + j * 4);
          return (int)(word >> (8 * c.q));
        }
      }
      return E8M0_ONE_X4;
    };
    // A stage of two K steps (FP4) reads both steps' B fragments and scales
    // up front, so that the second step's reads overlap the first step's
    // matrix work instead of stalling between the two (not in the first step
    // of a fused epilogue, nor with a transposed operand: both need those
    // registers).
    constexpr bool PRE = KS > 1 && !(FUSE && EPI) && !TA && !TB;
    v8i bpre[KS][FN];
    int spre[KS][FN];
    if constexpr (PRE) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          bpre[s][b] = read_b(s, b);
          spre[s][b] = b_scale(s, b);
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      v8i bf[FN];
      int sb[FN];
      if constexpr (FP4 && TB) {
#pragma unroll
        for (int b = 0; b < FN; b += 2) rdt4_pair(lb, L.bt, b, s, bf[b], bf[b + 1]);
#pragma unroll
        for (int b = 0; b < FN; ++b) sb[b] = b_scale(s, b);
      } else {
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          if constexpr (PRE) {
            bf[b] = bpre[s][b];
            sb[b] = spre[s][b];
          } else {
            bf[b] = read_b(s, b);
            sb[b] = b_scale(s, b);
          }
        }
      }
      // A scale words: with K-contiguous operands all of the step's up front
      // (read beside the matrix-core tile that needs them, each would stall
      // its tile on an LDS round trip); with a transposed operand, whose
      // fragment addressing needs more registers, one tile ahead with the A
      // fragment, so that two words are live instead of eight.
      constexpr bool SA_AHEAD = TA || TB;
      auto scale_word = [&](int a) -> uint32_t {
        if constexpr (GROUP) return lds_u32(ls + L.sa + a * 64 + ((st * KS + s) & 3) * 1024);
        return MX ? lds_u32(ls + L.sa + a * 256 + ((st * KS + s) & 3) * 4) : 0u;
      };
      // groupwise: the weight block scale of this K step (all lanes alike)
      float wsv = 1.0f;
      if constexpr (GROUP) wsv = __uint_as_float(lds_u32(ls + L.sb + ((st * KS + s) & 3) * 4));
      uint32_t saw[SA_AHEAD ? 1 : FM];
      if constexpr (SA_AHEAD) {
        saw[0] = scale_word(0);
      } else {
#pragma unroll
        for (int a = 0; a < FM; ++a) saw[a] = scale_word(a);
      }
      if constexpr (GROUP) {
        // The 128-K partial products (neutral E8M0 scales) of row tile a go
        // to one of two register sets while the partials of tile a - 1 are
        // scaled by xs(row, kb) * ws(column block, kb) and added in FP32:
        // each scaling then reads results of matrix-core instructions issued
        // a whole row tile earlier, instead of waiting for the one just
        // issued.
        const v4f zero = (v4f){0.f, 0.f, 0.f, 0.f};
        v4f part[2][FN];
        float scp[2];
        v8i af = read_a(s, 0);
#pragma unroll
        for (int a = 0; a <= FM; ++a) {
          if (a < FM) {
            v8i af_next;
            if (a + 1 < FM) af_next = read_a(s, a + 1);
            scp[a & 1] = __uint_as_float(saw[a]) * wsv;
            // the previous tile's rows leave before this tile's partials
            // replace them (one row tile later)
            if (EPI && s == 0 && e.on) store_rows(c, e, a, acc[a]);
#pragma unroll
            for (int b = 0; b < FN; ++b)
              part[a & 1][b] = mfma_scaled<FB, FA>(bf[b], af, zero, E8M0_ONE_X4, E8M0_ONE_X4);
            if (a + 1 < FM) af = af_next;
          }
          if (a > 0) {
            const int r = a - 1;
#pragma unroll
            for (int b = 0; b < FN; ++b) {
              if (EPI && s == 0) acc[r][b] = part[r & 1][b] * scp[r & 1];
              else acc[r][b] += part[r & 1][b] * scp[r & 1];
            }
          }
          // tile a's matrix-core instructions one at a time, each followed
          // by four of tile a - 1's scaling FMAs: the wave keeps its matrix
          // core fed by itself while the VALU works in the instruction's
          // shadow (left free, the scheduler put the independent FMAs first,
          // where they waited on tile a - 1's results; grouped after the
          // four instructions, they measured 2-10% slower)
          if (a > 0 && a < FM) {
#pragma unroll
            for (int i = 0; i < FN; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      // Transposed packed E2M1 A: tiles come in pairs (rdt4_pair); the pair
      // after tile a is read at odd a, with tile a + 1 the first of it.
      constexpr bool A_PAIRS = FP4 && TA;
      v8i af, apair1;
      if constexpr (A_PAIRS) rdt4_pair(la, L.at, 0, s, af, apair1);
      else af = read_a(s, 0);
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        v8i af_next;
        uint32_t sw_next = 0;
        if (a + 1 < FM) {
          if constexpr (A_PAIRS) {
            if (a & 1) rdt4_pair(la, L.at, a + 1, s, af_next, apair1);
            else af_next = apair1;
          } else {
            af_next = read_a(s, a + 1);
          }
          if constexpr (SA_AHEAD) sw_next = scale_word(a + 1);
        }
        int sa = E8M0_ONE_X4;
        if constexpr (MX) sa = (int)((SA_AHEAD ? saw[0] : saw[a]) >> (8 * c.q));
        if (EPI && s == 0) {
          if (e.on) store_rows(c, e, a, acc[a]);
#pragma unroll
          for (int b = 0; b < FN; ++b) {
            if constexpr (BF) acc[a][b] = mfma_bf16_x2(bf[b], af, (v4f){0.f, 0.f, 0.f, 0.f});
            else acc[a][b] = mfma_scaled<FB, FA>(bf[b], af, (v4f){0.f, 0.f, 0.f, 0.f}, sb[b], sa);
          }
        } else {
#pragma unroll
          for (int b = 0; b < FN; ++b) {
            // First operand = B tile: the result lane holds 4 consecutive n.
            if constexpr (BF) acc[a][b] = mfma_bf16_x2(bf[b], af, acc[a][b]);
            else acc[a][b] = mfma_scaled<FB, FA>(bf[b], af, acc[a][b], sb[b], sa);
          }
        }
        if (a + 1 < FM) {
          af = af_next;
          if constexpr (SA_AHEAD) saw[0] = sw_next;
        }
        // keep the A reads one tile ahead, not hoisted further (registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Keeps a step's matrix-core instructions ahead of the wait that ends the
  // step.  They only touch registers, so without this the compiler is free to
  // sink them past the wait and barrier into the next step, which leaves the
  // wait for the next stage's DMA with nothing to overlap.
  __device__ static inline void pin(v4f (&acc)[FM][FN]) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
      asm volatile("" : "+v"(acc[a][0]), "+v"(acc[a][1]), "+v"(acc[a][2]), "+v"(acc[a][3]));
  }

  // The K loop over every tile of this workgroup.  K step k of a tile reads
  // ring slot k % 2 while the next stage (K step k+1, or the first K step of
  // the next tile) streams into the other slot.  The DMAs are invisible to
  // the compiler (dma_asm), so the waits below are the only ones: the DMA
  // into a slot is issued after the barrier that retired every wave's reads
  // of it, and the slot is read only after the wait + barrier.
  //
  // A tile's first K step stores the previous tile's result (store_rows) as
  // its accumulators restart.  Vector-memory operations of a wave are counted
  // in issue order, so at the end of that step waiting until at most
  // EPI_STORES operations are outstanding means the stage DMA issued before
  // the stores has landed, and the stores drain during the next K step.
  template <class TileAt, class Resolve>
  __device__ static inline void run(const Ctx &c, int ntiles, TileAt tile_at, Resolve resolve,
                                    float alpha, uint8_t *smem) {
    Lanes L;
    lane_offsets(c, L);

    v4f acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

    int tm, tn;
    tile_at(0, tm, tn);
    Tile cur;
    set_tile(c, resolve(tm, tn), cur);
    issue(c, cur, 0, 0, 0);
    wait_vmem_le<0>();
    __syncthreads();

    const int nst = c.nst;
    const bool odd = (nst & 1) != 0;
    const int ngrp = (int)c.ngrp;              // scale groups per tile
    Epi e;
    make_epi(c, 0, 0, 0, alpha, false, e);
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      const int g0 = t * ngrp;                 // scale slot of group g: (g0 + g) % 2
      if (more) tile_at(t + 1, tm, tn);
      auto step = [&](auto epi, auto slot, int k) {
        constexpr bool EPI = decltype(epi)::value;
        constexpr int SC = decltype(slot)::value, SN = 1 - SC;
        auto issue_any = [&](const Tile &src, int st, int gs) {
          if constexpr (!TA && !TB) issue_hi(c, src, st, SN, gs);
          else issue(c, src, st, SN, gs);
        };
        if (k + 1 < nst) {
          issue_any(cur, k + 1, (g0 + (k + 1) * KS / 4) & 1);
        } else if (more && !odd) {
          // first stage of the next tile into slot 0 (this step reads slot 1);
          // its sources are built here, not kept live through the K loop
          Tile nxt;
          set_tile(c, resolve(tm, tn), nxt);
          nxt.bslot = (t + 1) & 1;
          issue_any(nxt, 0, (g0 + ngrp) & 1);
        }
        compute<EPI>(c, L, k, smem, SC, (g0 + k * KS / 4) & 1, acc, e);
        // Only where registers allow: for the transposed FP8 variants and MX
        // FP8 with plain B it costs spills in the K loop.  The transposed E2M1
        // variants need it: unpinned, the compiler holds a whole stage of
        // fragments in registers to run the step's matrix work after the
        // barrier, and spills in the K loop.
        if constexpr (PIN) pin(acc);
        __builtin_amdgcn_sched_barrier(0);
        // This wave's part of the next stage has landed (and, with no
        // epilogue in flight, everything else); the barrier publishes every
        // wave's DMA.
        if (EPI && e.on && e.full) wait_vmem_le<EPI_STORES>();
        else wait_vmem_le<0>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      };
      step(std::true_type{}, std::integral_constant<int, 0>{}, 0);
      int k = 1;
      for (; k + 2 <= nst; k += 2) {
        step(std::false_type{}, std::integral_constant<int, 1>{}, k);
        step(std::false_type{}, std::integral_constant<int, 0>{}, k + 1);
      }
      if (k < nst) step(std::false_type{}, std::integral_constant<int, 1>{}, k);
      // this tile's result goes out during the next tile's first step
      make_epi(c, cur.m0, cur.n0, cur.lim, alpha, true, e, cur.bslot);
      if (more) {
        set_tile(c, resolve(tm, tn), cur);
        cur.bslot = (t + 1) & 1;
        if (odd) {
          // the last step read slot 0: the next tile's first stage follows it
          issue(c, cur, 0, 0, (g0 + ngrp) & 1);
          wait_vmem_le<0>();
          __syncthreads();
        }
      }
    }
#pragma unroll
    for (int a = 0; a < FM; ++a) store_rows(c, e, a, acc[a]);
  }
};

// Tile b of the tile order: groups of 8 tile-rows, each walked column by
// column, so that 32 consecutive tiles share 8 A panels and 4 B panels.
__device__ inline void tile_in_order(int b, int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int g = b / per_group;
  const int first = g * GM;
  const int rows = min(GM, tiles_m - first);
  const int in = b - g * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

// The k-th tile of workgroup bid in a persistent grid of P workgroups: it
// takes virtual tiles bid, bid + P, bid + 2P, ...  Workgroups are dealt to
// the eight XCDs round-robin, so within each round of P virtual tiles (the
// ones that run at the same time) those of one XCD (bid % 8 equal) are
// remapped to a compact band of the tile order, and the 32 tiles an XCD runs
// at once share their panels in its L2.
__device__ inline void persistent_tile(int bid, int k, int P, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nb = tiles_m * tiles_n;
  const int base = k * P;
  const int size = min(P, nb - base);
  const int b = base + (((size & 7) == 0) ? (bid & 7) * (size >> 3) + (bid >> 3) : bid);
  tile_in_order(b, tiles_m, tiles_n, tm, tn);
}

template <int FA, int FB, int SMODE, bool TA, bool TB, bool PSB, bool FUSE = false>
__global__ __launch_bounds__(DNW8 * 64, 1) void dense_kernel(DenseArgs p) {
  typedef DenseLoop<FA, FB, SMODE, TA, TB, PSB, FUSE> L;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::LDS_BYTES];

  const int nb = p.tiles_m * p.tiles_n;
  const int P = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  if (bid >= nb) return;
  const int ntiles = (nb - bid + P - 1) / P;

  typename L::Ctx c;
  L::init(c, p, smem);

  float alpha = 1.0f;
  if constexpr (SMODE == SM_TENSOR) alpha = *(const float *)p.sA * *(const float *)p.sB;

  auto tile_at = [&](int k, int &tm, int &tn) {
    // Opaque copies: keeps the division set-up of the tile order from being
    // hoisted out of the tile loop into registers the K loop needs.
    int P_ = P, tm_ = p.tiles_m, tn_ = p.tiles_n;
    asm volatile("" : "+s"(P_), "+s"(tm_), "+s"(tn_));
    persistent_tile(bid, k, P_, tm_, tn_, tm, tn);
  };
  auto resolve = [&](int tm, int tn) -> TileId {
    return TileId{(int64_t)tm * DBM, (int64_t)tn * DBN, p.M, 0, 0, 0};
  };
  L::run(c, ntiles, tile_at, resolve, alpha, smem);
}

}  // namespace mxg
