// Grouped groupwise FP8 GEMM for gfx950 ("Add FlyDSL grouped groupwise FP8
// GEMM for ROCm"): for each group g of rows (an expert),
//   D[r, n] = sum_k dec(XQ[r,k]) xs(r, k/128) * dec(WQ[g,n,k]) ws[g, n/128, k/128].
//
// * Tile scheduling: every grid is derived from static shapes only (a
//   persistent grid sized by the compute units), and each kernel resolves
//   its tiles' groups from m_sizes on the device (Tile selection; commit on
//   in-kernel group resolution).  A tile never spans two groups.  Every
//   group is clamped to [0, totM) so a violated sum(m_sizes) == totM
//   precondition cannot reach memory outside D.
// * Software scaling (Architecture support): each 128-K step runs the scaled
//   matrix-core instruction with the neutral E8M0 scale into a zeroed
//   accumulator, then adds that partial times xs(row, kb) * ws(g, n/128, kb)
//   in FP32.
// * Activation scales are read in the per-group block layout (commit on the
//   scale_a layout): group g's block begins at start_g*(K/128); (local row i,
//   k-block kb) sits at i + kb*M_g.
// * B is either plain [G, N, K] (staged through XOR-swizzled LDS like A) or
//   preshuffled per group (copied linearly into LDS).
// This file holds two kernel families: grouped_stream_kernel (BM x BN tiles,
// for few rows per group) and grouped_dense_kernel (256 x 256 tiles on the
// dense kernel's pipeline, for many rows per group), whose last, partial
// round of tiles the streaming kernel can take over in 128 x 64 or 64 x 64
// pieces (grouped_split_end).  Both families also run the BF16 grouped GEMM
// (FMT = F_BF16: BF16 operands, no scales).
#pragma once
#include "../../include/mxgemm.h"
#include "dense.hpp"

namespace mxg {

struct GroupedArgs {
  const int64_t *m_sizes;
  const uint8_t *XQ, *WQ;
  const float *xs, *ws;
  uint16_t *D;
  int64_t totM, N, K;
  int G, tiles_n;
  // the streaming kernel as the tail of the 256 x 256 kernel only: that
  // kernel's 256-column tiles, grid and rule (see grouped_split_end)
  int tiles_nb, main_grid, tail_rounds;
};

// The split of the 256 x 256 grouped kernel's nb tiles (persistent grid of
// P workgroups, one per compute unit) into [0, end), which it runs in full
// rounds, and [end, nb), which the streaming kernel (P_tail workgroups)
// runs after it, each tile cut into 8 pieces of 128 x 64, or into 16 of
// 64 x 64 when those 16 r fill at most one round of the streaming kernel
// (then twice as many of its workgroups share the work).  A last round of
// r = nb mod P tiles would leave P - r compute units idle for a whole tile;
// its pieces take ceil(pieces / P_tail) rounds of the streaming kernel, each
// much shorter than a 256 x 256 tile, so the split is made when that count
// is at most max_rounds.  Both kernels evaluate this from the same nb.
__device__ inline int grouped_tail_pieces(int r, int P_tail) { return 16 * r <= P_tail ? 16 : 8; }

__device__ inline int grouped_split_end(int nb, int P, int P_tail, int max_rounds) {
  const int r = nb % P;
  if (max_rounds <= 0 || nb <= P || r == 0) return nb;
  const int pieces = grouped_tail_pieces(r, P_tail) * r;
  return (pieces + P_tail - 1) / P_tail <= max_rounds ? nb - r : nb;
}

// Grouped kernel for few rows per group (the weight-streaming regime: the
// weights dominate the bytes and HBM, not the matrix cores, sets the time).
//
// * BM x BN output tiles (64 x 64, or 128 x 128 where a group's rows are
//   read by many column tiles: each 128-row A block is then streamed half
//   as often as with 128 x 64 tiles).  The real tiles (groups with rows
//   only, none spanning two groups) are numbered group by group, N-tile
//   major and M-tile minor, so that consecutive tiles share one weight tile.
//   Each workgroup finds a tile's group by binary search in a table of the
//   groups' first rows and first tiles that wave 0 builds in LDS once.
// * Persistent grid of P workgroups, two per compute unit (one for the
//   tail of the 256 x 256 kernel, with two K steps per stage): each walks one
//   tile of every round of P consecutive tiles; within a round each XCD (one
//   L2) takes a contiguous band of tiles, the eight bands as even as the
//   round allows, so tiles that read the same weights at the same time
//   share an L2 and no XCD idles while another holds two tiles per CU.
// * A two-slot ring of stages of KS 128-K steps (per step: A rows, weight
//   rows, the tile's activation scales and weight block scale) is filled by
//   buffer-load-to-LDS DMA issued from inline assembly with explicit waits.
//   The ring runs across tile boundaries, so a workgroup's stream never
//   drains between its tiles; the second workgroup on the compute unit
//   covers this one's wait-barrier-compute chain.
// * Per K step, four waves (2 x 2, (BM/2) x (BN/2) each) run the scaled
//   matrix-core instruction with the neutral E8M0 scale into a zeroed
//   accumulator and add the partial times xs(row, kb) * ws(g, n/128, kb) in
//   FP32.  A tile's result is stored as BF16 straight from the accumulators.
// * 8-row blocks of A past the tile's group read nothing (empty range).
template <int BM_, int BN_>
struct GroupedStream {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int FM = BM / 32, FN = BN / 32;
  static constexpr int AB = BM * 128, BB = BN * 128;
  static constexpr int SC = BM * 4 + 256;           // xs (BM floats) + ws (64 copies)
  static constexpr int STEP = AB + BB + SC;         // one 128-K step
  static constexpr int ABLK = BM / 32;              // A DMAs per wave and K step
  static constexpr int BBLK = BN / 32;              // B DMAs per wave and K step
};

// Group table of a workgroup, in LDS: rows[g] = first row of group g (groups
// clamped to [0, totM) in order, so rows[g] = min(sum of the earlier
// max(m_sizes, 0), totM)), mtile[g] = number of BM-row tiles of the groups
// before g; entry G closes both.  Built by wave 0 with a 64-lane prefix sum
// per chunk of 64 groups.
struct GroupTable {
  int32_t rows[MXG_GROUPED_MAX_G + 1];
  int32_t mtile[MXG_GROUPED_MAX_G + 1];
};

__device__ inline int64_t wave_incl_sum(int64_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

template <int BM>
__device__ inline void build_group_table(const int64_t *m_sizes, int G, int64_t totM, GroupTable &gt,
                                         int lane) {
  int64_t rows = 0, tiles = 0;
  for (int c = 0; c < G; c += 64) {
    const int g = c + lane;
    int64_t s = g < G ? m_sizes[g] : 0;
    s = s < 0 ? 0 : (s > totM ? totM : s);
    const int64_t incl = wave_incl_sum(s, lane);
    const int64_t r0 = min(rows + incl - s, totM), r1 = min(rows + incl, totM);
    const int64_t mt = (r1 - r0 + BM - 1) / BM;
    const int64_t tincl = wave_incl_sum(mt, lane);
    if (g < G) {
      gt.rows[g] = (int32_t)r0;
      gt.mtile[g] = (int32_t)(tiles + tincl - mt);
    }
    rows = min(rows + __shfl(incl, 63, 64), totM);
    tiles += __shfl(tincl, 63, 64);
  }
  if (lane == 0) {
    gt.rows[G] = (int32_t)rows;
    gt.mtile[G] = (int32_t)tiles;
  }
}

// A value every lane holds alike, moved to scalar registers.
__device__ inline int32_t uni32(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// The last group g with mtile[g] <= u, for a BM-row tile index u over all
// groups (a non-empty group: an empty one shares its mtile with the group
// after it).
__device__ inline int group_of_tile(const GroupTable &gt, int G, int32_t u) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uni32(gt.mtile[mid]) <= u) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Real tile t (t < mtile[G] * tiles_n): tiles are numbered group by group,
// N-tile major, M-tile minor within a group.  Group g's rows are
// [start, start + mg); the tile's are [row0, min(row0 + BM, lim)).
struct StreamTile {
  int64_t start, mg, row0, n0, lim;
  int g;
};

template <int BM, int BN>
__device__ inline StreamTile stream_tile(const GroupedArgs &p, const GroupTable &gt, int64_t t) {
  const int32_t u = (int32_t)(t / p.tiles_n);        // BM-row tile index over all groups
  const int g = group_of_tile(gt, p.G, u);
  const int32_t mt0 = uni32(gt.mtile[g]), r0 = uni32(gt.rows[g]);
  const int64_t mt = uni32(gt.mtile[g + 1]) - mt0;
  const int64_t local = t - (int64_t)mt0 * p.tiles_n;
  const int64_t tn = local / mt, tm = local - tn * mt;
  StreamTile r;
  r.g = g;
  r.start = r0;
  r.mg = uni32(gt.rows[g + 1]) - r0;
  r.row0 = r.start + tm * BM;
  r.n0 = tn * BN;
  r.lim = r.start + r.mg;
  return r;
}

// Piece t of the tail of the 256 x 256 kernel (tiles [end, nb) of its tile
// order), `pieces` (8 or 16) per tile: tile end + t / pieces, and with h =
// pieces / 4 row parts of 256 / h rows, row part (t % pieces) % h and
// column quarter (t % pieces) / h.  A part past its group's rows or a
// quarter past N (the last tile column when N is an odd multiple of 128) is
// empty: it reads zeros and stores nothing.
__device__ inline StreamTile tail_piece(const GroupedArgs &p, const GroupTable &gt, int64_t t, int end,
                                        int pieces) {
  const int v = end + (int)(t / pieces), s = (int)(t % pieces);
  const int h = pieces >> 2, rows = DBM / h;
  int tm, tn;
  tile_in_order(v, uni32(gt.mtile[p.G]), p.tiles_nb, tm, tn);
  const int g = group_of_tile(gt, p.G, tm);
  StreamTile r;
  r.g = g;
  r.start = uni32(gt.rows[g]);
  r.mg = uni32(gt.rows[g + 1]) - r.start;
  r.row0 = r.start + (int64_t)(tm - uni32(gt.mtile[g])) * DBM + (int64_t)rows * (s % h);
  r.n0 = (int64_t)tn * DBN + 64 * (s / h);
  if (r.row0 > r.start + r.mg || r.n0 >= p.N) r.row0 = r.start + r.mg;
  r.lim = min(r.start + r.mg, r.row0 + rows);
  return r;
}

// BM x BN tiles, KS 128-K steps per ring stage, NS ring slots.  TAIL: the
// kernel (128 x 64) runs the tail pieces of the 256 x 256 kernel in place
// of its own tiles (a 64 x 64 piece leaves the tile's lower 64 rows
// empty).
// FMT = F_BF16: BF16 operands and no scales (a 128-byte K step holds 64
// values, two 16x16x32 BF16 matrix-core instructions per fragment pair).
template <bool PSB, int BM, int BN, int KS, int NS, bool TAIL = false, int FMT = F_E4M3>
__global__ __launch_bounds__(256, 2) void grouped_stream_kernel(GroupedArgs p) {
  static_assert(!TAIL || (BM == 128 && BN == 64), "tail pieces are 128 x 64");
  constexpr bool BF = (FMT == F_BF16);
  typedef GroupedStream<BM, BN> S;
  constexpr int FM = S::FM, FN = S::FN, ABLK = S::ABLK, BBLK = S::BBLK;
  constexpr int STAGE = KS * S::STEP;
  // DMAs per stage and wave: ABLK for A and BBLK for B per K step, plus one
  // per K step for the activation scales (waves 0 and, with 128 rows, 2) or
  // the weight block scale (wave 1).
  constexpr int OPS_LO = (ABLK + BBLK) * KS, OPS_HI = (ABLK + BBLK + 1) * KS;
  static_assert(OPS_HI * (NS - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
  __shared__ GroupTable gt;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int i16 = lane & 15, q = lane >> 4;

  if (w == 0) build_group_table<TAIL ? DBM : BM>(p.m_sizes, p.G, p.totM, gt, lane);
  __syncthreads();
  const int P = (int)gridDim.x;
  int end = 0;                                      // TAIL: first tile of the tail
  int pieces = 8;                                   // TAIL: pieces per tile
  int64_t T;                                        // real tiles (TAIL: pieces)
  if constexpr (TAIL) {
    const int nb = uni32(gt.mtile[p.G]) * p.tiles_nb;
    end = grouped_split_end(nb, p.main_grid, P, p.tail_rounds);
    pieces = grouped_tail_pieces(nb - end, P);
    T = (int64_t)(nb - end) * pieces;
  } else {
    T = (int64_t)uni32(gt.mtile[p.G]) * p.tiles_n;
  }
  // Workgroup b runs on XCD x = b % 8 (workgroups are dealt to the eight
  // XCDs in turn) as that XCD's r-th, r = b / 8.  Each round of P
  // consecutive tiles (the last round holds T mod P) is cut into eight
  // contiguous bands as even as the round allows, band x for XCD x, and the
  // r-th workgroup of XCD x takes tile r of its band.  Every XCD then has
  // the same share of the work, also when there are fewer tiles than
  // workgroups, and tiles with the same weights share one L2.
  const int x = (int)(blockIdx.x & 7), r = (int)(blockIdx.x >> 3);
  const int64_t full = T / P, last = T - full * P;
  auto band_start = [&](int64_t size) -> int64_t { return x * (size >> 3) + (x < (size & 7) ? x : (size & 7)); };
  auto band_count = [&](int64_t size) -> int64_t { return (size >> 3) + (x < (size & 7) ? 1 : 0); };
  const int64_t ntile = full + (r < band_count(last) ? 1 : 0);   // tiles of this workgroup
  if (ntile == 0) return;
  const int64_t off_full = band_start(P) + r, off_last = band_start(last) + r;
  auto tile_of = [&](int64_t i) -> int64_t { return i * P + (i < full ? off_full : off_last); };
  auto tile_at = [&](int64_t i) -> StreamTile {
    if constexpr (TAIL) return tail_piece(p, gt, tile_of(i), end, pieces);
    else return stream_tile<BM, BN>(p, gt, tile_of(i));
  };
  const int64_t K = BF ? 2 * p.K : p.K, N = p.N;  // K: bytes per row
  const int nst = (int)(K / 128);                  // K steps (128 bytes) per tile
  const int nsg = (nst + KS - 1) / KS;             // stages per tile
  const int64_t kb_n = K / 128;
  const int64_t V = ntile * nsg;                   // stages of this workgroup

  const u32x4 rx = rsrc4(p.xs, clamp_records(p.totM * kb_n * 4));
  const u32x4 rw = rsrc4(p.ws, clamp_records((int64_t)p.G * (N / 128) * kb_n * 4));
  const u32x4 rzero = rsrc4(p.xs, 0);
  // lane offset of the row-tile DMAs (8 rows x 128 B per DMA; row r keeps
  // 16-byte piece c at position c ^ kswz(r))
  const uint32_t vo = (uint32_t)((lane >> 3) * K) + (uint32_t)(((lane & 7) ^ kswz(lane >> 3)) << 4);
  const uint32_t lds0 = lds_addr(smem);

  // Issue side: the tile whose stages are being issued.
  struct Src {
    u32x4 ra, rb;
    uint32_t xs0, ws0, mg4;
    int vrows;
  };
  auto make_src = [&](int64_t i) {
    const StreamTile t = tile_at(i);
    Src s;
    const int64_t abase = t.row0 * K;
    s.ra = rsrc4(p.XQ + abase, clamp_records(p.totM * K - abase));
    const int64_t bbase = (int64_t)t.g * N * K + t.n0 * K;
    s.rb = rsrc4(p.WQ + bbase, clamp_records(N * K - t.n0 * K));
    s.xs0 = (uint32_t)((t.start * kb_n + (t.row0 - t.start)) * 4);
    s.ws0 = (uint32_t)((((int64_t)t.g * (N / 128) + t.n0 / 128) * kb_n) * 4);
    s.mg4 = (uint32_t)(t.mg * 4);
    const int64_t left = t.lim - t.row0;
    s.vrows = (int)(left < BM ? left : BM);
    return s;
  };
  Src src = make_src(0);
  int64_t iss_i = 0;
  int iss_sg = 0;

  // Stage (iss_i, iss_sg) into slot sl, then advance; K steps past the
  // tile's last one and stages past the workgroup's last read an empty
  // range (zeros: their partials add exactly 0, and the wait counts stay
  // uniform).
  auto issue = [&](int sl) {
    const bool real = iss_i < ntile;
    const uint32_t slot = lds0 + (uint32_t)sl * STAGE;
    static_for<0, KS>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int st = iss_sg * KS + s;
      const bool live = real && st < nst;
      const uint32_t ka = slot + (uint32_t)s * S::AB;
      const uint32_t kb = slot + (uint32_t)(KS * S::AB + s * S::BB);
      const uint32_t ksc = slot + (uint32_t)(KS * (S::AB + S::BB) + s * S::SC);
      static_for<0, ABLK>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        const int blk = ABLK * w + jj;
        const u32x4 r = (live && blk * 8 < src.vrows) ? src.ra : rzero;
        dma_asm_v<16>(ka + (uint32_t)blk * 1024u, r, vo, (uint32_t)(blk * 8 * K + 128 * (int64_t)st));
      });
      const u32x4 rb = live ? src.rb : rzero;
      static_for<0, BBLK>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        const int blk = BBLK * w + jj;
        // preshuffled: 1 KiB block blk % 8 of 64-column group blk / 8, whose
        // K steps lie 64 K bytes after the previous group's
        if constexpr (PSB && BN == 64)
          dma_asm<16>(kb + (uint32_t)blk * 1024u, rb, (uint32_t)lane * 16u,
                      (uint32_t)(st * 8192 + blk * 1024));
        else if constexpr (PSB)
          dma_asm<16>(kb + (uint32_t)blk * 1024u, rb, (uint32_t)lane * 16u,
                      (uint32_t)((blk >> 3) * 64 * K + st * 8192 + (blk & 7) * 1024));
        else
          dma_asm<16>(kb + (uint32_t)blk * 1024u, rb, vo,
                      (uint32_t)(blk * 8 * K + 128 * (int64_t)st));
      });
      if constexpr (!BF) {
        // activation scales of rows 64h .. 64h + 63 by wave 2h
        if ((w & 1) == 0 && 32 * w < BM)
          dma_asm_v<4>(ksc + (uint32_t)(128 * w), live ? rx : rzero, (uint32_t)lane * 4u,
                       src.xs0 + (uint32_t)(128 * w) + (uint32_t)st * src.mg4);
        if (w == 1) dma_asm<4>(ksc + (uint32_t)(BM * 4), live ? rw : rzero, 0u, src.ws0 + (uint32_t)st * 4u);
      }
    });
    if (++iss_sg == nsg) {
      iss_sg = 0;
      ++iss_i;
      if (iss_i < ntile) src = make_src(iss_i);
    }
  };
  // Stage v has landed once only this wave's DMAs of the NS - 2 stages
  // issued after it (and any result stores, issued later still) are
  // outstanding.
  const bool hi_ops = w < 2 || (BM == 128 && w == 2);
  auto wait_stage = [&]() {
    if (hi_ops) wait_vmem_le<OPS_HI * (NS - 2)>();
    else wait_vmem_le<OPS_LO * (NS - 2)>();
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

  // fragment lane offsets
  const int f = kswz(i16);
  const uint32_t oa0 = (uint32_t)((wm * (BM / 2) + i16) * 128 + ((q ^ f) << 4));
  const uint32_t oa1 = (uint32_t)((wm * (BM / 2) + i16) * 128 + (((q + 4) ^ f) << 4));
  const uint32_t ob0 = PSB ? (uint32_t)(wn * (BN / 2) * 128 + lane * 16)
                           : (uint32_t)((wn * (BN / 2) + i16) * 128 + ((q ^ f) << 4));
  const uint32_t ob1 = PSB ? ob0 + 1024u : (uint32_t)((wn * (BN / 2) + i16) * 128 + (((q + 4) ^ f) << 4));
  const uint32_t oxs = (uint32_t)((wm * (BM / 2) + i16) * 4);

  for (int s = 0; s < NS - 1; ++s) issue(s);
  wait_stage();
  __syncthreads();

  int64_t ci = 0;      // tile being computed
  int csg = 0;         // its stage
  for (int64_t v = 0; v < V; ++v) {
    const int sl = (int)(v % NS);
    issue((int)((v + NS - 1) % NS));
    const uint8_t *stg = smem + sl * STAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint8_t *la = stg + s * S::AB, *lb = stg + KS * S::AB + s * S::BB;
      const uint8_t *lsc = stg + KS * (S::AB + S::BB) + s * S::SC;
      v8i bf[FN];
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const v4i x = lds_read16(lb + ob0 + b * 2048), y = lds_read16(lb + ob1 + b * 2048);
        bf[b] = (v8i){x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
      }
      float wsc = 1.0f;
      if constexpr (!BF) wsc = __uint_as_float(lds_load_u32(lsc + BM * 4));
      auto read_af = [&](int a) -> v8i {
        const v4i x = lds_read16(la + oa0 + a * 2048), y = lds_read16(la + oa1 + a * 2048);
        return (v8i){x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
      };
      if constexpr (BF) {
#pragma unroll
        for (int a = 0; a < FM; ++a) {
          const v8i af = read_af(a);
#pragma unroll
          for (int b = 0; b < FN; ++b) acc[a][b] = mfma_bf16_x2(bf[b], af, acc[a][b]);
        }
      } else {
        // As the 256 x 256 kernel: row tile a's partial products go to one
        // of two register sets while tile a - 1's are scaled and added, one
        // matrix-core instruction followed by four FMAs, and tile a + 1's A
        // fragment and scale are read ahead.
        v4f part[2][FN];
        float scp[2];
        v8i af = read_af(0);
        float scn = __uint_as_float(lds_load_u32(lsc + oxs)) * wsc;
#pragma unroll
        for (int a = 0; a <= FM; ++a) {
          v8i af_next;
          float sc_next = 0.0f;
          if (a + 1 < FM) {
            af_next = read_af(a + 1);
            sc_next = __uint_as_float(lds_load_u32(lsc + oxs + (a + 1) * 64)) * wsc;
          }
          if (a < FM) {
            scp[a & 1] = scn;
#pragma unroll
            for (int b = 0; b < FN; ++b)
              part[a & 1][b] = mfma_scaled<F_E4M3, F_E4M3>(bf[b], af, (v4f){0.f, 0.f, 0.f, 0.f},
                                                            E8M0_ONE_X4, E8M0_ONE_X4);
          }
          if (a > 0) {
#pragma unroll
            for (int b = 0; b < FN; ++b) acc[a - 1][b] += part[(a - 1) & 1][b] * scp[(a - 1) & 1];
          }
          if (a > 0 && a < FM) {
#pragma unroll
            for (int i = 0; i < FN; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if (a + 1 < FM) {
            af = af_next;
            scn = sc_next;
          }
        }
      }
    }
    if (++csg == nsg) {
      // Last K step of tile ci: lane (i16, q) holds rows 16a + i16 and
      // columns 16b + 4q .. +3 of the wave's (BM/2) x (BN/2) block.
      const StreamTile t = tile_at(ci);
      const int64_t row_lim = t.lim;
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int64_t row = t.row0 + wm * (BM / 2) + a * 16 + i16;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          const v4f r = acc[a][b];
          const uint32_t lo = pack_bf16x2(r.x, r.y), hi = pack_bf16x2(r.z, r.w);
          if (row < row_lim)
            *(v2i *)(p.D + row * N + t.n0 + wn * (BN / 2) + b * 16 + 4 * q) = (v2i){(int)lo, (int)hi};
          acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};
        }
      }
      csg = 0;
      ++ci;
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_stage();   // stage v + 1
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmem_le<0>();
}

}  // namespace mxg

namespace mxg {

// Grouped kernel for many rows per group (the matrix-core regime), on the
// dense kernel's pipeline (DenseLoop with groupwise scales): 256 x 256
// output tiles, eight waves, the two-slot LDS ring fed by inline-assembly
// DMA, a persistent grid with one workgroup per compute unit walking its
// tiles in XCD-banded order, and the epilogue of a tile stored from
// registers during the next tile's first K step.
//
// * Tiles: each group's rows are cut into 256-row tiles (a tile never spans
//   two groups; its stores stop at the group's last row), numbered over all
//   groups; wave 0 builds the table of every group's first row and first
//   tile in LDS once, and a tile's group is found by binary search.
// * Software scaling ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm",
//   Architecture support): each 128-K step runs the scaled matrix-core
//   instruction with the neutral E8M0 scale into a zero accumulator and adds
//   that partial times xs(row, kb) * ws(g, n/128, kb) in FP32.  The scales of
//   four K steps come into LDS with the operand stages: 256 activation scales
//   per K step, read in the per-group block layout (commit fixing the scale_a
//   addressing), and the weight block scales of the tile's two 128-column
//   blocks.
// * Weights: group g is rows [g N, g N + N) of one [G N, K] operand, plain
//   or preshuffled (the dense kernel's B layout); the last tile of a group
//   whose N is not a multiple of 256 reads the next group's rows (or zeros
//   past the end), which no stored output uses.
//
// FMT = F_BF16: the BF16 grouped GEMM ("PyTorch on AMD GPUs gains a FlyDSL
// backend", Interpretation: grouped GEMM over uneven and empty expert
// groups) on the same pipeline: BF16 operands (a 128-byte K chunk holds 64
// elements, two 16x16x32 BF16 matrix-core instructions per fragment pair),
// no scales, FP32 accumulation, BF16 output.
template <bool PSB, int FMT = F_E4M3>
__global__ __launch_bounds__(DNW8 * 64, 1) void grouped_dense_kernel(DenseArgs p) {
  typedef DenseLoop<FMT, FMT, FMT == F_BF16 ? SM_GNONE : SM_GROUP, false, false, PSB> L;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::LDS_BYTES];
  __shared__ GroupTable gt;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w == 0) build_group_table<DBM>(p.m_sizes, p.G, p.M, gt, lane);
  __syncthreads();
  const int tiles_m = uni32(gt.mtile[p.G]);          // 256-row tiles over all groups
  const int P = (int)gridDim.x;
  // tiles [nb, tiles_m * tiles_n) are left to the streaming kernel
  const int nb = grouped_split_end(tiles_m * p.tiles_n, P, p.tail_grid, p.tail_rounds);
  const int bid = (int)blockIdx.x;
  if (bid >= nb) return;
  const int ntiles = (nb - bid + P - 1) / P;

  typename L::Ctx c;
  L::init(c, p, smem);
  auto tile_at = [&](int k, int &tm, int &tn) {
    int P_ = P, tm_ = tiles_m, tn_ = p.tiles_n;
    asm volatile("" : "+s"(P_), "+s"(tm_), "+s"(tn_));
    persistent_tile(bid, k, P_, tm_, tn_, tm, tn);
  };
  auto resolve = [&](int tm, int tn) -> TileId {
    const int g = group_of_tile(gt, p.G, tm);
    const int64_t start = uni32(gt.rows[g]);
    const int64_t mg = uni32(gt.rows[g + 1]) - start;
    const int64_t m0 = start + (int64_t)(tm - uni32(gt.mtile[g])) * DBM;
    return TileId{m0, (int64_t)tn * DBN, start + mg, start, mg, g};
  };
  L::run(c, ntiles, tile_at, resolve, 1.0f, smem);
}

}  // namespace mxg
