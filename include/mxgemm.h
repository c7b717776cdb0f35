/*
 * mxgemm.h -- C ABI of the MI355X (gfx950) block-scaled GEMM library.
 *
 * One operation, three scale families:
 *
 *     D[m,n] = sum_k a(m,k) * b(n,k)        (FP32 accumulation, BF16 output)
 *
 * with a, b the dequantized operands:
 *   MX          a = dec(qA[m,k]) * 2^(eA[m,k/32]-127)       (E8M0 per 32 K)
 *   tensor-wise a = dec(qA[m,k]) * sA                        (one FP32)
 *   groupwise   a = dec(XQ[r,k]) * xs(r,k/128), b = dec(WQ[g,n,k]) * ws[g,n/128,k/128]
 *
 * Sources: "Experimental FlyDSL GEMM backend for TE PyTorch
 * (BF16/FP16/FP32/FP8/MXFP8)" (Summary; Supported Data Types; Validation: the
 * TN/NN/NT layouts, mixed E4M3/E5M2, MXFP8); "Add FlyDSL grouped groupwise
 * FP8 GEMM for ROCm" (PR body: plain and preshuffled [G,N,K] weights, N and K
 * multiples of 128, activation scales in the per-group block layout; Tile
 * selection: grid from static shapes only, no host read of tensor contents,
 * one kernel per call; Architecture support: wide scaled MFMA with a neutral
 * E8M0 scale and FP32 scales applied in software); "[gfx1250] Add MXFP4 GEMM
 * support to FlyDSL backend" (Description: plain scales in, shuffled inside);
 * "PyTorch on AMD GPUs gains a FlyDSL backend" (Interpretation: FP8 or packed
 * FP4 operands, one E8M0 scale per 32 values along K, NT scaled GEMM).
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains caller memory and uses no workspace.
 *  - Calls are stream-ordered and asynchronous: exactly one kernel is
 *    enqueued on `stream` (0 = the null stream) per successful call, with
 *    two exceptions: mxgemm_quantize_tensor enqueues four (its scale output
 *    serves as the amax word between them; see there), and
 *    grouped_fp8_gemm_run and grouped_bf16_gemm_run enqueue two when they
 *    run MXG_GROUPED_TILED on more 256 x 256 tiles than the device has
 *    compute units (see grouped_fp8_gemm_variant).  The tuning call grouped_fp8_gemm_autotune
 *    is the one call that waits for the device (see there).
 *  - All argument checks are synchronous and happen before anything is
 *    enqueued; on error nothing is enqueued and outputs are untouched.
 *  - No C++ exception crosses this ABI.  Returns MXG_OK (0) or a negative
 *    mxg_status; mxgemm_status_string() names it.
 *  - The host never reads device data, so calls are safe to capture into a
 *    HIP graph after mxgemm_init().
 *  - Sizes are int64.  M, N (or totM) == 0 is a no-op returning MXG_OK;
 *    K == 0 writes zeros.
 *  - Layout names are row-major, first letter for A, second for B:
 *      A 'N' = [M,K] (K contiguous)   A 'T' = [K,M] (M contiguous)
 *      B 'T' = [N,K] (K contiguous)   B 'N' = [K,N] (N contiguous)
 *    so NT is D = A * B^T with both operands K-contiguous.
 *  - D is BF16 (raw uint16 bits), row-major [M,N], rounded to nearest even.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXG_OK = 0,
  MXG_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum          */
  MXG_ERR_UNSUPPORTED = -2,   /* combination or divisibility not built          */
  MXG_ERR_MISALIGNED = -3,    /* a pointer is not 16-byte aligned               */
  MXG_ERR_HIP = -4,           /* the HIP runtime reported an error              */
  MXG_ERR_IO = -5             /* tune cache file unreadable, unwritable, malformed */
} mxg_status;

/* Operand format = element encoding + scale kind (one per operand). */
enum {
  MXG_MXFP8_E4M3 = 0,         /* E4M3 codes + E8M0 scale per 32 along K          */
  MXG_MXFP8_E5M2 = 1,         /* E5M2 codes + E8M0 scale per 32 along K          */
  MXG_MXFP4_E2M1 = 4,         /* E2M1 codes two per byte (element 2j in bits 3:0,
                                 2j+1 in bits 7:4) + E8M0 scale per 32 along K  */
  MXG_FP8_E4M3_TENSOR = 16,   /* E4M3 codes + one FP32 dequant multiplier        */
  MXG_FP8_E5M2_TENSOR = 17    /* E5M2 codes + one FP32 dequant multiplier        */
};

/* OR into fmtB: B's codes (and, for MX, sB) were produced by
 * mxgemm_preshuffle_b / mxgemm_preshuffle_scales. */
#define MXG_PRESHUFFLED 0x100

enum { MXG_NT = 0, MXG_NN = 1, MXG_TN = 2 };

/* Largest G accepted by grouped_fp8_gemm_run. */
#define MXG_GROUPED_MAX_G 1024

/*
 * mxgemm_init -- load the library's code objects on the current device and
 * query its compute-unit count once, so that later calls read no device
 * state and can be captured into a HIP graph ("Add FlyDSL grouped groupwise
 * FP8 GEMM for ROCm", Tile selection: a captured call must not depend on
 * anything a capture cannot replay).  Call once per device before capture.
 * Idempotent.  Returns MXG_OK, or MXG_ERR_HIP if no device is usable.
 */
int mxgemm_init(void);

/* Static description of a status code ("ok", "invalid argument", ...);
 * never freed, never NULL ("unknown status" for a code not listed above).
 * The pages' wrappers report unsupported configurations rather than
 * failing silently ("Experimental FlyDSL GEMM backend for TE PyTorch",
 * Summary: unsupported configs fall back); this library has no fallback and
 * names the reason instead. */
const char *mxgemm_status_string(int status);

/*
 * mxgemm_run -- dense block-scaled GEMM D[M,N] = sum_k a(m,k) b(n,k).
 *
 * fmtA, fmtB  operand formats (MXG_MXFP8_*, MXG_MXFP4_E2M1, MXG_FP8_*_TENSOR);
 *             both MX or both tensor-wise; E2M1 only with E2M1.  fmtB may
 *             carry MXG_PRESHUFFLED (NT only).
 * layout      MXG_NT, MXG_NN or MXG_TN (see the header comment).
 * A, B        codes: uint8, row-major in the layout's storage shape.  E2M1 is
 *             packed two per byte along the contiguous dimension (element
 *             2j in bits 3:0): along K for a K-contiguous operand, along M
 *             (A 'T') or N (B 'N') for a transposed one ("[gfx1250] Add
 *             MXFP4 GEMM support to FlyDSL backend", review of the MXFP4
 *             storage chosen per layout: rowwise or columnwise buffers).
 * sA, sB      MX: uint8 E8M0 [rows, K/32] row-major (rows = M for A, N for B),
 *             always blocked along K whatever the code layout; a preshuffled
 *             sB has the size given by mxgemm_preshuffle_scales_bytes(N, K).
 *             Tensor-wise: pointer to one float (device), the dequant
 *             multiplier (value = code value * s).
 * D           BF16 [M,N] row-major, written in full.
 * Divisibility: MX needs K % 128 == 0 (E2M1: K % 256 == 0); NN/TN need the
 *             contiguous dimension of each transposed operand (M for A 'T',
 *             N for B 'N') to be a multiple of 16 (E2M1: 32), and each transposed
 *             operand to hold fewer than 2^31 - 16 bytes, and a
 *             preshuffled B to hold fewer than 2^32 - 2^16 bytes.  Otherwise
 *             MXG_ERR_UNSUPPORTED.  A, B, sA, sB and D must be 16-byte
 *             aligned (MXG_ERR_MISALIGNED).
 * Edge rows/columns (M, N not multiples of the tile) are masked.
 */
int mxgemm_run(int fmtA, int fmtB, int layout,
               const void *A, const void *sA, const void *B, const void *sB,
               void *D, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * mxgemm_dense_variant: which kernel mxgemm_run / mxgemm_run_fused launch
 * for these static shapes on the current device: MXG_DENSE_TILE256, the
 * persistent kernel with 256 x 256 tiles, or MXG_DENSE_TILE64 (NT only),
 * 64 x 64 tiles with one workgroup each, for outputs too small to occupy
 * the device with 256 x 256 tiles ("Add FlyDSL grouped groupwise FP8 GEMM
 * for ROCm", Tile selection and Performance: the tile is picked per shape,
 * and narrow outputs lose when they cannot produce enough tiles).  Both
 * compute the same function with the same per-element sequence of
 * matrix-core instructions, so their outputs are identical.  Never fails.
 */
enum { MXG_DENSE_TILE256 = 0, MXG_DENSE_TILE64 = 1 };
int mxgemm_dense_variant(int fmtA, int fmtB, int layout, int64_t M, int64_t N, int64_t K);

/* Host-only check of mxgemm_run's arguments (no device call), for the
 * operation cited at mxgemm_run.  Returns the status mxgemm_run would return
 * before enqueueing anything. */
int mxgemm_validate(int fmtA, int fmtB, int layout,
                    const void *A, const void *sA, const void *B, const void *sB,
                    const void *D, int64_t M, int64_t N, int64_t K);

/*
 * mxgemm_run_fused -- mxgemm_run with the epilogue of a linear layer's
 * forward GEMM fused into the kernel:
 *
 *     D[m,n] = act( sum_k a(m,k) b(n,k) + bias[n] )
 *
 * "[gfx1250] Add MXFP4 GEMM support to FlyDSL backend" (Description): the
 * GEMM's activation and bias are its stated follow-up; the pages name no
 * function, so the set below is this library's reading.  The sum (scaled by
 * sA*sB for tensor-wise operands) stays in FP32, the bias is added and the
 * activation applied in FP32, and the result is rounded once to BF16.
 *
 * bias        device BF16 [N] (raw uint16 bits), 4-byte aligned, or NULL.
 * activation  MXG_ACT_NONE, MXG_ACT_RELU (max(z, 0)), MXG_ACT_GELU_TANH
 *             (z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))) or MXG_ACT_SILU
 *             (z / (1 + e^-z)); the GPU evaluates both logistic forms with
 *             its base-2 exponential and reciprocal instructions.
 * Everything else as mxgemm_run.  With a bias or an activation only the NT
 * layout (the forward GEMM) is built, and a bias needs N even
 * (MXG_ERR_UNSUPPORTED otherwise); an unknown activation is
 * MXG_ERR_INVALID_ARG, a misaligned bias MXG_ERR_MISALIGNED.  With
 * bias == NULL and MXG_ACT_NONE the call is mxgemm_run.  K == 0 writes
 * act(bias[n]).
 */
enum { MXG_ACT_NONE = 0, MXG_ACT_RELU = 1, MXG_ACT_GELU_TANH = 2, MXG_ACT_SILU = 3 };
int mxgemm_run_fused(int fmtA, int fmtB, int layout,
                     const void *A, const void *sA, const void *B, const void *sB,
                     void *D, int64_t M, int64_t N, int64_t K,
                     const void *bias, int activation, hipStream_t stream);

/* Host-only check of mxgemm_run_fused's arguments (no device call), for the
 * operation cited at mxgemm_run_fused; same return as that call's checks. */
int mxgemm_validate_fused(int fmtA, int fmtB, int layout,
                          const void *A, const void *sA, const void *B, const void *sB,
                          const void *D, int64_t M, int64_t N, int64_t K,
                          const void *bias, int activation);

/*
 * grouped_fp8_gemm_run -- grouped groupwise FP8 GEMM (one GEMM per group of
 * rows, e.g. per expert): "Add FlyDSL grouped groupwise FP8 GEMM for ROCm"
 * (PR body: E4M3 X and W with FP32 1x128 activation and 128x128 weight
 * scales, plain or preshuffled [G,N,K] weights, BF16 out; commit message
 * fixing the scale_a addressing: the per-group block layout of x_scale;
 * Tile selection: the grid comes from static shapes only and m_sizes is
 * resolved in the kernel; Architecture support: the scaled matrix-core
 * instruction with a neutral E8M0 scale and the FP32 scales applied in
 * software per 128-K block).
 *
 * G           number of groups, 1 <= G <= MXG_GROUPED_MAX_G.
 * m_sizes     device int64[G]: rows per group, in order.  Group g owns rows
 *             [start_g, start_g + m_sizes[g]) with start_g the prefix sum.
 *             Caller precondition (not checked: the host reads no device
 *             data): m_sizes[g] >= 0 and sum = totM.  The kernel clamps every
 *             group to [0, totM), so a violated precondition can leave rows
 *             unwritten but never touches memory outside D.
 * XQ          E4M3 [totM, K] row-major.
 * x_scale     FP32, totM*K/128 values in the per-group block layout: group
 *             g's block begins at start_g*(K/128) and holds (local row i,
 *             k-block kb) at i + kb*m_sizes[g].
 * WQ          E4M3 weights [G, N, K] row-major, or (b_preshuffled != 0) the
 *             output of grouped_fp8_preshuffle_b.
 * w_scale     FP32 [G, N/128, K/128] row-major (one per 128x128 block).
 * D           BF16 [totM, N] row-major; rows of empty groups do not exist,
 *             rows outside every group are left untouched.
 * N and K must be multiples of 128 (MXG_ERR_UNSUPPORTED).
 */
int grouped_fp8_gemm_run(int G, const int64_t *m_sizes,
                         const void *XQ, const float *x_scale,
                         const void *WQ, const float *w_scale,
                         void *D, int64_t totM, int64_t N, int64_t K,
                         int b_preshuffled, hipStream_t stream);

int grouped_fp8_gemm_validate(int G, const int64_t *m_sizes,
                              const void *XQ, const float *x_scale,
                              const void *WQ, const float *w_scale,
                              const void *D, int64_t totM, int64_t N, int64_t K,
                              int b_preshuffled);

/*
 * grouped_fp8_gemm_variant: which kernel grouped_fp8_gemm_run launches for
 * these static shapes (and b_preshuffled) on the current device (the
 * choice never depends on m_sizes' contents): MXG_GROUPED_STREAM64 or
 * MXG_GROUPED_STREAM128, the persistent kernel with 64 x 64 or 128 x 128
 * tiles for the weight-streaming regime (few rows per group), or
 * MXG_GROUPED_TILED, the persistent 256 x 256 kernel on the dense pipeline
 * for the matrix-core regime (one tile per compute unit per round; when a
 * last, partial round would leave most compute units idle, its tiles go to
 * the streaming kernel, launched after it, as 128 x 64 or 64 x 64 pieces).  A
 * static table keyed on (nextPow2(totM), N, K, b_preshuffled) decides for
 * the shapes it lists ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm",
 * Tile selection: the same key), an estimate of each kernel's time
 * otherwise.  All run the same per-element arithmetic (one matrix-core
 * partial per 128-K block, scaled and added in FP32 in K order), so their
 * outputs are identical up to the sign of an exactly zero result.  Never
 * fails.
 */
enum { MXG_GROUPED_STREAM64 = 0, MXG_GROUPED_TILED = 1, MXG_GROUPED_STREAM128 = 2 };
int grouped_fp8_gemm_variant(int G, int64_t totM, int64_t N, int64_t K, int b_preshuffled);

/*
 * Autotuning of the grouped kernel choice ("Add FlyDSL grouped groupwise
 * FP8 GEMM for ROCm", Tile selection: winners are autotuned per shape and
 * persisted in a cache keyed on (nextPow2(totM), N, K, b_preshuffled), the
 * static table being the default).  The cache here is keyed on (G,
 * nextPow2(totM), N, K, b_preshuffled), lives in the process, is shared by
 * every thread and device, and is consulted by grouped_fp8_gemm_variant
 * (and so by grouped_fp8_gemm_run) before the static table.
 *
 * grouped_fp8_gemm_autotune: runs the grouped GEMM of these arguments
 * (validated as grouped_fp8_gemm_run validates them) with each of the three
 * kernels, once untimed and then `reps` times (1..1000), timed with HIP
 * events on `stream`; records the fastest in the cache and returns it in
 * *variant_out (may be NULL) and the three mean times in us_out[variant]
 * (three floats, microseconds per call, indexed by MXG_GROUPED_*; may be
 * NULL).  D holds a correct result afterwards.  Unlike every other call it
 * waits for the device (it synchronizes on its events), so it must not be
 * called while `stream` is being captured (MXG_ERR_INVALID_ARG); totM, N or
 * K of 0 is MXG_ERR_INVALID_ARG (nothing to time).  Tune before capture.
 *
 * mxgemm_tune_cache_save / _load: write the cache to, or merge entries from,
 * a text file: a '#' comment line, then one line per entry,
 * "grouped G log2m N K b_preshuffled variant" (log2m: log2 of nextPow2(totM)).
 * A file that cannot be opened or written, or any malformed line, is
 * MXG_ERR_IO; a failed load changes nothing.  NULL path: MXG_ERR_INVALID_ARG.
 * mxgemm_tune_cache_clear empties the cache; mxgemm_tune_cache_size counts
 * its entries.  These four never touch the device.
 */
int grouped_fp8_gemm_autotune(int G, const int64_t *m_sizes,
                              const void *XQ, const float *x_scale,
                              const void *WQ, const float *w_scale,
                              void *D, int64_t totM, int64_t N, int64_t K,
                              int b_preshuffled, int reps, int *variant_out,
                              float *us_out, hipStream_t stream);
int mxgemm_tune_cache_save(const char *path);
int mxgemm_tune_cache_load(const char *path);
int mxgemm_tune_cache_clear(void);
int64_t mxgemm_tune_cache_size(void);

/*
 * Preshuffle: one-time re-layout of a B operand (weights) into the order in
 * which the matrix-core K-loop consumes it ("Add FlyDSL grouped groupwise FP8
 * GEMM for ROCm", PR body: callers shuffle once at load time).
 *
 * mxgemm_preshuffle_b: B codes of format fmtB (E4M3/E5M2/E2M1, MX or tensor)
 * stored per `layout`'s B ('T' = [N,K], 'N' = [K,N]; E2M1 only [N,K]) ->
 * B_out of mxgemm_preshuffle_b_bytes(fmtB, N, K) bytes, consumable by
 * mxgemm_run with fmtB | MXG_PRESHUFFLED and layout MXG_NT.  N is padded to
 * a multiple of 256 and the padding is zero-filled.  K must satisfy mxgemm_run's divisibility rule.
 */
int64_t mxgemm_preshuffle_b_bytes(int fmtB, int64_t N, int64_t K);
int mxgemm_preshuffle_b(int fmtB, int layout, const void *B, void *B_out,
                        int64_t N, int64_t K, hipStream_t stream);

/*
 * mxgemm_preshuffle_scales: E8M0 scales [rows, K/32] -> s_out of
 * mxgemm_preshuffle_scales_bytes(rows, K) bytes, in per-lane order (one
 * 32-bit word per lane covers four consecutive 128-K steps).  Padding is
 * filled with 127 (scale 1).  "[gfx1250] Add MXFP4 GEMM support to FlyDSL
 * backend" (Description: callers pass plain scales and the library reorders
 * them once so that the K loop reads them in iteration order).
 * s: device uint8 [rows, K/32], 4-byte aligned; s_out: device, 16-byte
 * aligned, caller-allocated.  Errors: MXG_ERR_INVALID_ARG (negative size,
 * null pointer), MXG_ERR_UNSUPPORTED (K % 32 != 0), MXG_ERR_MISALIGNED.
 * rows or K = 0: no-op.
 */
int64_t mxgemm_preshuffle_scales_bytes(int64_t rows, int64_t K);
int mxgemm_preshuffle_scales(const void *s, void *s_out, int64_t rows, int64_t K,
                             hipStream_t stream);

/*
 * grouped_bf16_gemm_run -- BF16 grouped GEMM over uneven and empty groups
 * of rows ("PyTorch on AMD GPUs gains a FlyDSL backend", Interpretation:
 * grouped GEMM that tolerates uneven and empty expert groups, with BF16
 * grouped cases in its operator suite; "Experimental FlyDSL GEMM backend for
 * TE PyTorch", Supported Data Types: BF16 inputs).  For each group g of
 * rows [start_g, start_g + m_sizes[g]):
 *     D[r, n] = sum_k x(r, k) * w(g, n, k)
 * with BF16 operands, FP32 accumulation and one rounding to BF16 (RNE).
 *
 * G, m_sizes, totM, D, b_preshuffled: as grouped_fp8_gemm_run (caller
 *             precondition sum(m_sizes) = totM, rows outside every group
 *             untouched, empty groups own no rows).
 * X           BF16 [totM, K] row-major (K contiguous), 16-byte aligned.
 * W           BF16 [G, N, K] row-major, 16-byte aligned, or (b_preshuffled
 *             != 0) the output of grouped_bf16_preshuffle_b.
 * N and K must be multiples of 64 (MXG_ERR_UNSUPPORTED).  K == 0 writes
 * zeros to every row of every group.  The kernel is the one
 * grouped_bf16_gemm_variant names (the three kernels of the FP8 grouped
 * GEMM, with BF16 operands; the 256 x 256 one followed, when its last round
 * is partial, by the streaming kernel on that round's tiles).
 * Errors as grouped_fp8_gemm_run.
 */
int grouped_bf16_gemm_run(int G, const int64_t *m_sizes, const void *X, const void *W, void *D,
                          int64_t totM, int64_t N, int64_t K, int b_preshuffled, hipStream_t stream);

/* Which kernel grouped_bf16_gemm_run launches for these static shapes
 * (MXG_GROUPED_*, as grouped_fp8_gemm_variant): the same cost model with
 * each 128-byte K step holding 64 BF16 values, no static table ("Add FlyDSL
 * grouped groupwise FP8 GEMM for ROCm", Tile selection: the tile is picked
 * per shape from static shapes alone).  All three compute the same
 * per-element sequence (one 64-value partial per 128-byte K step, added in
 * K order in FP32), so their outputs are identical.  Never fails. */
int grouped_bf16_gemm_variant(int G, int64_t totM, int64_t N, int64_t K);

/* Host-only check of grouped_bf16_gemm_run's arguments (no device call), for
 * the operation cited there; same return as that call's checks. */
int grouped_bf16_gemm_validate(int G, const int64_t *m_sizes, const void *X, const void *W,
                               const void *D, int64_t totM, int64_t N, int64_t K, int b_preshuffled);

/*
 * grouped_bf16_preshuffle_b -- the one-time weight swizzle of the BF16
 * grouped GEMM ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", PR body:
 * weights preshuffled once at load time into the matrix-core operand order).
 * W: BF16 [G, N, K], 16-byte aligned; W_out: caller-allocated, the same
 * G*N*K*2 bytes, 16-byte aligned, not overlapping W.  N and K multiples of
 * 64 (MXG_ERR_UNSUPPORTED); MXG_ERR_INVALID_ARG for G outside
 * 1..MXG_GROUPED_MAX_G, a negative size or a null pointer;
 * MXG_ERR_MISALIGNED.  N or K = 0: no-op.
 */
int grouped_bf16_preshuffle_b(int G, const void *W, void *W_out, int64_t N, int64_t K,
                              hipStream_t stream);

/*
 * grouped_fp8_preshuffle_b -- the one-time weight swizzle that callers run at
 * load time so that the grouped GEMM reads its B operand in the order its
 * matrix-core K-loop consumes it ("Add FlyDSL grouped groupwise FP8 GEMM for
 * ROCm", PR body: the preshuffled sibling op and its weight swizzle).
 *
 * WQ      device E4M3 [G, N, K] row-major (K contiguous), 16-byte aligned.
 * WQ_out  device, caller-allocated, the same G*N*K bytes, 16-byte aligned;
 *         each group's [N, K] block becomes the preshuffled block that
 *         grouped_fp8_gemm_run reads with b_preshuffled = 1.  Must not
 *         overlap WQ.
 * Errors: MXG_ERR_INVALID_ARG (G outside 1..MXG_GROUPED_MAX_G, negative
 * size, null pointer), MXG_ERR_UNSUPPORTED (N or K not a multiple of 128,
 * the weight scale-block size), MXG_ERR_MISALIGNED.  N or K = 0: no-op.
 */
int grouped_fp8_preshuffle_b(int G, const void *WQ, void *WQ_out,
                             int64_t N, int64_t K, hipStream_t stream);

/*
 * mxgemm_quantize_mx -- FP32 data -> MX operand (codes + E8M0 scales), the
 * step that produces mxgemm_run's MX inputs ("PyTorch on AMD GPUs gains a
 * FlyDSL backend", Interpretation: one E8M0 scale per 32 values along K).
 *
 * fmt     MXG_MXFP8_E4M3, MXG_MXFP8_E5M2 or MXG_MXFP4_E2M1.
 * x       device FP32 [rows, K] row-major (K contiguous), 16-byte aligned.
 * codes   device out: [rows, K] bytes (FP8) or [rows, K/2] (E2M1, element
 *         2j in bits 3:0), 16-byte aligned.
 * scales  device out: E8M0 [rows, K/32] bytes.
 * Per 32-value block: X = floor(log2(amax / fmt_max)) exactly (fmt_max 448,
 * 57344 or 6; X = -127 for an all-zero block; clamped to [-127, 127]),
 * scale code X + 127, element code = nearest representable value of
 * x * 2^-X, ties to the even code, saturating at +-fmt_max.  Inputs must be
 * finite.  The caller owns every buffer; nothing is allocated.
 * Errors (before anything is enqueued): MXG_ERR_INVALID_ARG (not an MX fmt,
 * negative size, null pointer), MXG_ERR_UNSUPPORTED (K % 32 != 0, sizes
 * past the 32-bit grid), MXG_ERR_MISALIGNED.  rows or K = 0: no-op.
 */
int mxgemm_quantize_mx(int fmt, const float *x, void *codes, void *scales,
                       int64_t rows, int64_t K, hipStream_t stream);

/*
 * mxgemm_quantize_tensor -- FP32 data -> tensor-wise FP8 operand (codes +
 * one FP32 dequant scale), the step that produces mxgemm_run's tensor-wise
 * inputs ("Experimental FlyDSL GEMM backend for TE PyTorch", Supported Data
 * Types: tensor-wise FP8, scales from the tensor's amax).
 *
 * fmt     MXG_FP8_E4M3_TENSOR or MXG_FP8_E5M2_TENSOR.
 * x       device FP32, n values (any shape, flattened), 16-byte aligned.
 * codes   device out: n bytes, 16-byte aligned.
 * scale   device out: one FP32, 4-byte aligned: s = amax(|x|) / fmt_max
 *         (448 or 57344) as an FP32 quotient, 1.0 when every value is zero
 *         (and for n = 0); pass it as mxgemm_run's sA or sB.
 * Element code = nearest representable value of the FP32 quotient x / s,
 * ties to the even code, saturating at +-fmt_max.  Inputs must be finite.
 * Four launches on `stream` (clear, amax, encode, scale); until the last
 * one completes the scale word holds the amax bits, so calls that share a
 * scale pointer must not overlap.  Nothing is allocated.
 * Errors (before anything is enqueued): MXG_ERR_INVALID_ARG (not a
 * tensor-wise fmt, n < 0, null pointer), MXG_ERR_UNSUPPORTED (n % 8 != 0,
 * sizes past the 32-bit grid), MXG_ERR_MISALIGNED.
 */
int mxgemm_quantize_tensor(int fmt, const float *x, void *codes, float *scale, int64_t n,
                           hipStream_t stream);

/*
 * grouped_fp8_quantize_act -- FP32 activations -> the XQ and x_scale inputs
 * of grouped_fp8_gemm_run: E4M3 codes with one FP32 scale per row and
 * 128-value K block ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", PR
 * body), the scales in the per-group block layout (commit message fixing
 * the scale_a addressing): (row r of group g, block kb) at
 * start_g * (K/128) + (r - start_g) + kb * m_sizes[g].
 *
 * G, m_sizes   as for grouped_fp8_gemm_run (device int64[G], 8-byte aligned;
 *              the host does not read it).  Negative sizes count as 0 and
 *              the groups are cut at totM; rows in no group are not written.
 * x            device FP32 [totM, K] row-major, 16-byte aligned.
 * codes        device out: E4M3 [totM, K], 16-byte aligned.
 * x_scale      device out: FP32, totM * K / 128 entries, 4-byte aligned.
 * Per block: s = amax / 448 as an FP32 quotient (1.0 for an all-zero
 * block); element code = nearest E4M3 value of the FP32 quotient x / s,
 * ties to the even code, saturating at +-448.  Inputs must be finite.
 * Errors: MXG_ERR_UNSUPPORTED (G outside [1, MXG_GROUPED_MAX_G],
 * K % 128 != 0, sizes past the 32-bit scale offsets), MXG_ERR_INVALID_ARG,
 * MXG_ERR_MISALIGNED.  totM or K = 0: no-op.
 */
int grouped_fp8_quantize_act(int G, const int64_t *m_sizes, const float *x, void *codes,
                             float *x_scale, int64_t totM, int64_t K, hipStream_t stream);

/*
 * grouped_fp8_quantize_weight -- FP32 weights -> the WQ and w_scale inputs
 * of grouped_fp8_gemm_run: E4M3 codes with one FP32 scale per 128 x 128
 * block ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", PR body).
 *
 * w        device FP32 [G, N, K] row-major (K contiguous), 16-byte aligned.
 * codes    device out: E4M3 [G, N, K] (plain layout; grouped_fp8_preshuffle_b
 *          makes the preshuffled one), 4-byte aligned.
 * w_scale  device out: FP32 [G, N/128, K/128] row-major, 4-byte aligned.
 * Per block: s = amax / 448 as an FP32 quotient (1.0 for an all-zero
 * block); element code = nearest E4M3 value of the FP32 quotient w / s,
 * ties to the even code, saturating.  Inputs must be finite.
 * Errors: MXG_ERR_UNSUPPORTED (G outside [1, MXG_GROUPED_MAX_G], N or K not
 * a multiple of 128), MXG_ERR_INVALID_ARG, MXG_ERR_MISALIGNED.  N or K = 0:
 * no-op.
 */
int grouped_fp8_quantize_weight(int G, const float *w, void *codes, float *w_scale,
                                int64_t N, int64_t K, hipStream_t stream);

/*
 * mxgemm_mfma_ceiling -- a measurement aid, not part of the GEMM path: one
 * workgroup per compute unit, eight waves each running 32 independent chains
 * of the scaled 16x16x128 matrix-core instruction that the GEMMs are built on
 * ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", Architecture support)
 * for `iters` iterations
 * (2 * 16 * 16 * 128 FLOP per instruction), E4M3 operands for an FP8 fmt and
 * E2M1 for MXG_MXFP4_E2M1, neutral scales.  Its time gives the throughput the
 * instruction sustains on this device with nothing else running.  clk: device
 * memory for three uint64 (8-byte aligned); the call writes the shader-clock
 * ticks (s_memtime) and 100 MHz reference ticks (s_memrealtime) that wave 0
 * of workgroup 0 spent in the loop to clk[0] and clk[1] (their ratio times
 * 100 MHz is the shader clock under that load).  Errors: MXG_ERR_INVALID_ARG
 * (unknown fmt, iters < 0, null clk), MXG_ERR_MISALIGNED.
 */
int mxgemm_mfma_ceiling(int fmt, int64_t iters, void *clk, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
