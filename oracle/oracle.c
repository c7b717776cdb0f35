/*
 * oracle.c -- plain FP64 CPU reference for block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: every decoder below is
 * written out from the closed forms of the element formats.
 *
 * What it computes (the plain definition of the method):
 *
 *     D[m,n] = sum_k  a(m,k) * b(n,k)
 *
 * where a and b are the dequantized operands.  Block scaling is only an
 * encoding of a and b; the method ("Add FlyDSL grouped groupwise FP8 GEMM for
 * ROCm", section "Architecture support"; "PyTorch on AMD GPUs gains a FlyDSL
 * backend", section "Interpretation") reaches this same sum with FP32
 * accumulation on matrix cores.  Here every dequantized value and every
 * product is formed in FP64 and summed in FP64 in plain k order, with no
 * blocking and no reordering.
 *
 * Element formats (OCP Microscaling Formats MX v1.0; external to the pages,
 * which only name the formats -- "Experimental FlyDSL GEMM backend for TE
 * PyTorch", section "Supported Data Types"; "PyTorch on AMD GPUs gains a
 * FlyDSL backend", section "Interpretation"):
 *   E4M3: bias 7, no infinities, S.1111.111 is NaN, max 448.
 *   E5M2: bias 15, IEEE-like: exponent 31 is Inf (m=0) or NaN.
 *   E2M1: bias 1, no Inf/NaN, values {0,.5,1,1.5,2,3,4,6}.
 *   E8M0: 2^(c-127); c=255 is NaN.
 *   BF16 (operands of the BF16 grouped GEMM): bias 127, 7 fraction bits,
 *   IEEE-like specials (the upper half of an IEEE binary32).
 *
 * Parity status: every function here is pinned by CPU tests (closed forms,
 * an independent library decoder, exact rational brute force, one-hot and
 * identity inputs, exact scale doubling, reduction to a library matmul).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

/* Element-format selectors for this file (the oracle's own numbering). */
#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_E2M1 4

/* Scale kinds. */
#define ORC_SCALE_MX     0   /* one E8M0 byte per 32 consecutive K values   */
#define ORC_SCALE_TENSOR 1   /* one FP32 dequant multiplier for the tensor  */

/* ---- element decoders (closed forms) ---------------------------------- */

double oracle_decode_e4m3(unsigned c)
{
    unsigned s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
    double v;
    if (e == 15u && m == 7u) return NAN;           /* the only NaN pattern */
    if (e == 0u) v = ldexp((double)m, -9);          /* subnormal: m * 2^-9  */
    else v = ldexp((double)(8u + m), (int)e - 10);  /* (1+m/8) * 2^(e-7)    */
    return s ? -v : v;
}

double oracle_decode_e5m2(unsigned c)
{
    unsigned s = (c >> 7) & 1u, e = (c >> 2) & 31u, m = c & 3u;
    double v;
    if (e == 31u) {
        if (m == 0u) return s ? -INFINITY : INFINITY;
        return NAN;
    }
    if (e == 0u) v = ldexp((double)m, -16);         /* m * 2^-16            */
    else v = ldexp((double)(4u + m), (int)e - 17);  /* (1+m/4) * 2^(e-15)   */
    return s ? -v : v;
}

double oracle_decode_e2m1(unsigned nib)
{
    unsigned s = (nib >> 3) & 1u, e = (nib >> 1) & 3u, m = nib & 1u;
    double v;
    if (e == 0u) v = 0.5 * (double)m;               /* subnormal: m * 2^-1  */
    else v = ldexp((double)(2u + m), (int)e - 2);   /* (1+m/2) * 2^(e-1)    */
    return s ? -v : v;
}

double oracle_decode_e8m0(unsigned c)
{
    c &= 255u;
    if (c == 255u) return NAN;
    return ldexp(1.0, (int)c - 127);
}

double oracle_decode(int fmt, unsigned code)
{
    switch (fmt) {
    case ORC_E4M3: return oracle_decode_e4m3(code & 255u);
    case ORC_E5M2: return oracle_decode_e5m2(code & 255u);
    case ORC_E2M1: return oracle_decode_e2m1(code & 15u);
    default: return NAN;
    }
}

/* ---- operand element access -------------------------------------------
 *
 * An operand is a logical [rows, K] matrix (rows = M for A, N for B).
 * Storage:
 *   transposed == 0 : codes row-major [rows, K]   (K contiguous)
 *   transposed == 1 : codes row-major [K, rows]   (rows contiguous)
 * For E2M1, two codes share a byte along the contiguous dimension; the
 * element with the even index sits in the low nibble (bits 3:0).
 * MX scales are always blocked along K and stored [rows, K/32] row-major,
 * whatever the code layout ("[gfx1250] Add MXFP4 GEMM support to FlyDSL
 * backend", review thread: rowwise and columnwise copies each carry their
 * own K-blocked scales).  Tensor scales are one float.
 */
typedef struct {
    int fmt;             /* ORC_E4M3 / ORC_E5M2 / ORC_E2M1 */
    int scale_kind;      /* ORC_SCALE_MX / ORC_SCALE_TENSOR */
    int transposed;
    const uint8_t *codes;
    const void *scales;
    int64_t rows, K;
} orc_operand;

static unsigned orc_code(const orc_operand *op, int64_t r, int64_t k)
{
    int64_t idx, ld;
    if (!op->transposed) { idx = r * op->K + k; ld = idx; }
    else { idx = k * op->rows + r; ld = idx; }
    if (op->fmt == ORC_E2M1) {
        uint8_t byte = op->codes[ld / 2];
        return (ld & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    }
    return op->codes[ld];
}

static double orc_scale(const orc_operand *op, int64_t r, int64_t k)
{
    if (op->scale_kind == ORC_SCALE_TENSOR)
        return (double)*(const float *)op->scales;
    return oracle_decode_e8m0(((const uint8_t *)op->scales)[r * (op->K / 32) + k / 32]);
}

/* Dequantized value a(r,k) = decode(code) * scale. */
static double orc_value(const orc_operand *op, int64_t r, int64_t k)
{
    return oracle_decode(op->fmt, orc_code(op, r, k)) * orc_scale(op, r, k);
}

/* Dequantize a whole operand into a row-major [rows, K] FP64 matrix. */
int oracle_dequant(int fmt, int scale_kind, int transposed,
                   const uint8_t *codes, const void *scales,
                   int64_t rows, int64_t K, double *out)
{
    orc_operand op = {fmt, scale_kind, transposed, codes, scales, rows, K};
    int64_t r;
    if (scale_kind == ORC_SCALE_MX && K % 32 != 0) return -1;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = orc_value(&op, r, k);
    return 0;
}

/* ---- dense GEMM: D = sum_k a(m,k) b(n,k) --------------------------------
 * A is [M,K]-logical, B is [N,K]-logical (each possibly stored transposed).
 * Dequantize both, then the textbook triple loop in FP64.  D is FP64 [M,N].
 * Scratch: caller passes workspace of (M+N)*K doubles.
 */
int oracle_gemm(int fmtA, int skA, int trA, const uint8_t *A, const void *sA,
                int fmtB, int skB, int trB, const uint8_t *B, const void *sB,
                int64_t M, int64_t N, int64_t K, double *work, double *D)
{
    double *a = work, *b = work + M * K;
    int64_t m;
    if (oracle_dequant(fmtA, skA, trA, A, sA, M, K, a)) return -1;
    if (oracle_dequant(fmtB, skB, trB, B, sB, N, K, b)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            const double *ar = a + m * K, *br = b + n * K;
            for (int64_t k = 0; k < K; ++k) acc += ar[k] * br[k];
            D[m * N + n] = acc;
        }
    }
    return 0;
}

/* Selected entries D[idx_m[i], idx_n[i]], each a direct sum over k with the
 * operands decoded on the fly.  For spot checks at sizes where the full
 * product is out of reach. */
int oracle_gemm_entries(int fmtA, int skA, int trA, const uint8_t *A, const void *sA,
                        int fmtB, int skB, int trB, const uint8_t *B, const void *sB,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t *idx_m, const int64_t *idx_n, int64_t count,
                        double *out)
{
    orc_operand a = {fmtA, skA, trA, A, sA, M, K};
    orc_operand b = {fmtB, skB, trB, B, sB, N, K};
    int64_t i;
    if ((skA == ORC_SCALE_MX || skB == ORC_SCALE_MX) && K % 32 != 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += orc_value(&a, idx_m[i], k) * orc_value(&b, idx_n[i], k);
        out[i] = acc;
    }
    return 0;
}

/* ---- grouped groupwise GEMM ---------------------------------------------
 * "Add FlyDSL grouped groupwise FP8 GEMM for ROCm" (PR body; commit on the
 * activation-scale layout):
 *   - G groups of rows, sizes m_sizes[g]; group g owns rows
 *     [start_g, start_g + m_sizes[g]) with start_g = sum_{h<g} m_sizes[h].
 *   - XQ is E4M3 [totM, K]; WQ is E4M3 [G, N, K] (plain row-major).
 *   - Activation scales: one FP32 per row per 128-K block, stored in the
 *     per-group block layout: group g's block begins at start_g * (K/128)
 *     and holds (local row i, k-block kb) at offset i + kb * m_sizes[g].
 *   - Weight scales: one FP32 per 128x128 block of W[g], stored
 *     [G, N/128, K/128] row-major (the pages give the granularity only).
 *   - N and K must be multiples of 128.
 * a(r,k) = dec(XQ[r,k]) * xs(r,k),  b_g(n,k) = dec(WQ[g,n,k]) * ws[g,n/128,k/128]
 * D[r,n] = sum_k a(r,k) * b_g(n,k) for r in group g.  Rows that belong to no
 * group are not written.
 */
static double orc_xs(const float *xs, int64_t start, int64_t mg, int64_t K,
                     int64_t local, int64_t kb)
{
    return (double)xs[start * (K / 128) + local + kb * mg];
}

int oracle_grouped_gemm(int G, const int64_t *m_sizes,
                        const uint8_t *XQ, const float *xs,
                        const uint8_t *WQ, const float *ws,
                        int64_t totM, int64_t N, int64_t K, double *D)
{
    int64_t start = 0;
    if (N % 128 != 0 || K % 128 != 0) return -1;
    for (int g = 0; g < G; ++g) {
        int64_t mg = m_sizes[g], i;
        if (mg < 0 || start + mg > totM) return -2;
        const uint8_t *W = WQ + (int64_t)g * N * K;
        const float *wsg = ws + (int64_t)g * (N / 128) * (K / 128);
#pragma omp parallel for schedule(dynamic, 1)
        for (i = 0; i < mg; ++i) {
            int64_t r = start + i;
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double av = oracle_decode_e4m3(XQ[r * K + k]) * orc_xs(xs, start, mg, K, i, k / 128);
                    double bv = oracle_decode_e4m3(W[n * K + k]) * (double)wsg[(n / 128) * (K / 128) + k / 128];
                    acc += av * bv;
                }
                D[r * N + n] = acc;
            }
        }
        start += mg;
    }
    return 0;
}

/* Selected entries of the grouped product.  Row r's group is found by
 * walking m_sizes; a row in no group yields NaN. */
int oracle_grouped_entries(int G, const int64_t *m_sizes,
                           const uint8_t *XQ, const float *xs,
                           const uint8_t *WQ, const float *ws,
                           int64_t totM, int64_t N, int64_t K,
                           const int64_t *idx_m, const int64_t *idx_n, int64_t count,
                           double *out)
{
    int64_t i;
    if (N % 128 != 0 || K % 128 != 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t r = idx_m[i], n = idx_n[i], start = 0, mg = 0;
        int g, found = -1;
        for (g = 0; g < G; ++g) {
            mg = m_sizes[g];
            if (r >= start && r < start + mg) { found = g; break; }
            start += mg;
        }
        if (found < 0 || r >= totM) { out[i] = NAN; continue; }
        const uint8_t *W = WQ + (int64_t)found * N * K;
        const float *wsg = ws + (int64_t)found * (N / 128) * (K / 128);
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double av = oracle_decode_e4m3(XQ[r * K + k]) * orc_xs(xs, start, mg, K, r - start, k / 128);
            double bv = oracle_decode_e4m3(W[n * K + k]) * (double)wsg[(n / 128) * (K / 128) + k / 128];
            acc += av * bv;
        }
        out[i] = acc;
    }
    return 0;
}

/* ---- BF16 round-to-nearest-even of an FP64 value ------------------------
 * BF16 keeps 8 significant bits (1 implicit + 7 stored), exponent range as
 * FP32.  Rounds the exact FP64 value once (no intermediate FP32 step).
 * Overflow goes to +-Inf; NaN maps to the canonical quiet NaN 0x7FC0.
 */
uint16_t oracle_bf16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    int e;
    if (isnan(x)) return 0x7FC0u;
    if (ax == 0.0) return sign;
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    frexp(ax, &e);                     /* ax = f * 2^e, f in [0.5, 1)      */
    /* unit in the last place of a BF16 number with this exponent: normal
     * numbers have 8 significant bits -> ulp = 2^(e-8); below 2^-126 the
     * spacing is fixed at 2^-133 (subnormal). */
    int ulp_exp = e - 8;
    if (ulp_exp < -133) ulp_exp = -133;
    double q = ldexp(ax, -ulp_exp);    /* exact scaling by a power of two   */
    double fl = floor(q), rem = q - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = ldexp(fl, ulp_exp);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    /* encode r (exactly representable in BF16) */
    {
        float f = (float)r;            /* exact: r has <= 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, 4);
        return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
    }
}

void oracle_bf16_rne_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(x[i]);
}

/* ---- quantizers: FP32 data -> codes + scales (the step before the GEMM) --
 *
 * "PyTorch on AMD GPUs gains a FlyDSL backend" (Interpretation): MX operands
 * carry one E8M0 power-of-two scale per 32 values along K.  "Add FlyDSL
 * grouped groupwise FP8 GEMM for ROCm" (PR body; commit messages): E4M3
 * activations with one FP32 scale per row and 128-value K block, stored in
 * the per-group block layout.  The pages give formats and granularities;
 * the scale rules are this project's readings:
 *   MX:        X = floor(log2(amax / fmt_max)) exactly (X = -127 for an
 *              all-zero block), clamped to [-127, 127]; scale code X + 127;
 *              element code = nearest(x / 2^X).
 *   groupwise: s = amax / 448 as an FP32 quotient (1.0 for an all-zero
 *              block); element code = nearest(FP32 quotient x / s).
 * nearest(v) is the format's representable value closest to v, ties to the
 * even code (mantissa LSB 0), saturating at +-fmt_max; the sign of v is kept
 * (a negative value that rounds to zero gives the negative-zero code).
 */

/* Largest positive finite code of each format; the positive codes 0..max
 * decode to strictly increasing values. */
static unsigned orc_max_code(int fmt)
{
    return fmt == ORC_E4M3 ? 0x7Eu : (fmt == ORC_E5M2 ? 0x7Bu : 0x7u);
}

static unsigned orc_nearest(int fmt, double v)
{
    const unsigned top = orc_max_code(fmt);
    const unsigned neg = signbit(v) ? 1u : 0u;
    const double a = fabs(v);
    unsigned c;
    if (a >= oracle_decode(fmt, top)) {
        c = top;
    } else {
        /* dec(lo) <= a < dec(hi), by bisection over the ordered codes */
        unsigned lo = 0u, hi = top;
        while (hi - lo > 1u) {
            const unsigned mid = (lo + hi) / 2u;
            if (oracle_decode(fmt, mid) <= a) lo = mid; else hi = mid;
        }
        const double dl = a - oracle_decode(fmt, lo), dh = oracle_decode(fmt, hi) - a;
        c = dl < dh ? lo : (dh < dl ? hi : ((lo & 1u) ? hi : lo));
    }
    if (neg) c |= (fmt == ORC_E2M1) ? 0x8u : 0x80u;
    return c;
}

unsigned oracle_nearest_code(int fmt, double v) { return orc_nearest(fmt, v); }

static double orc_fmt_max(int fmt)
{
    return oracle_decode(fmt, orc_max_code(fmt));
}

/* X = floor(log2(amax / fmt_max)), by exact comparisons in FP64. */
static int orc_e8m0_exponent(double amax, double fmt_max)
{
    if (!(amax > 0.0)) return -127;
    int X = ilogb(amax) - ilogb(fmt_max);
    while (ldexp(fmt_max, X) > amax) --X;
    while (ldexp(fmt_max, X + 1) <= amax) ++X;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    return X;
}

/* x: FP32 [rows, K] row-major, K % 32 == 0.  codes: [rows, K] bytes (E4M3,
 * E5M2) or [rows, K/2] (E2M1, element 2j in the low nibble); scales: E8M0
 * [rows, K/32]. */
int oracle_quant_mx(int fmt, const float *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales)
{
    if (K % 32 != 0 || (fmt != ORC_E4M3 && fmt != ORC_E5M2 && fmt != ORC_E2M1)) return -1;
    const double fmax = orc_fmt_max(fmt);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const float *blk = x + r * K + 32 * b;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) if (fabs((double)blk[j]) > amax) amax = fabs((double)blk[j]);
            const int X = orc_e8m0_exponent(amax, fmax);
            scales[r * (K / 32) + b] = (uint8_t)(X + 127);
            for (int j = 0; j < 32; ++j) {
                const unsigned c = orc_nearest(fmt, ldexp((double)blk[j], -X));
                const int64_t k = 32 * b + j;
                if (fmt == ORC_E2M1) {
                    uint8_t *p = codes + r * (K / 2) + k / 2;
                    if (k % 2 == 0) *p = (uint8_t)((*p & 0xF0u) | c);
                    else *p = (uint8_t)((*p & 0x0Fu) | (c << 4));
                } else {
                    codes[r * K + k] = (uint8_t)c;
                }
            }
        }
    }
    return 0;
}

/* Groupwise E4M3 activations: x FP32 [totM, K], K % 128 == 0; group g owns
 * rows [start_g, start_g + m_sizes[g]).  codes: [totM, K]; xs: FP32 scale of
 * (row r of group g, k block kb) at start_g*(K/128) + (r - start_g) +
 * kb*m_sizes[g] ("Add FlyDSL grouped groupwise FP8 GEMM for ROCm", commit
 * fixing the activation-scale addressing).  Rows in no group are not
 * written. */
int oracle_quant_group_act(int G, const int64_t *m_sizes, const float *x, int64_t totM, int64_t K,
                           uint8_t *codes, float *xs)
{
    if (K % 128 != 0) return -1;
    const int64_t nkb = K / 128;
    int64_t start = 0;
    for (int g = 0; g < G; ++g) {
        int64_t mg = m_sizes[g] < 0 ? 0 : m_sizes[g];
        if (mg > totM - start) mg = totM - start;
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < mg; ++i) {
            const int64_t r = start + i;
            for (int64_t kb = 0; kb < nkb; ++kb) {
                const float *blk = x + r * K + 128 * kb;
                float amax = 0.0f;
                for (int j = 0; j < 128; ++j) if (fabsf(blk[j]) > amax) amax = fabsf(blk[j]);
                volatile float s = amax / 448.0f;          /* FP32 quotient */
                const float sc = amax > 0.0f ? s : 1.0f;
                xs[start * nkb + i + kb * mg] = sc;
                for (int j = 0; j < 128; ++j) {
                    volatile float q = blk[j] / sc;         /* FP32 quotient */
                    codes[r * K + 128 * kb + j] = (uint8_t)orc_nearest(ORC_E4M3, (double)q);
                }
            }
        }
        start += mg;
    }
    return 0;
}

/* Tensor-wise FP8 (E4M3 or E5M2): one FP32 dequant scale for the whole
 * tensor ("Experimental FlyDSL GEMM backend for TE PyTorch", Supported Data
 * Types: tensor-wise FP8 with delayed scaling), taken from the current
 * tensor: s = amax / fmt_max as an FP32 quotient (1.0 for an all-zero
 * tensor), element code = nearest(FP32 quotient x / s), the same rule as the
 * groupwise quantizers with the whole tensor as one block.  x: n FP32
 * values; codes: n bytes. */
int oracle_quant_tensor(int fmt, const float *x, int64_t n, uint8_t *codes, float *s_out)
{
    if (fmt != ORC_E4M3 && fmt != ORC_E5M2) return -1;
    const float fmax = (float)orc_fmt_max(fmt);
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    volatile float s = amax / fmax;                     /* FP32 quotient */
    const float sc = amax > 0.0f ? s : 1.0f;
    *s_out = sc;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        volatile float q = x[i] / sc;                   /* FP32 quotient */
        codes[i] = (uint8_t)orc_nearest(fmt, (double)q);
    }
    return 0;
}

/* Groupwise E4M3 weights: w FP32 [G, N, K], N % 128 == 0, K % 128 == 0; one
 * FP32 scale per 128 x 128 block, ws [G, N/128, K/128] row-major ("Add
 * FlyDSL grouped groupwise FP8 GEMM for ROCm", PR body: 128x128 weight
 * blocks), with the same rule as the activations: s = amax / 448 as an FP32
 * quotient (1.0 for an all-zero block), element code = nearest(FP32
 * quotient w / s). */
int oracle_quant_group_weight(int G, const float *w, int64_t N, int64_t K, uint8_t *codes, float *ws)
{
    if (N % 128 != 0 || K % 128 != 0) return -1;
    const int64_t nb = N / 128, kb = K / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < (int64_t)G * nb * kb; ++blk) {
        const int64_t g = blk / (nb * kb), bn = (blk / kb) % nb, bk = blk % kb;
        const float *base = w + (g * N + bn * 128) * K + bk * 128;
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i)
            for (int j = 0; j < 128; ++j)
                if (fabsf(base[i * K + j]) > amax) amax = fabsf(base[i * K + j]);
        volatile float s = amax / 448.0f;              /* FP32 quotient */
        const float sc = amax > 0.0f ? s : 1.0f;
        ws[blk] = sc;
        uint8_t *out = codes + (g * N + bn * 128) * K + bk * 128;
        for (int i = 0; i < 128; ++i)
            for (int j = 0; j < 128; ++j) {
                volatile float q = base[i * K + j] / sc;   /* FP32 quotient */
                out[i * K + j] = (uint8_t)orc_nearest(ORC_E4M3, (double)q);
            }
    }
    return 0;
}

/* ---- epilogue: bias and activation ---------------------------------------
 *
 * "[gfx1250] Add MXFP4 GEMM support to FlyDSL backend" (Description): the
 * GEMM's activation and bias are the follow-up to the plain product.  The
 * pages name no function, so this project reads it as the fused epilogue of
 * a linear layer's forward GEMM:
 *     D[m,n] = act( sum_k a(m,k) b(n,k) + bias[n] )
 * with bias a BF16 vector over N (NULL: none) and act one of
 *     0 none, 1 ReLU max(z, 0),
 *     2 GELU, tanh form: z/2 (1 + tanh( sqrt(2/pi) (z + 0.044715 z^3) )),
 *     3 SiLU z / (1 + e^-z),
 * all in FP64 on the FP64 sum, rounded once to BF16 by the caller.  D is
 * [M, N] row-major, updated in place. */
#define ORC_ACT_NONE 0
#define ORC_ACT_RELU 1
#define ORC_ACT_GELU_TANH 2
#define ORC_ACT_SILU 3

static double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double oracle_activation(int act, double z)
{
    switch (act) {
    case ORC_ACT_NONE: return z;
    case ORC_ACT_RELU: return z > 0.0 ? z : 0.0;
    case ORC_ACT_GELU_TANH: {
        const double c = sqrt(2.0 / 3.14159265358979323846);
        return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
    }
    case ORC_ACT_SILU: return z / (1.0 + exp(-z));
    default: return NAN;
    }
}

int oracle_epilogue(double *D, int64_t M, int64_t N, const uint16_t *bias, int act)
{
    int64_t m;
    if (act < ORC_ACT_NONE || act > ORC_ACT_SILU) return -1;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double z = D[m * N + n];
            if (bias) z += orc_bf16_value(bias[n]);
            D[m * N + n] = oracle_activation(act, z);
        }
    return 0;
}

/* ---- BF16 grouped GEMM ---------------------------------------------------
 *
 * "PyTorch on AMD GPUs gains a FlyDSL backend" (Interpretation; the BF16
 * grouped-GEMM cases of its operator suite): a grouped GEMM over expert
 * groups of rows that tolerates uneven and empty groups, here with BF16
 * operands ("Experimental FlyDSL GEMM backend for TE PyTorch", Supported
 * Data Types, names BF16 among the GEMM input types).  For each group g of
 * rows [start_g, start_g + m_g):
 *
 *     D[r, n] = sum_k x(r, k) * w(g, n, k)
 *
 * with x and w the BF16 values, no scales.  Same layout conventions as the
 * FP8 grouped GEMM above: X [totM, K], W [G, N, K], both K-contiguous.
 */

/* BF16 from its closed form: sign, 8-bit exponent with bias 127, 7-bit
 * fraction; exponent 0 is zero or subnormal (f * 2^-133), exponent 255 is
 * Inf (f = 0) or NaN. */
double oracle_decode_bf16(unsigned bits)
{
    const int s = (bits >> 15) & 1, e = (bits >> 7) & 0xFF, f = bits & 0x7F;
    double v;
    if (e == 0xFF) v = f ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)f, -133);
    else v = ldexp(1.0 + f / 128.0, e - 127);
    return s ? -v : v;
}

int oracle_grouped_gemm_bf16(int G, const int64_t *m_sizes, const uint16_t *X, const uint16_t *W,
                             int64_t totM, int64_t N, int64_t K, double *D)
{
    int64_t start = 0;
    for (int g = 0; g < G; ++g) {
        int64_t mg = m_sizes[g], i;
        if (mg < 0 || start + mg > totM) return -2;
        const uint16_t *Wg = W + (int64_t)g * N * K;
#pragma omp parallel for schedule(dynamic, 1)
        for (i = 0; i < mg; ++i) {
            int64_t r = start + i;
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += oracle_decode_bf16(X[r * K + k]) * oracle_decode_bf16(Wg[n * K + k]);
                D[r * N + n] = acc;
            }
        }
        start += mg;
    }
    return 0;
}

/* Selected entries; a row in no group yields NaN. */
int oracle_grouped_entries_bf16(int G, const int64_t *m_sizes, const uint16_t *X, const uint16_t *W,
                                int64_t totM, int64_t N, int64_t K,
                                const int64_t *idx_m, const int64_t *idx_n, int64_t count, double *out)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t r = idx_m[i], n = idx_n[i], start = 0;
        int g, found = -1;
        for (g = 0; g < G; ++g) {
            if (r >= start && r < start + m_sizes[g]) { found = g; break; }
            start += m_sizes[g];
        }
        if (found < 0 || r >= totM) { out[i] = NAN; continue; }
        const uint16_t *Wg = W + (int64_t)found * N * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_decode_bf16(X[r * K + k]) * oracle_decode_bf16(Wg[n * K + k]);
        out[i] = acc;
    }
    return 0;
}
