"""Pins of the oracle's dense GEMM (CPU only).

The oracle computes D = sum_k a(m,k) b(n,k) from codes and scales.  It is
checked against things that do not share its code:
* exact rational arithmetic (Python Fractions) on tiny shapes, decoding with
  torch's float8 views (independent of the oracle's decoders);
* a library matmul (numpy float64) of independently dequantized operands;
* one-hot and identity inputs, exact scale doubling, layout equivalences.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_03_amd import synth

TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
FMAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0, oracle.E2M1: 6.0}


def _indep_decode(fmt, codes):
    """Decode with torch (fp8) or the E2M1->E4M3 embedding (fp4)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt in TORCH_DT:
        return torch.from_numpy(codes.copy()).view(TORCH_DT[fmt]).to(torch.float64).numpy()
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    out = np.empty(codes.shape)
    for idx, nib in np.ndenumerate(codes):
        s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
        code = (0x30 if m else 0) if e == 0 else ((e + 6) << 3) | (m << 2)
        out[idx] = -t[code] if s else t[code]
    return out


def _unpack_rows(packed, rows, K):
    """Packed E2M1 [rows, K/2] -> nibble codes [rows, K] (even k = low nibble)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(rows, K // 2)
    out = np.empty((rows, K), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def _rand_codes(rng, fmt, shape):
    """Random finite codes (no NaN/Inf)."""
    if fmt == oracle.E2M1:
        return rng.integers(0, 16, shape).astype(np.uint8)
    c = rng.integers(0, 256, shape).astype(np.uint8)
    v = _indep_decode(fmt, c)
    c[~np.isfinite(v)] = 0x38 if fmt == oracle.E4M3 else 0x3C
    return c


def _make_operand(rng, fmt, sk, rows, K, transposed, escale=(120, 134)):
    """Returns (oracle operand tuple, independent FP64 dequantized [rows, K])."""
    nib = _rand_codes(rng, fmt, (rows, K))
    vals = _indep_decode(fmt, nib)
    if sk == oracle.SCALE_MX:
        s = rng.integers(escale[0], escale[1] + 1, (rows, K // 32)).astype(np.uint8)
        mult = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    else:
        s = np.float32(rng.uniform(0.01, 3.0))
        mult = float(s)
    deq = vals * mult
    stored = nib.T.copy() if transposed else nib
    if fmt == oracle.E2M1:
        stored = synth.pack_e2m1(stored)
    return (fmt, sk, transposed, stored, s), deq


CASES = []
for fa, fb in [(oracle.E4M3, oracle.E4M3), (oracle.E4M3, oracle.E5M2), (oracle.E5M2, oracle.E4M3),
               (oracle.E5M2, oracle.E5M2), (oracle.E2M1, oracle.E2M1)]:
    for sk in (oracle.SCALE_MX, oracle.SCALE_TENSOR):
        if fa == oracle.E2M1 and sk == oracle.SCALE_TENSOR:
            continue
        for ta, tb in [(0, 0), (0, 1), (1, 1)]:     # NT, NN, TN in row-major naming
            # a transposed E2M1 operand [K, rows] packs two rows per byte
            # along its contiguous dimension (row 2j in the low nibble)
            CASES.append((fa, fb, sk, ta, tb))


@pytest.mark.parametrize("fa,fb,sk,ta,tb", CASES)
@pytest.mark.parametrize("K", [32, 128, 256])
def test_exact_rational_brute_force(fa, fb, sk, ta, tb, K):
    rng = np.random.default_rng(hash((fa, fb, sk, ta, tb, K)) % (2 ** 32))
    M, N = (4, 6) if fa == oracle.E2M1 and ta else (3, 4)
    opA, a = _make_operand(rng, fa, sk, M, K, ta)
    opB, b = _make_operand(rng, fb, sk, N, K, tb)
    D = oracle.gemm(opA, opB, M, N, K)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(a[m, k]) * Fraction(b[n, k]) for k in range(K)), Fraction(0))
            bound = K * 2.0 ** -52 * float(sum(abs(Fraction(a[m, k]) * Fraction(b[n, k])) for k in range(K)))
            assert abs(Fraction(D[m, n]) - exact) <= Fraction(bound), (m, n)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E2M1])
def test_exact_when_representable(fmt):
    """Neutral scales: every partial sum is exact in FP64, so the oracle must
    equal the rational sum exactly."""
    rng = np.random.default_rng(3)
    M, N, K = 4, 4, 256
    lo = hi = 127
    opA, a = _make_operand(rng, fmt, oracle.SCALE_MX, M, K, 0, (lo, hi))
    opB, b = _make_operand(rng, fmt, oracle.SCALE_MX, N, K, 0, (lo, hi))
    D = oracle.gemm(opA, opB, M, N, K)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(a[m, k]) * Fraction(b[n, k]) for k in range(K)), Fraction(0))
            assert Fraction(D[m, n]) == exact


@pytest.mark.parametrize("fa,fb,sk,ta,tb", CASES)
def test_matches_numpy_matmul(fa, fb, sk, ta, tb):
    rng = np.random.default_rng(11)
    M, N, K = 37, 29, 192
    if fa == oracle.E2M1:
        M, N = M + ta, N + tb          # even row counts when packed along rows
    opA, a = _make_operand(rng, fa, sk, M, K, ta)
    opB, b = _make_operand(rng, fb, sk, N, K, tb)
    D = oracle.gemm(opA, opB, M, N, K)
    ref = a @ b.T
    scale = np.abs(a) @ np.abs(b).T
    assert np.all(np.abs(D - ref) <= 1e-13 * scale + 1e-300)


def test_entries_match_full():
    rng = np.random.default_rng(5)
    M, N, K = 40, 33, 256
    opA, _ = _make_operand(rng, oracle.E4M3, oracle.SCALE_MX, M, K, 0)
    opB, _ = _make_operand(rng, oracle.E5M2, oracle.SCALE_MX, N, K, 1)
    D = oracle.gemm(opA, opB, M, N, K)
    im = rng.integers(0, M, 100)
    inn = rng.integers(0, N, 100)
    e = oracle.gemm_entries(opA, opB, M, N, K, im, inn)
    assert np.array_equal(e, D[im, inn])


def test_one_hot():
    M, N, K = 8, 8, 128
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[3, 77] = 0x48        # E4M3 4.0
    B[5, 77] = 0xB0        # E4M3 -0.5
    sA = np.full((M, K // 32), 127, np.uint8)
    sB = np.full((N, K // 32), 127, np.uint8)
    sA[3, 2] = 130         # x8 on block 2 (k 64..95) of row 3
    D = oracle.gemm((oracle.E4M3, 0, 0, A, sA), (oracle.E4M3, 0, 0, B, sB), M, N, K)
    expect = np.zeros((M, N))
    expect[3, 5] = 4.0 * 8.0 * -0.5
    assert np.array_equal(D, expect)


def test_identity_gives_B_transposed():
    rng = np.random.default_rng(9)
    K = 64
    N = 24
    A = np.zeros((K, K), np.uint8)
    np.fill_diagonal(A, 0x38)                      # 1.0
    sA = np.full((K, K // 32), 127, np.uint8)
    opB, b = _make_operand(rng, oracle.E4M3, oracle.SCALE_MX, N, K, 0)
    D = oracle.gemm((oracle.E4M3, 0, 0, A, sA), opB, K, N, K)
    assert np.array_equal(D, b.T)


def test_scale_doubling_exact():
    rng = np.random.default_rng(13)
    M, N, K = 16, 12, 256
    opA, _ = _make_operand(rng, oracle.E4M3, oracle.SCALE_MX, M, K, 0)
    opB, _ = _make_operand(rng, oracle.E4M3, oracle.SCALE_MX, N, K, 0)
    D = oracle.gemm(opA, opB, M, N, K)
    sA2 = opA[4] + 1
    D2 = oracle.gemm(opA[:4] + (sA2,), opB, M, N, K)
    assert np.array_equal(D2, 2 * D)
    # doubling a single 32-K block of one row doubles exactly that block's share
    sA3 = opA[4].copy()
    sA3[7, 3] += 1
    D3 = oracle.gemm(opA[:4] + (sA3,), opB, M, N, K)
    codes = opA[3].copy()
    keep = np.zeros_like(codes)
    keep[7, 96:128] = codes[7, 96:128]
    part = oracle.gemm((opA[0], opA[1], 0, keep, opA[4]), opB, M, N, K)
    assert np.allclose(D3[7], D[7] + part[7], rtol=0, atol=1e-13 * np.abs(D).max())
    mask = np.ones(M, bool)
    mask[7] = False
    assert np.array_equal(D3[mask], D[mask])


def test_tensor_scale_doubling_exact():
    rng = np.random.default_rng(17)
    M, N, K = 9, 7, 128
    opA, _ = _make_operand(rng, oracle.E4M3, oracle.SCALE_TENSOR, M, K, 0)
    opB, _ = _make_operand(rng, oracle.E5M2, oracle.SCALE_TENSOR, N, K, 0)
    D = oracle.gemm(opA, opB, M, N, K)
    D2 = oracle.gemm(opA[:4] + (np.float32(opA[4] * 2),), opB, M, N, K)
    assert np.array_equal(D2, 2 * D)


def test_mx_neutral_equals_tensor_unit():
    rng = np.random.default_rng(19)
    M, N, K = 20, 18, 128
    A = _rand_codes(rng, oracle.E4M3, (M, K))
    B = _rand_codes(rng, oracle.E5M2, (N, K))
    s127a = np.full((M, K // 32), 127, np.uint8)
    s127b = np.full((N, K // 32), 127, np.uint8)
    D1 = oracle.gemm((oracle.E4M3, 0, 0, A, s127a), (oracle.E5M2, 0, 0, B, s127b), M, N, K)
    D2 = oracle.gemm((oracle.E4M3, 1, 0, A, np.float32(1)), (oracle.E5M2, 1, 0, B, np.float32(1)), M, N, K)
    assert np.array_equal(D1, D2)


def test_layouts_equivalent():
    """NN with the transposed copy of B, and TN with transposed copies of
    both, reproduce NT exactly (same values, same k order)."""
    rng = np.random.default_rng(23)
    M, N, K = 24, 40, 96
    A = _rand_codes(rng, oracle.E4M3, (M, K))
    B = _rand_codes(rng, oracle.E4M3, (N, K))
    sA = np.float32(0.75)
    sB = np.float32(1.5)
    nt = oracle.gemm((0, 1, 0, A, sA), (0, 1, 0, B, sB), M, N, K)
    nn = oracle.gemm((0, 1, 0, A, sA), (0, 1, 1, B.T.copy(), sB), M, N, K)
    tn = oracle.gemm((0, 1, 1, A.T.copy(), sA), (0, 1, 1, B.T.copy(), sB), M, N, K)
    assert np.array_equal(nt, nn) and np.array_equal(nt, tn)


def test_fp4_transposed_nibble_order():
    """A transposed E2M1 operand [K, rows] packs rows 2j (low nibble) and
    2j + 1 (high nibble) of one k in a byte: A^T[0, 0] = 0x72 puts 1.0 in
    row 0 and 6.0 in row 1 at k = 0; B = 1.0 at k = 0 gives D = [1, 6]^T.
    With A^T[1, 0] = 0x40 (code 4 = 2.0 in row 1 at k = 1) and B = 1.0 at
    k = 1 as well, row 1 becomes 6 + 2 = 8."""
    K = 32
    s1 = np.full((2, K // 32), 127, np.uint8)
    sb = np.full((1, K // 32), 127, np.uint8)
    At = np.zeros((K, 1), np.uint8)
    At[0, 0] = 0x72
    B = np.zeros((1, K // 2), np.uint8)
    B[0, 0] = 0x02
    D = oracle.gemm((oracle.E2M1, 0, 1, At, s1), (oracle.E2M1, 0, 0, B, sb), 2, 1, K)
    assert D.tolist() == [[1.0], [6.0]]
    At[1, 0] = 0x40
    B[0, 0] = 0x22
    D = oracle.gemm((oracle.E2M1, 0, 1, At, s1), (oracle.E2M1, 0, 0, B, sb), 2, 1, K)
    assert D.tolist() == [[1.0], [8.0]]
    # the same operand stored K-contiguous, packed along k, gives the same D
    A = np.zeros((2, K // 2), np.uint8)
    A[0, 0] = 0x02                                  # row 0: 1.0 at k = 0
    A[1, 0] = 0x47                                  # row 1: 6.0 at k = 0, 2.0 at k = 1
    D2 = oracle.gemm((oracle.E2M1, 0, 0, A, s1), (oracle.E2M1, 0, 0, B, sb), 2, 1, K)
    assert np.array_equal(D, D2)


def test_fp4_nibble_order():
    """Even k sits in the low nibble: A = [1.0 at k=0, 6.0 at k=1] packed as
    0x72; B row 0 has 1.0 at k=0 only, B row 1 has 1.0 at k=1 only."""
    K = 32
    A = np.zeros((1, K // 2), np.uint8)
    A[0, 0] = 0x72                                  # low: code 2 (1.0), high: code 7 (6.0)
    B = np.zeros((2, K // 2), np.uint8)
    B[0, 0] = 0x02
    B[1, 0] = 0x20
    s1 = np.full((1, 1), 127, np.uint8)
    s2 = np.full((2, 1), 127, np.uint8)
    D = oracle.gemm((oracle.E2M1, 0, 0, A, s1), (oracle.E2M1, 0, 0, B, s2), 1, 2, K)
    assert D[0, 0] == 1.0 and D[0, 1] == 6.0


def test_quantized_inputs_round_trip():
    """The seeded recipe's codes and scales dequantize (by the oracle) to the
    FP32 data within half an E4M3 step, except elements at or above the
    block's saturation point, which land exactly on +-448 * scale."""
    x = synth.normal(1, (8, 256))
    codes, s = synth.quant_mx(x, "e4m3")
    deq = oracle.dequant(oracle.E4M3, oracle.SCALE_MX, 0, codes, s, 8, 256)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    y = np.abs(x) / scale
    sat = y >= 464                      # beyond the last rounding midpoint
    assert np.all(np.abs(deq[sat]) == 448 * scale[sat])
    ok = ~sat
    assert np.all(np.abs(deq[ok] - x[ok]) <= np.maximum(np.abs(x[ok]) * 2.0 ** -4, 2.0 ** -10 * scale[ok]))
    # every block's largest element saturates under the floor(log2(amax/448)) rule
    assert np.all(np.abs(deq).reshape(8, 8, 32).max(-1) == 448 * scale.reshape(8, 8, 32)[..., 0])
