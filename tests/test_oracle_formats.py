"""Pins of the oracle's element decoders and BF16 rounding (CPU only).

Each decoder is checked against (a) an independent library decoder (torch's
CPU float8 views), (b) the OCP reference values in tests/golden, and (c)
closed-form invariants (counts of NaN/Inf, extremes, monotonicity).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMT = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2, "e2m1": oracle.E2M1}


def _torch_decode(dtype):
    return torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


@pytest.mark.parametrize("name,dtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_all_codes_match_torch(name, dtype):
    ours = oracle.decode(FMT[name], np.arange(256))
    assert _same(ours, _torch_decode(dtype))


def test_e8m0_all_codes_match_torch():
    ours = oracle.decode_e8m0(np.arange(256))
    ref = _torch_decode(torch.float8_e8m0fnu)
    assert _same(ours, ref)


def test_e2m1_matches_e4m3_embedding():
    """Every E2M1 value is an E4M3 value: exponent e -> e+6 (bias 1 vs 7),
    mantissa bit m -> m<<2; the subnormal 0.5 is the E4M3 code 0x30.  Decode
    the embedded codes with torch's E4M3 view and compare."""
    t = _torch_decode(torch.float8_e4m3fn)
    for nib in range(16):
        s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
        if e == 0:
            code = 0x30 if m else 0x00
        else:
            code = ((e + 6) << 3) | (m << 2)
        ref = t[code] * (-1.0 if s else 1.0)
        got = oracle.decode(oracle.E2M1, [nib])[0]
        assert got == ref and (np.signbit(got) == (s == 1)), nib


def _parse(v):
    if v == "nan":
        return math.nan
    if v in ("inf", "-inf"):
        return float(v)
    if "^" in v:
        b, e = v.split("^")
        return float(int(b)) ** int(e)
    return float(v)


def test_golden_format_values():
    n = 0
    with open(os.path.join(GOLDEN, "ocp_format_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, code, val = line.split()
            c = int(code, 16)
            got = oracle.decode_e8m0([c])[0] if fmt == "e8m0" else oracle.decode(FMT[fmt], [c])[0]
            exp = _parse(val)
            if math.isnan(exp):
                assert math.isnan(got), line
            else:
                assert got == exp and math.copysign(1, got) == math.copysign(1, exp), line
            n += 1
    assert n >= 30


@pytest.mark.parametrize("name,nan,inf,vmax,vmin_sub", [
    ("e4m3", 2, 0, 448.0, 2.0 ** -9),
    ("e5m2", 6, 2, 57344.0, 2.0 ** -16),
])
def test_fp8_invariants(name, nan, inf, vmax, vmin_sub):
    v = oracle.decode(FMT[name], np.arange(256))
    assert int(np.isnan(v).sum()) == nan
    assert int(np.isinf(v).sum()) == inf
    fin = v[np.isfinite(v)]
    assert fin.max() == vmax and fin.min() == -vmax
    assert fin[fin > 0].min() == vmin_sub
    # positive codes 0x00..0x7f are strictly increasing over finite values
    pos = v[:128]
    pos = pos[np.isfinite(pos)]
    assert np.all(np.diff(pos) > 0)
    # sign symmetry: code ^ 0x80 negates
    neg = v[128:]
    ok = np.isnan(v[:128]) & np.isnan(neg) | (neg == -v[:128])
    assert np.all(ok)


def test_e2m1_grid():
    v = oracle.decode(oracle.E2M1, np.arange(16))
    assert list(v[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(v[8:]) == [-x for x in v[:8]]


def test_e8m0_is_power_of_two():
    v = oracle.decode_e8m0(np.arange(255))
    for c, x in enumerate(v):
        assert x == math.ldexp(1.0, c - 127)


def _bf16_values_near(x):
    """All BF16 values bracketing x (from float32 bit patterns)."""
    f = np.float32(x)
    u = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) & 0xFFFF0000
    cands = []
    for du in (-0x10000, 0, 0x10000, 0x20000):
        w = (u + du) & 0xFFFFFFFF
        cands.append(float(np.array([w], dtype=np.uint32).view(np.float32)[0]))
    return cands


def test_bf16_rne_brute_force():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000)))
    # exact ties and near-ties: midpoints between adjacent bf16 values
    for k in range(200):
        base = float(np.float32(1.0 + k / 128.0))
        xs += [base + 2.0 ** -8, base - 2.0 ** -8, base + 2.0 ** -8 + 2.0 ** -40]
    for x in xs:
        bits = oracle.bf16_rne(np.array([x]))[0]
        got = oracle.bf16_bits_to_f64([bits])[0]
        cands = [c for c in _bf16_values_near(x) if np.isfinite(c)]
        fx = Fraction(x)
        best = min(abs(Fraction(c) - fx) for c in cands)
        near = [c for c in cands if abs(Fraction(c) - fx) == best]
        if len(near) > 1:  # tie: even last mantissa bit
            near = [c for c in near
                    if (int(np.array([c], np.float32).view(np.uint32)[0]) >> 16) & 1 == 0]
        assert got == near[0], (x, got, near)


def test_bf16_rne_specials():
    b = oracle.bf16_rne(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.5e38, 1.0]))
    assert list(b[:4]) == [0x0000, 0x8000, 0x7F80, 0xFF80]
    assert b[4] == 0x7FC0 and b[5] == 0x7F80 and b[6] == 0x3F80
