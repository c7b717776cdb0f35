"""Shared helpers for the GPU parity tests: build seeded inputs with the
input generator, run the HIP library through its C ABI binding, and compare
with the CPU oracle."""
import numpy as np
import torch

import oracle
from block_scaled_precision_03_amd import synth

# library format code -> (oracle element fmt, oracle scale kind, synth elem name)
LIB2ORC = {
    0: (oracle.E4M3, oracle.SCALE_MX, "e4m3"),
    1: (oracle.E5M2, oracle.SCALE_MX, "e5m2"),
    4: (oracle.E2M1, oracle.SCALE_MX, "e2m1"),
    16: (oracle.E4M3, oracle.SCALE_TENSOR, "e4m3"),
    17: (oracle.E5M2, oracle.SCALE_TENSOR, "e5m2"),
}

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_to_f64(t):
    """Device bf16 tensor (or uint16 bits) -> host float64 numpy."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    bits = t.cpu().numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(bits)


def bits(t):
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def empty_d(M, N, fill=None):
    d = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    if fill is not None:
        d.fill_(fill)
    return d


class Operand:
    """One GEMM operand: codes as stored (layout applied), scales, and what
    the oracle needs."""

    def __init__(self, lib_fmt, codes, scales, transposed, rows, K):
        self.lib_fmt = lib_fmt
        self.codes = codes
        self.scales = scales
        self.transposed = transposed
        self.rows = rows
        self.K = K

    def orc(self):
        f, sk, _ = LIB2ORC[self.lib_fmt]
        return (f, sk, self.transposed, self.codes, self.scales)

    def dev_codes(self):
        return dev(self.codes)

    def dev_scales(self):
        if LIB2ORC[self.lib_fmt][1] == oracle.SCALE_TENSOR:
            return dev(np.array([self.scales], dtype=np.float32))
        return dev(self.scales)


def make_operand(lib_fmt, x, transposed):
    """x: FP32 logical [rows, K].  Quantize per the format's recipe and store
    K-contiguous (transposed=False) or rows-contiguous (transposed=True)."""
    rows, K = x.shape
    _, sk, elem = LIB2ORC[lib_fmt]
    if sk == oracle.SCALE_MX:
        codes, s = synth.quant_mx(x, elem)
    else:
        codes, s = synth.quant_tensor(x, elem)
    if transposed:
        if elem == "e2m1":
            codes = synth.transpose_e2m1(codes)
        else:
            codes = np.ascontiguousarray(codes.T)
    return Operand(lib_fmt, codes, s, transposed, rows, K)


def unpack_e2m1(packed):
    """Packed E2M1 codes (two per byte along the last axis, even index in
    the low nibble) -> one nibble code per byte."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def k_contiguous(op):
    """The same logical operand stored K-contiguous (codes and scales)."""
    if not op.transposed:
        return op
    if op.lib_fmt == 4:
        codes = synth.pack_e2m1(np.ascontiguousarray(unpack_e2m1(op.codes).T))
    else:
        codes = np.ascontiguousarray(op.codes.T)
    return Operand(op.lib_fmt, codes, op.scales, False, op.rows, op.K)


def run_dense(layout, opA, opB, M, N, K, preshuffle_b=False, d_fill=None):
    from block_scaled_precision_03_amd import mxgemm
    A, sA = opA.dev_codes(), opA.dev_scales()
    B, sB = opB.dev_codes(), opB.dev_scales()
    fmtB = opB.lib_fmt
    if preshuffle_b:
        blayout = mxgemm.NN if opB.transposed else mxgemm.NT
        Bp = torch.empty(mxgemm.preshuffle_b_bytes(fmtB, N, K), dtype=torch.uint8, device=DEV)
        mxgemm.preshuffle_b(fmtB, blayout, B, Bp, N, K)
        B = Bp
        if LIB2ORC[fmtB][1] == oracle.SCALE_MX:
            sBp = torch.empty(mxgemm.preshuffle_scales_bytes(N, K), dtype=torch.uint8, device=DEV)
            mxgemm.preshuffle_scales(sB, sBp, N, K)
            sB = sBp
        fmtB |= mxgemm.PRESHUFFLED
        layout = mxgemm.NT if layout == mxgemm.NN else layout
    D = empty_d(M, N, d_fill)
    mxgemm.run(opA.lib_fmt, fmtB, layout, A, sA, B, sB, D, M, N, K)
    torch.cuda.synchronize()
    return D


def assert_close(d, ref, what=""):
    ok, worst = oracle.within_tolerance(d, ref)
    if not ok:
        err = np.abs(d - ref)
        idx = np.unravel_index(np.argmax(err / (2.0 ** -7 * np.abs(ref) + 1e-3 * np.abs(ref).max() + 1e-300)), err.shape)
        raise AssertionError("%s: outside tolerance (worst ratio %.3g) at %s: got %r ref %r"
                             % (what, worst, idx, d[idx], ref[idx]))
    return worst


def sample_indices(rng, M, N, count):
    """Random (m, n) pairs plus the four corners and the last row/column."""
    im = list(rng.integers(0, M, count))
    inn = list(rng.integers(0, N, count))
    for m, n in [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]:
        im.append(m)
        inn.append(n)
    for n in rng.integers(0, N, 64):
        im.append(M - 1)
        inn.append(n)
    for m in rng.integers(0, M, 64):
        im.append(m)
        inn.append(N - 1)
    return np.array(im, np.int64), np.array(inn, np.int64)


def int_operand(rng, fmt, rows, K, transposed=False, mx=True):
    """Codes of small integers {-2..2} and power-of-two scales 1, 2 or 4
    (tensor-wise: s = 2).  With such inputs every partial sum of a GEMM is an
    integer far below 2^24, exact in FP32 in any order, so a kernel's BF16
    output must equal the oracle's exact result rounded once, bit for bit.
    A transposed E2M1 operand [K, rows] is packed two rows per byte."""
    table = {0: [0xC0, 0xB8, 0x00, 0x38, 0x40], 1: [0xC0, 0xBC, 0x00, 0x3C, 0x40],
             4: [0xC, 0xA, 0x0, 0x2, 0x4]}
    base = 0 if fmt in (0, 16) else (1 if fmt in (1, 17) else 4)
    codes = np.array(table[base], np.uint8)[rng.integers(0, 5, (rows, K))]
    if transposed:
        codes = np.ascontiguousarray(codes.T)
    if base == 4:
        codes = synth.pack_e2m1(codes)
    if mx:
        s = rng.integers(127, 130, (rows, K // 32)).astype(np.uint8)
    else:
        s = np.float32(2.0)
    return Operand(fmt, codes, s, transposed, rows, K)
