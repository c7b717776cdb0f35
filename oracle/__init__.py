"""Python handle on the FP64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.  It shares no code
with the GPU path; it receives the same seeded codes and scales and returns
FP64 results of the plain definition D[m,n] = sum_k a(m,k) b(n,k).

Format selectors (the oracle's own numbering): ``E4M3=0, E5M2=1, E2M1=4``;
scale kinds ``SCALE_MX=0`` (E8M0 per 32 K values, stored [rows, K/32]) and
``SCALE_TENSOR=1`` (one FP32 multiplier).
"""
import ctypes
import os

import numpy as np

from . import build as _build

E4M3, E5M2, E2M1 = 0, 1, 4
SCALE_MX, SCALE_TENSOR = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3

_lib = None


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB: another build of the same source (the sanitizer build
        # of the CPU test suite)
        path = os.environ.get("ORACLE_LIB") or _build.build(force=False)
        L = ctypes.CDLL(path)
        d, i64, p, i = ctypes.c_double, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        for name in ("oracle_decode_e4m3", "oracle_decode_e5m2", "oracle_decode_e2m1",
                     "oracle_decode_e8m0"):
            getattr(L, name).restype = d
            getattr(L, name).argtypes = [ctypes.c_uint]
        L.oracle_decode.restype = d
        L.oracle_decode.argtypes = [i, ctypes.c_uint]
        L.oracle_dequant.restype = i
        L.oracle_dequant.argtypes = [i, i, i, p, p, i64, i64, p]
        L.oracle_gemm.restype = i
        L.oracle_gemm.argtypes = [i, i, i, p, p, i, i, i, p, p, i64, i64, i64, p, p]
        L.oracle_gemm_entries.restype = i
        L.oracle_gemm_entries.argtypes = [i, i, i, p, p, i, i, i, p, p, i64, i64, i64,
                                          p, p, i64, p]
        L.oracle_grouped_gemm.restype = i
        L.oracle_grouped_gemm.argtypes = [i, p, p, p, p, p, i64, i64, i64, p]
        L.oracle_grouped_entries.restype = i
        L.oracle_grouped_entries.argtypes = [i, p, p, p, p, p, i64, i64, i64, p, p, i64, p]
        L.oracle_nearest_code.restype = ctypes.c_uint
        L.oracle_nearest_code.argtypes = [i, d]
        L.oracle_quant_mx.restype = i
        L.oracle_quant_mx.argtypes = [i, p, i64, i64, p, p]
        L.oracle_quant_group_weight.restype = i
        L.oracle_quant_group_weight.argtypes = [i, p, i64, i64, p, p]
        L.oracle_quant_group_act.restype = i
        L.oracle_quant_group_act.argtypes = [i, p, p, i64, i64, p, p]
        L.oracle_quant_tensor.restype = i
        L.oracle_quant_tensor.argtypes = [i, p, i64, p, p]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [d]
        L.oracle_bf16_rne_array.restype = None
        L.oracle_bf16_rne_array.argtypes = [p, i64, p]
        L.oracle_activation.restype = d
        L.oracle_activation.argtypes = [i, d]
        L.oracle_epilogue.restype = i
        L.oracle_epilogue.argtypes = [p, i64, i64, p, i]
        L.oracle_decode_bf16.restype = d
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint]
        L.oracle_grouped_gemm_bf16.restype = i
        L.oracle_grouped_gemm_bf16.argtypes = [i, p, p, p, i64, i64, i64, p]
        L.oracle_grouped_entries_bf16.restype = i
        L.oracle_grouped_entries_bf16.argtypes = [i, p, p, p, i64, i64, i64, p, p, i64, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def decode(fmt, codes):
    """Decode an array of codes (one code per element, nibbles unpacked)."""
    L = lib()
    flat = np.asarray(codes, dtype=np.int64).ravel()
    out = np.array([L.oracle_decode(fmt, int(c)) for c in flat], dtype=np.float64)
    return out.reshape(np.shape(codes))


def decode_e8m0(codes):
    L = lib()
    flat = np.asarray(codes, dtype=np.int64).ravel()
    return np.array([L.oracle_decode_e8m0(int(c)) for c in flat]).reshape(np.shape(codes))


def _scale_arg(scale_kind, s):
    if scale_kind == SCALE_TENSOR:
        return _c(np.asarray(s, dtype=np.float32).reshape(1), np.float32)
    return _c(s, np.uint8)


def dequant(fmt, scale_kind, transposed, codes, scales, rows, K):
    """Dequantized logical [rows, K] operand in FP64."""
    codes = _c(codes, np.uint8)
    s = _scale_arg(scale_kind, scales)
    out = np.empty((rows, K), dtype=np.float64)
    rc = lib().oracle_dequant(fmt, scale_kind, int(transposed), _ptr(codes), _ptr(s),
                              rows, K, _ptr(out))
    if rc:
        raise ValueError("oracle_dequant rejected the arguments (%d)" % rc)
    return out


def gemm(opA, opB, M, N, K):
    """opX = (fmt, scale_kind, transposed, codes, scales).  Returns FP64 [M,N]."""
    fa, ska, ta, A, sA = opA
    fb, skb, tb, B, sB = opB
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    sA = _scale_arg(ska, sA)
    sB = _scale_arg(skb, sB)
    work = np.empty((M + N) * K, dtype=np.float64)
    D = np.empty((M, N), dtype=np.float64)
    rc = lib().oracle_gemm(fa, ska, int(ta), _ptr(A), _ptr(sA), fb, skb, int(tb), _ptr(B),
                           _ptr(sB), M, N, K, _ptr(work), _ptr(D))
    if rc:
        raise ValueError("oracle_gemm rejected the arguments (%d)" % rc)
    return D


def gemm_entries(opA, opB, M, N, K, idx_m, idx_n):
    fa, ska, ta, A, sA = opA
    fb, skb, tb, B, sB = opB
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    sA = _scale_arg(ska, sA)
    sB = _scale_arg(skb, sB)
    im = _c(idx_m, np.int64)
    inn = _c(idx_n, np.int64)
    out = np.empty(im.size, dtype=np.float64)
    rc = lib().oracle_gemm_entries(fa, ska, int(ta), _ptr(A), _ptr(sA), fb, skb, int(tb),
                                   _ptr(B), _ptr(sB), M, N, K, _ptr(im), _ptr(inn), im.size,
                                   _ptr(out))
    if rc:
        raise ValueError("oracle_gemm_entries rejected the arguments (%d)" % rc)
    return out


def grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K, fill=np.nan):
    """FP64 [totM, N]; rows in no group keep ``fill``."""
    ms = _c(m_sizes, np.int64)
    XQ = _c(XQ, np.uint8)
    WQ = _c(WQ, np.uint8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    D = np.full((totM, N), fill, dtype=np.float64)
    rc = lib().oracle_grouped_gemm(ms.size, _ptr(ms), _ptr(XQ), _ptr(xs), _ptr(WQ), _ptr(ws),
                                   totM, N, K, _ptr(D))
    if rc:
        raise ValueError("oracle_grouped_gemm rejected the arguments (%d)" % rc)
    return D


def grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, idx_m, idx_n):
    ms = _c(m_sizes, np.int64)
    XQ = _c(XQ, np.uint8)
    WQ = _c(WQ, np.uint8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    im = _c(idx_m, np.int64)
    inn = _c(idx_n, np.int64)
    out = np.empty(im.size, dtype=np.float64)
    rc = lib().oracle_grouped_entries(ms.size, _ptr(ms), _ptr(XQ), _ptr(xs), _ptr(WQ),
                                      _ptr(ws), totM, N, K, _ptr(im), _ptr(inn), im.size,
                                      _ptr(out))
    if rc:
        raise ValueError("oracle_grouped_entries rejected the arguments (%d)" % rc)
    return out


def decode_bf16(bits):
    """FP64 values of BF16 bit patterns (the oracle's closed-form decoder)."""
    b = np.asarray(bits, dtype=np.uint16)
    f = np.vectorize(lambda v: lib().oracle_decode_bf16(int(v)), otypes=[np.float64])
    return f(b) if b.size else b.astype(np.float64)


def grouped_gemm_bf16(m_sizes, X, W, totM, N, K, fill=np.nan):
    """BF16 grouped GEMM, FP64 [totM, N]: X [totM, K] and W [G, N, K] are BF16
    bit patterns (uint16); rows in no group keep ``fill``."""
    ms = _c(m_sizes, np.int64)
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    D = np.full((totM, N), fill, dtype=np.float64)
    rc = lib().oracle_grouped_gemm_bf16(ms.size, _ptr(ms), _ptr(X), _ptr(W), totM, N, K, _ptr(D))
    if rc:
        raise ValueError("oracle_grouped_gemm_bf16 rejected the arguments (%d)" % rc)
    return D


def grouped_entries_bf16(m_sizes, X, W, totM, N, K, idx_m, idx_n):
    ms = _c(m_sizes, np.int64)
    X = _c(X, np.uint16)
    W = _c(W, np.uint16)
    im = _c(idx_m, np.int64)
    inn = _c(idx_n, np.int64)
    out = np.empty(im.size, dtype=np.float64)
    rc = lib().oracle_grouped_entries_bf16(ms.size, _ptr(ms), _ptr(X), _ptr(W), totM, N, K,
                                           _ptr(im), _ptr(inn), im.size, _ptr(out))
    if rc:
        raise ValueError("oracle_grouped_entries_bf16 rejected the arguments (%d)" % rc)
    return out


def bf16_rne(x):
    """Round FP64 values once to BF16 (RNE); returns uint16 bit patterns."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def within_tolerance(d, ref):
    """|d - ref| <= 2^-7 |ref| + 1e-3 max|ref| element-wise (NaN in d fails).

    Returns (ok, worst_ratio) where ratio = |d-ref| / bound.
    """
    d = np.asarray(d, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = 2.0 ** -7 * np.abs(ref) + 1e-3 * mx
    err = np.abs(d - ref)
    ok = bool(np.all(np.isfinite(d)) and np.all(err <= bound))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return ok, worst


def nearest_code(fmt, v):
    """The code of the representable value nearest to v (ties to the even
    code, saturating at +-fmt_max, sign kept)."""
    return int(lib().oracle_nearest_code(fmt, float(v)))


def quant_mx(fmt, x):
    """FP32 [rows, K] -> (codes, E8M0 scales [rows, K/32]); codes [rows, K]
    bytes, or [rows, K/2] packed nibbles for E2M1.  Exact E8M0 exponent
    floor(log2(amax / fmt_max)), nearest-value element rounding."""
    x = _c(x, np.float32)
    rows, K = x.shape
    codes = np.zeros((rows, K // 2 if fmt == E2M1 else K), np.uint8)
    scales = np.zeros((rows, K // 32), np.uint8)
    if lib().oracle_quant_mx(fmt, _ptr(x), rows, K, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("oracle_quant_mx: unsupported format or K")
    return codes, scales


def quant_group_act(m_sizes, x, codes_fill=0, xs_fill=np.nan):
    """Groupwise E4M3 activations: FP32 [totM, K] -> (codes [totM, K], FP32
    scales in the per-group block layout, totM*K/128).  Rows in no group keep
    the fill values."""
    x = _c(x, np.float32)
    totM, K = x.shape
    ms = _c(np.asarray(m_sizes), np.int64)
    codes = np.full((totM, K), codes_fill, np.uint8)
    xs = np.full(totM * (K // 128), xs_fill, np.float32)
    if lib().oracle_quant_group_act(len(ms), _ptr(ms), _ptr(x), totM, K, _ptr(codes), _ptr(xs)) != 0:
        raise ValueError("oracle_quant_group_act: K % 128 != 0")
    return codes, xs


def quant_group_weight(w):
    """Groupwise E4M3 weights: FP32 [G, N, K] -> (codes [G, N, K], FP32
    scales [G, N/128, K/128]), one scale per 128 x 128 block."""
    w = _c(w, np.float32)
    G, N, K = w.shape
    codes = np.zeros((G, N, K), np.uint8)
    ws = np.zeros((G, N // 128, K // 128), np.float32)
    if lib().oracle_quant_group_weight(G, _ptr(w), N, K, _ptr(codes), _ptr(ws)) != 0:
        raise ValueError("oracle_quant_group_weight: N or K not a multiple of 128")
    return codes, ws


def quant_tensor(fmt, x):
    """Tensor-wise E4M3 / E5M2: FP32 array -> (codes of the same shape,
    FP32 dequant scale s = amax / fmt_max, 1.0 for an all-zero tensor);
    codes = nearest(FP32 quotient x / s)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.shape, np.uint8)
    s = np.zeros(1, np.float32)
    if lib().oracle_quant_tensor(fmt, _ptr(x), x.size, _ptr(codes), _ptr(s)) != 0:
        raise ValueError("oracle_quant_tensor: format must be E4M3 or E5M2")
    return codes, np.float32(s[0])


def activation(act, z):
    """The epilogue's activation of one FP64 value (see oracle.c)."""
    return float(lib().oracle_activation(int(act), float(z)))


def epilogue(D, bias_bits=None, act=ACT_NONE):
    """act(D + bias[n]) in FP64 on a copy of the FP64 [M, N] product; bias as
    BF16 bit patterns [N] (uint16) or None."""
    out = np.array(D, dtype=np.float64, order="C", copy=True)
    M, N = out.shape
    b = None if bias_bits is None else _c(bias_bits, np.uint16)
    if b is not None and b.size != N:
        raise ValueError("bias must have N entries")
    if lib().oracle_epilogue(_ptr(out), M, N, _ptr(b), int(act)) != 0:
        raise ValueError("oracle_epilogue: unknown activation")
    return out
