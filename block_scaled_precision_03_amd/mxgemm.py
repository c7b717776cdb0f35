"""Thin ctypes binding of libmxgemm.so (C ABI in include/mxgemm.h).

Argument marshalling only: torch tensors are passed as raw device pointers
plus sizes, and the current HIP stream of torch.  Every step of the GEMM runs
in the library's kernels; there is no fallback path.  Importing this module
raises if the library has not been built.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxgemm.so")

# Values mirror include/mxgemm.h.
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP = 0, -1, -2, -3, -4
MXFP8_E4M3, MXFP8_E5M2, MXFP4_E2M1 = 0, 1, 4
FP8_E4M3_TENSOR, FP8_E5M2_TENSOR = 16, 17
PRESHUFFLED = 0x100
NT, NN, TN = 0, 1, 2
GROUPED_MAX_G = 1024
GROUPED_STREAM64, GROUPED_TILED, GROUPED_STREAM128 = 0, 1, 2
ACT_NONE, ACT_RELU, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3
DENSE_TILE256, DENSE_TILE64 = 0, 1

EXPORTS = (
    "mxgemm_init", "mxgemm_status_string", "mxgemm_run", "mxgemm_validate",
    "mxgemm_run_fused", "mxgemm_validate_fused", "mxgemm_dense_variant",
    "grouped_fp8_gemm_run", "grouped_fp8_gemm_validate", "grouped_fp8_gemm_variant",
    "grouped_fp8_gemm_autotune", "mxgemm_tune_cache_save", "mxgemm_tune_cache_load",
    "mxgemm_tune_cache_clear", "mxgemm_tune_cache_size",
    "mxgemm_preshuffle_b_bytes", "mxgemm_preshuffle_b",
    "mxgemm_preshuffle_scales_bytes", "mxgemm_preshuffle_scales",
    "grouped_fp8_preshuffle_b", "mxgemm_mfma_ceiling",
    "grouped_bf16_gemm_run", "grouped_bf16_gemm_validate", "grouped_bf16_gemm_variant",
    "grouped_bf16_preshuffle_b",
    "mxgemm_quantize_mx", "mxgemm_quantize_tensor", "grouped_fp8_quantize_act", "grouped_fp8_quantize_weight",
)

if not os.path.exists(LIB_PATH):
    raise ImportError("libmxgemm.so is not built (run __graft_entry__.build() or "
                      "python -m block_scaled_precision_03_amd.csrc.build)")

_lib = ctypes.CDLL(LIB_PATH)
_i, _i64, _p = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
_lib.mxgemm_init.restype = _i
_lib.mxgemm_init.argtypes = []
_lib.mxgemm_status_string.restype = ctypes.c_char_p
_lib.mxgemm_status_string.argtypes = [_i]
_lib.mxgemm_run.restype = _i
_lib.mxgemm_run.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p]
_lib.mxgemm_validate.restype = _i
_lib.mxgemm_validate.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _i64, _i64, _i64]
_lib.mxgemm_dense_variant.restype = _i
_lib.mxgemm_dense_variant.argtypes = [_i, _i, _i, _i64, _i64, _i64]
_lib.mxgemm_run_fused.restype = _i
_lib.mxgemm_run_fused.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i, _p]
_lib.mxgemm_validate_fused.restype = _i
_lib.mxgemm_validate_fused.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i]
_lib.grouped_fp8_gemm_run.restype = _i
_lib.grouped_fp8_gemm_run.argtypes = [_i, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i, _p]
_lib.grouped_fp8_gemm_validate.restype = _i
_lib.grouped_fp8_gemm_validate.argtypes = [_i, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i]
_lib.grouped_fp8_gemm_variant.restype = _i
_lib.grouped_fp8_gemm_variant.argtypes = [_i, _i64, _i64, _i64, _i]
_lib.grouped_fp8_gemm_autotune.restype = _i
_lib.grouped_fp8_gemm_autotune.argtypes = [_i, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i, _i, _p, _p, _p]
_lib.mxgemm_tune_cache_save.restype = _i
_lib.mxgemm_tune_cache_save.argtypes = [ctypes.c_char_p]
_lib.mxgemm_tune_cache_load.restype = _i
_lib.mxgemm_tune_cache_load.argtypes = [ctypes.c_char_p]
_lib.mxgemm_tune_cache_clear.restype = _i
_lib.mxgemm_tune_cache_clear.argtypes = []
_lib.mxgemm_tune_cache_size.restype = _i64
_lib.mxgemm_tune_cache_size.argtypes = []
_lib.mxgemm_preshuffle_b_bytes.restype = _i64
_lib.mxgemm_preshuffle_b_bytes.argtypes = [_i, _i64, _i64]
_lib.mxgemm_preshuffle_b.restype = _i
_lib.mxgemm_preshuffle_b.argtypes = [_i, _i, _p, _p, _i64, _i64, _p]
_lib.mxgemm_preshuffle_scales_bytes.restype = _i64
_lib.mxgemm_preshuffle_scales_bytes.argtypes = [_i64, _i64]
_lib.mxgemm_preshuffle_scales.restype = _i
_lib.mxgemm_preshuffle_scales.argtypes = [_p, _p, _i64, _i64, _p]
_lib.mxgemm_mfma_ceiling.restype = _i
_lib.mxgemm_mfma_ceiling.argtypes = [_i, _i64, _p, _p]
_lib.grouped_fp8_preshuffle_b.restype = _i
_lib.grouped_fp8_preshuffle_b.argtypes = [_i, _p, _p, _i64, _i64, _p]
_lib.grouped_bf16_gemm_run.restype = _i
_lib.grouped_bf16_gemm_run.argtypes = [_i, _p, _p, _p, _p, _i64, _i64, _i64, _i, _p]
_lib.grouped_bf16_gemm_validate.restype = _i
_lib.grouped_bf16_gemm_validate.argtypes = [_i, _p, _p, _p, _p, _i64, _i64, _i64, _i]
_lib.grouped_bf16_gemm_variant.restype = _i
_lib.grouped_bf16_gemm_variant.argtypes = [_i, _i64, _i64, _i64]
_lib.grouped_bf16_preshuffle_b.restype = _i
_lib.grouped_bf16_preshuffle_b.argtypes = [_i, _p, _p, _i64, _i64, _p]
_lib.mxgemm_quantize_mx.restype = _i
_lib.mxgemm_quantize_mx.argtypes = [_i, _p, _p, _p, _i64, _i64, _p]
_lib.mxgemm_quantize_tensor.restype = _i
_lib.mxgemm_quantize_tensor.argtypes = [_i, _p, _p, _p, _i64, _p]
_lib.grouped_fp8_quantize_weight.restype = _i
_lib.grouped_fp8_quantize_weight.argtypes = [_i, _p, _p, _p, _i64, _i64, _p]
_lib.grouped_fp8_quantize_act.restype = _i
_lib.grouped_fp8_quantize_act.argtypes = [_i, _p, _p, _p, _p, _i64, _i64, _p]


class MxgemmError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (%d)" % (what, status_string(status), status))
        self.status = status


def lib():
    return _lib


def status_string(s):
    return _lib.mxgemm_status_string(int(s)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_current_raw_stream = None


def _stream(stream):
    """The HIP stream handle of `stream`, or torch's current stream on the
    current device.  After the first call (which goes through the public API
    and so initializes torch's device state), the current stream is read
    with torch's raw-handle accessor, which builds no Stream object: a
    launch-bound call then spends less time here than in the launch."""
    global _current_raw_stream
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    if _current_raw_stream is None:
        import torch
        handle = torch.cuda.current_stream().cuda_stream
        get_raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        get_dev = getattr(torch._C, "_cuda_getDevice", None)
        if get_raw is not None and get_dev is not None:
            _current_raw_stream = lambda: get_raw(get_dev())
        else:
            _current_raw_stream = lambda: torch.cuda.current_stream().cuda_stream
        return handle
    return _current_raw_stream()


def _check(rc, what):
    if rc != OK:
        raise MxgemmError(rc, what)


def init():
    _check(_lib.mxgemm_init(), "mxgemm_init")


def run(fmtA, fmtB, layout, A, sA, B, sB, D, M, N, K, stream=None):
    """D[M,N] (bf16) = sum_k a(m,k) b(n,k); see include/mxgemm.h."""
    _check(_lib.mxgemm_run(fmtA, fmtB, layout, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(D),
                           M, N, K, _stream(stream)), "mxgemm_run")


def validate(fmtA, fmtB, layout, A, sA, B, sB, D, M, N, K):
    return _lib.mxgemm_validate(fmtA, fmtB, layout, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB),
                                _ptr(D), M, N, K)


def dense_variant(fmtA, fmtB, layout, M, N, K):
    """DENSE_TILE256 or DENSE_TILE64: the kernel run / run_fused launch for
    these shapes on the current device."""
    return _lib.mxgemm_dense_variant(fmtA, fmtB, layout, M, N, K)


def run_fused(fmtA, fmtB, layout, A, sA, B, sB, D, M, N, K, bias=None, activation=ACT_NONE,
              stream=None):
    """D = act(sum_k a(m,k) b(n,k) + bias[n]) in BF16; bias: BF16 [N] or None."""
    _check(_lib.mxgemm_run_fused(fmtA, fmtB, layout, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(D),
                                 M, N, K, _ptr(bias), activation, _stream(stream)), "mxgemm_run_fused")


def validate_fused(fmtA, fmtB, layout, A, sA, B, sB, D, M, N, K, bias=None, activation=ACT_NONE):
    return _lib.mxgemm_validate_fused(fmtA, fmtB, layout, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB),
                                      _ptr(D), M, N, K, _ptr(bias), activation)


def grouped_run(G, m_sizes, XQ, x_scale, WQ, w_scale, D, totM, N, K, b_preshuffled=False,
                stream=None):
    _check(_lib.grouped_fp8_gemm_run(G, _ptr(m_sizes), _ptr(XQ), _ptr(x_scale), _ptr(WQ),
                                     _ptr(w_scale), _ptr(D), totM, N, K, int(bool(b_preshuffled)),
                                     _stream(stream)), "grouped_fp8_gemm_run")


def grouped_validate(G, m_sizes, XQ, x_scale, WQ, w_scale, D, totM, N, K, b_preshuffled=False):
    return _lib.grouped_fp8_gemm_validate(G, _ptr(m_sizes), _ptr(XQ), _ptr(x_scale), _ptr(WQ),
                                          _ptr(w_scale), _ptr(D), totM, N, K,
                                          int(bool(b_preshuffled)))


def grouped_variant(G, totM, N, K, b_preshuffled=True):
    """GROUPED_STREAM64, GROUPED_STREAM128 or GROUPED_TILED: the kernel
    grouped_run launches for these shapes on the current device."""
    return _lib.grouped_fp8_gemm_variant(G, totM, N, K, int(bool(b_preshuffled)))


def grouped_autotune(G, m_sizes, XQ, x_scale, WQ, w_scale, D, totM, N, K, b_preshuffled=True, reps=10,
                     stream=None):
    """Time the three grouped kernels on these buffers, record the fastest in
    the library's tune cache; returns (variant, [us per call by variant])."""
    v = ctypes.c_int(-1)
    us = (ctypes.c_float * 3)()
    _check(_lib.grouped_fp8_gemm_autotune(G, _ptr(m_sizes), _ptr(XQ), _ptr(x_scale), _ptr(WQ), _ptr(w_scale),
                                          _ptr(D), totM, N, K, int(bool(b_preshuffled)), reps,
                                          ctypes.byref(v), us, _stream(stream)), "grouped_fp8_gemm_autotune")
    return v.value, list(us)


def tune_cache_save(path):
    _check(_lib.mxgemm_tune_cache_save(os.fsencode(path)), "mxgemm_tune_cache_save")


def tune_cache_load(path):
    _check(_lib.mxgemm_tune_cache_load(os.fsencode(path)), "mxgemm_tune_cache_load")


def tune_cache_clear():
    _check(_lib.mxgemm_tune_cache_clear(), "mxgemm_tune_cache_clear")


def tune_cache_size():
    return _lib.mxgemm_tune_cache_size()

def preshuffle_b_bytes(fmtB, N, K):
    return _lib.mxgemm_preshuffle_b_bytes(fmtB, N, K)


def preshuffle_b(fmtB, layout, B, B_out, N, K, stream=None):
    _check(_lib.mxgemm_preshuffle_b(fmtB, layout, _ptr(B), _ptr(B_out), N, K, _stream(stream)),
           "mxgemm_preshuffle_b")


def preshuffle_scales_bytes(rows, K):
    return _lib.mxgemm_preshuffle_scales_bytes(rows, K)


def preshuffle_scales(s, s_out, rows, K, stream=None):
    _check(_lib.mxgemm_preshuffle_scales(_ptr(s), _ptr(s_out), rows, K, _stream(stream)),
           "mxgemm_preshuffle_scales")


def grouped_preshuffle_b(G, WQ, WQ_out, N, K, stream=None):
    _check(_lib.grouped_fp8_preshuffle_b(G, _ptr(WQ), _ptr(WQ_out), N, K, _stream(stream)),
           "grouped_fp8_preshuffle_b")


def grouped_bf16_run(G, m_sizes, X, W, D, totM, N, K, b_preshuffled=False, stream=None):
    """BF16 grouped GEMM: D[rows of g] = X[rows of g] W[g]^T; see include/mxgemm.h."""
    _check(_lib.grouped_bf16_gemm_run(G, _ptr(m_sizes), _ptr(X), _ptr(W), _ptr(D), totM, N, K,
                                      int(bool(b_preshuffled)), _stream(stream)), "grouped_bf16_gemm_run")


def grouped_bf16_validate(G, m_sizes, X, W, D, totM, N, K, b_preshuffled=False):
    return _lib.grouped_bf16_gemm_validate(G, _ptr(m_sizes), _ptr(X), _ptr(W), _ptr(D), totM, N, K,
                                           int(bool(b_preshuffled)))


def grouped_bf16_variant(G, totM, N, K):
    """GROUPED_STREAM64, GROUPED_STREAM128 or GROUPED_TILED: the kernel
    grouped_bf16_run launches for these static shapes."""
    return _lib.grouped_bf16_gemm_variant(G, totM, N, K)


def grouped_bf16_preshuffle_b(G, W, W_out, N, K, stream=None):
    _check(_lib.grouped_bf16_preshuffle_b(G, _ptr(W), _ptr(W_out), N, K, _stream(stream)),
           "grouped_bf16_preshuffle_b")


def mfma_ceiling(fmt, iters, clk, stream=None):
    """Matrix-core throughput probe (see include/mxgemm.h); clk: device
    tensor of three int64."""
    _check(_lib.mxgemm_mfma_ceiling(fmt, iters, _ptr(clk), _stream(stream)), "mxgemm_mfma_ceiling")


def quantize_mx(fmt, x, codes, scales, rows, K, stream=None):
    """FP32 [rows, K] -> MX codes and E8M0 scales (see include/mxgemm.h)."""
    _check(_lib.mxgemm_quantize_mx(fmt, _ptr(x), _ptr(codes), _ptr(scales), rows, K, _stream(stream)),
           "mxgemm_quantize_mx")


def quantize_tensor(fmt, x, codes, scale, n, stream=None):
    """FP32 values -> tensor-wise FP8 codes and one FP32 dequant scale (see
    include/mxgemm.h)."""
    _check(_lib.mxgemm_quantize_tensor(fmt, _ptr(x), _ptr(codes), _ptr(scale), n, _stream(stream)),
           "mxgemm_quantize_tensor")


def grouped_quantize_act(G, m_sizes, x, codes, x_scale, totM, K, stream=None):
    """FP32 activations -> E4M3 codes and per-group block-layout FP32 scales."""
    _check(_lib.grouped_fp8_quantize_act(G, _ptr(m_sizes), _ptr(x), _ptr(codes), _ptr(x_scale), totM, K,
                                         _stream(stream)), "grouped_fp8_quantize_act")


def grouped_quantize_weight(G, w, codes, w_scale, N, K, stream=None):
    """FP32 weights [G, N, K] -> E4M3 codes and FP32 128 x 128 block scales."""
    _check(_lib.grouped_fp8_quantize_weight(G, _ptr(w), _ptr(codes), _ptr(w_scale), N, K, _stream(stream)),
           "grouped_fp8_quantize_weight")
