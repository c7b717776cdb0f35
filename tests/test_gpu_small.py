"""GPU parity of the 64 x 64 dense NT kernel (small outputs) against the
oracle, and its agreement bit for bit with the persistent 256 x 256 kernel:
the small problem is embedded in the first rows and columns of one large
enough for the persistent kernel, whose output block must equal the small
kernel's exactly (both run the same sequence of matrix-core instructions
per output element).  Every format and scale mode, plain and preshuffled B,
ragged edges, long K, the fused epilogue and the benchmark's 256^3 GEMM."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_03_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

E4, E5, F4 = 0, 1, 4
T4, T5 = 16, 17
NT, NN = 0, 1


def _variant(fa, fb, layout, M, N, K):
    from block_scaled_precision_03_amd import mxgemm
    return mxgemm.dense_variant(fa, fb, layout, M, N, K)


def test_variant_choice():
    from block_scaled_precision_03_amd import mxgemm
    assert _variant(E4, E4, NT, 256, 256, 256) == mxgemm.DENSE_TILE64
    assert _variant(E4, E4, NT, 200, 136, 1024) == mxgemm.DENSE_TILE64
    assert _variant(E4, E4, NT, 8192, 8192, 8192) == mxgemm.DENSE_TILE256
    assert _variant(E4, E4, NT, 16384, 14336, 4096) == mxgemm.DENSE_TILE256
    assert _variant(E4, E4, NN, 256, 256, 256) == mxgemm.DENSE_TILE256     # NT only


def _embed(op, rows_big, rng, fmt):
    """The operand with extra random rows after its own (same K)."""
    extra = H.make_operand(fmt, synth.normal(int(rng.integers(1 << 30)), (rows_big - op.rows, op.K)), False)
    codes = np.concatenate([op.codes, extra.codes])
    if H.LIB2ORC[fmt][1] == oracle.SCALE_MX:
        s = np.concatenate([op.scales, extra.scales])
    else:
        s = op.scales                             # one scale per tensor: keep the small one's
    return H.Operand(fmt, codes, s, False, rows_big, op.K)


CASES = [(E4, E4), (E4, E5), (E5, E4), (E5, E5), (T4, T5), (T5, T4), (T4, T4), (F4, F4)]


@pytest.mark.parametrize("pre", [False, True])
@pytest.mark.parametrize("fa,fb", CASES)
def test_small_equals_persistent_bitwise(fa, fb, pre):
    M, N, K = 200, 136, 1024                      # ragged in both directions
    rng = np.random.default_rng(fa * 31 + fb + 2 * pre)
    opA = H.make_operand(fa, synth.normal(6001, (M, K)), False)
    opB = H.make_operand(fb, synth.normal(6002, (N, K), 0.05), False)
    assert _variant(fa, fb, NT, M, N, K) == 1
    Ds = H.run_dense(NT, opA, opB, M, N, K, preshuffle_b=pre, d_fill=float("nan"))
    Mb = Nb = 4160                                # 17 x 17 tiles of 256: the persistent kernel
    assert _variant(fa, fb, NT, Mb, Nb, K) == 0
    bigA, bigB = _embed(opA, Mb, rng, fa), _embed(opB, Nb, rng, fb)
    Db = H.run_dense(NT, bigA, bigB, Mb, Nb, K, preshuffle_b=pre, d_fill=float("nan"))
    assert np.array_equal(H.bits(Ds), H.bits(Db)[:M, :N])
    ref = oracle.gemm(opA.orc(), opB.orc(), M, N, K)
    H.assert_close(H.bf16_to_f64(Ds), ref, "small kernel (%d, %d)" % (fa, fb))


@pytest.mark.parametrize("fmt", [E4, F4])
def test_small_integer_valued_bit_exact(fmt):
    rng = np.random.default_rng(61 + fmt)
    M, N, K = 130, 250, 2048
    opA, opB = H.int_operand(rng, fmt, M, K), H.int_operand(rng, fmt, N, K)
    for pre in (False, True):
        D = H.run_dense(NT, opA, opB, M, N, K, preshuffle_b=pre, d_fill=float("nan"))
        assert np.array_equal(H.bits(D), oracle.bf16_rne(oracle.gemm(opA.orc(), opB.orc(), M, N, K)))


def test_small_long_k():
    """256 x 512 x 16384: 128 K steps in one workgroup per tile."""
    M, N, K = 256, 512, 16384
    assert _variant(E4, E4, NT, M, N, K) == 1
    opA = H.make_operand(E4, synth.normal(6011, (M, K)), False)
    opB = H.make_operand(E4, synth.normal(6012, (N, K), 0.02), False)
    D = H.run_dense(NT, opA, opB, M, N, K, preshuffle_b=True)
    H.assert_close(H.bf16_to_f64(D), oracle.gemm(opA.orc(), opB.orc(), M, N, K), "small long K")


def test_small_benchmark_256_cube():
    M = N = K = 256
    x = synth.normal(synth.seed_for(1, 1), (M, K))
    w = synth.normal(synth.seed_for(1, 2), (N, K))
    opA, opB = H.make_operand(E4, x, False), H.make_operand(E4, w, False)
    for pre in (False, True):
        D = H.run_dense(NT, opA, opB, M, N, K, preshuffle_b=pre)
        H.assert_close(H.bf16_to_f64(D), oracle.gemm(opA.orc(), opB.orc(), M, N, K), "256^3")


@pytest.mark.parametrize("fa,fb", [(E4, E4), (T4, T5), (F4, F4)])
def test_small_fused_epilogue(fa, fb):
    from block_scaled_precision_03_amd import mxgemm
    M, N, K = 100, 192, 512
    opA = H.make_operand(fa, synth.normal(6021, (M, K)), False)
    opB = H.make_operand(fb, synth.normal(6022, (N, K), 0.05), False)
    bias = (synth.normal(6023, (N,)).view(np.uint32) >> 16).astype(np.uint16)
    for act in (oracle.ACT_RELU, oracle.ACT_GELU_TANH, oracle.ACT_SILU):
        D = H.empty_d(M, N, float("nan"))
        mxgemm.run_fused(fa, fb, NT, opA.dev_codes(), opA.dev_scales(), opB.dev_codes(), opB.dev_scales(),
                         D, M, N, K, bias=H.dev(bias.view(np.int16)), activation=act)
        torch.cuda.synchronize()
        ref = oracle.epilogue(oracle.gemm(opA.orc(), opB.orc(), M, N, K), bias, act)
        H.assert_close(H.bf16_to_f64(D), ref, "small fused act=%d" % act)
