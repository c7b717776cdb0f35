"""GPU parity of the dense path where each persistent workgroup walks
several output tiles (more 256 x 256 tiles than compute units): the K steps
of consecutive tiles share one pipeline, a tile's first stage streams in
during the previous tile's last step, and its result is stored while the
next tile runs.  Covered: even and odd numbers of K steps per tile (the ring
slot of a tile's first step alternates when odd), ragged edges on tiles
walked later, N not a multiple of 4 (element-wise edge stores), every
format family and layout.  Entries are sampled (rows, columns, corners, the
last row and column) and compared with the FP64 oracle."""
import numpy as np
import pytest

import oracle
from block_scaled_precision_03_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

E4, E5, F4 = 0, 1, 4
T4, T5 = 16, 17
NT, NN, TN = 0, 1, 2


def _sampled(layout, opA, opB, M, N, K, what, preshuffle_b=False, count=3000):
    from block_scaled_precision_03_amd import mxgemm
    # these shapes run the persistent kernel (not the 64 x 64 one)
    assert mxgemm.dense_variant(opA.lib_fmt, opB.lib_fmt, layout, M, N, K) == mxgemm.DENSE_TILE256
    D = H.run_dense(layout, opA, opB, M, N, K, preshuffle_b=preshuffle_b)
    d = H.bf16_to_f64(D)
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    im, inn = H.sample_indices(rng, M, N, count)
    # every tile row and tile column, at a tile edge and in the middle
    for tm in range(0, M, 256):
        for off in (0, 127, 255):
            if tm + off < M:
                im = np.append(im, tm + off)
                inn = np.append(inn, rng.integers(0, N))
    for tn in range(0, N, 256):
        for off in (0, 100, 255):
            if tn + off < N:
                im = np.append(im, rng.integers(0, M))
                inn = np.append(inn, tn + off)
    ref = oracle.gemm_entries(opA.orc(), opB.orc(), M, N, K, im, inn)
    H.assert_close(d[im, inn], ref, what)
    return D


@pytest.mark.parametrize("M,N,K", [(4352, 4096, 384), (4352, 4096, 512), (4100, 4098, 256)])
@pytest.mark.parametrize("pre", [False, True])
def test_mxfp8_multitile(M, N, K, pre):
    x = synth.normal(7001 + M, (M, K))
    w = synth.normal(7002 + N, (N, K), 0.02)
    opA = H.make_operand(E4, x, False)
    opB = H.make_operand(E4, w, False)
    _sampled(NT, opA, opB, M, N, K, "mxfp8 %dx%dx%d pre=%d" % (M, N, K, pre), preshuffle_b=pre)


def test_mxfp8_multitile_preshuffled_equals_plain():
    M, N, K = 4352, 4160, 384
    x = synth.normal(7011, (M, K))
    w = synth.normal(7012, (N, K), 0.02)
    opA = H.make_operand(E4, x, False)
    opB = H.make_operand(E5, w, False)
    Dp = H.run_dense(NT, opA, opB, M, N, K)
    Ds = H.run_dense(NT, opA, opB, M, N, K, preshuffle_b=True)
    assert np.array_equal(H.bits(Dp), H.bits(Ds))


@pytest.mark.parametrize("M,N,K", [(4352, 4096, 768), (4100, 4160, 512)])
def test_mxfp4_multitile(M, N, K):
    x = synth.normal(7021 + M, (M, K))
    w = synth.normal(7022 + N, (N, K))
    opA = H.make_operand(F4, x, False)
    opB = H.make_operand(F4, w, False)
    _sampled(NT, opA, opB, M, N, K, "mxfp4 %dx%dx%d" % (M, N, K), preshuffle_b=True)


@pytest.mark.parametrize("layout,ta,tb", [(NT, False, False), (NN, False, True), (TN, True, True)])
@pytest.mark.parametrize("K", [384, 256])
def test_tensorwise_multitile(layout, ta, tb, K):
    M, N = 4352, 4112
    x = synth.normal(7031 + K, (M, K))
    w = synth.normal(7032 + K, (N, K), 0.02)
    opA = H.make_operand(T4, x, ta)
    opB = H.make_operand(T5, w, tb)
    _sampled(layout, opA, opB, M, N, K, "tensor layout %d K=%d" % (layout, K))


@pytest.mark.parametrize("fa,fb,M,N,K", [
    (E4, E4, 300, 520, 384), (E5, E5, 300, 520, 384), (E4, E5, 512, 768, 256),
    (E5, E4, 4352, 4096, 256), (F4, F4, 512, 512, 512),
])
def test_every_output_written_repeatedly(fa, fb, M, N, K):
    """Each call must write every element of D: a NaN sentinel fill may not
    survive, and five calls in a row give the same bits (guards against an
    epilogue whose cross-lane exchange or store ordering is unreliable)."""
    x = synth.normal(7041 + M + fa, (M, K))
    w = synth.normal(7042 + N + fb, (N, K))
    opA = H.make_operand(fa, x, False)
    opB = H.make_operand(fb, w, False)
    ref = oracle.gemm(opA.orc(), opB.orc(), M, N, K)
    first = None
    for rep in range(5):
        D = H.run_dense(NT, opA, opB, M, N, K, preshuffle_b=(rep % 2 == 1), d_fill=float("nan"))
        d = H.bf16_to_f64(D)
        assert not np.isnan(d).any(), "unwritten outputs on call %d" % rep
        H.assert_close(d, ref, "call %d" % rep)
        b = H.bits(D)
        if first is None:
            first = b
        assert np.array_equal(first, b), "call %d differs from call 0" % rep


@pytest.mark.parametrize("layout,ta,tb", [(NN, False, True), (TN, True, True)])
@pytest.mark.parametrize("K", [384, 512])
def test_mxfp8_backward_layouts_multitile(layout, ta, tb, K):
    M, N = 4352, 4112
    x = synth.normal(7051 + K, (M, K))
    w = synth.normal(7052 + K, (N, K), 0.02)
    opA = H.make_operand(E5, x, ta)
    opB = H.make_operand(E4, w, tb)
    _sampled(layout, opA, opB, M, N, K, "mx layout %d K=%d" % (layout, K))


@pytest.mark.parametrize("layout,ta,tb", [(NN, False, True), (TN, True, True)])
def test_mxfp4_backward_layouts_multitile(layout, ta, tb):
    """17 x 17 tiles of 256 with ragged last ones (rows and columns past
    the end of a transposed operand's k-row read the next k-row)."""
    M, N, K = 4384, 4128, 768
    x = synth.normal(7061 + layout, (M, K))
    w = synth.normal(7062 + layout, (N, K))
    opA = H.make_operand(F4, x, ta)
    opB = H.make_operand(F4, w, tb)
    _sampled(layout, opA, opB, M, N, K, "mxfp4 layout %d" % layout)

