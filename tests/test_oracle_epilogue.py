"""Pins of the oracle's epilogue, D = act(sum_k a b + bias[n]) (CPU only).

The activations are checked against torch's float64 implementations (an
independent library routine: relu, gelu with the tanh approximation, silu),
against identities they satisfy (act(x) - act(-x) = x for all three,
limits at large |x|), and the bias handling against hand-decoded BF16
values, with cases that fail if the bias is added after the activation or
indexed by row instead of column.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

ACTS = {
    oracle.ACT_RELU: lambda t: F.relu(t),
    oracle.ACT_GELU_TANH: lambda t: F.gelu(t, approximate="tanh"),
    oracle.ACT_SILU: lambda t: F.silu(t),
}


def _zs():
    rng = np.random.default_rng(3)
    z = np.concatenate([np.linspace(-20, 20, 4001), rng.standard_normal(2000) * 4,
                        [0.0, -0.0, 1e-30, -1e-30, 700.0, -700.0, 1e6, -1e6]])
    return z


@pytest.mark.parametrize("act", sorted(ACTS))
def test_activation_matches_torch_float64(act):
    z = _zs()
    ref = ACTS[act](torch.from_numpy(z)).numpy()
    got = np.array([oracle.activation(act, v) for v in z])
    # absolute slack 1e-15: for large negative z the tanh form's 1 + tanh(u)
    # cancels in either implementation (both values are ~1e-16, far below
    # anything a BF16 output of these magnitudes resolves)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-15), np.max(np.abs(got - ref))


@pytest.mark.parametrize("act", sorted(ACTS))
def test_activation_odd_part_is_identity(act):
    # relu, gelu (x Phi~(x) with Phi~(-x) = 1 - Phi~(x)) and silu
    # (x sigma(x), sigma(-x) = 1 - sigma(x)) all satisfy f(x) - f(-x) = x
    for x in np.linspace(-8, 8, 161):
        assert oracle.activation(act, x) - oracle.activation(act, -x) == pytest.approx(x, abs=1e-13)


def test_activation_limits_and_zero():
    for act in ACTS:
        assert oracle.activation(act, 0.0) == 0.0
        assert oracle.activation(act, 50.0) == pytest.approx(50.0, rel=1e-15)
        assert abs(oracle.activation(act, -50.0)) < 1e-15
    assert oracle.activation(oracle.ACT_NONE, -3.25) == -3.25
    assert oracle.activation(oracle.ACT_RELU, -3.25) == 0.0
    assert oracle.activation(oracle.ACT_RELU, 3.25) == 3.25
    # the tanh form differs from the erf form: at x = 1, 0.84119... vs 0.84134...
    assert abs(oracle.activation(oracle.ACT_GELU_TANH, 1.0) - 0.8413447460685429) > 1e-4


def test_epilogue_bias_by_column_before_activation():
    # bias bits: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E00 = 0.125 (sign, 8-bit
    # exponent with bias 127, 7-bit mantissa)
    D = np.array([[-1.5, 0.5, 3.0],
                  [0.0, -4.0, 1.0]])
    bias = np.array([0x3F80, 0xC000, 0x3E00], np.uint16)
    out = oracle.epilogue(D, bias, oracle.ACT_NONE)
    assert out.tolist() == [[-0.5, -1.5, 3.125], [1.0, -6.0, 1.125]]
    out = oracle.epilogue(D, bias, oracle.ACT_RELU)
    # relu after the bias: relu(-1.5 + 1) = 0 (bias after relu would give 1)
    assert out.tolist() == [[0.0, 0.0, 3.125], [1.0, 0.0, 1.125]]
    out = oracle.epilogue(D, None, oracle.ACT_RELU)
    assert out.tolist() == [[0.0, 0.5, 3.0], [0.0, 0.0, 1.0]]
    assert D[0, 0] == -1.5                       # the input is not modified


def test_epilogue_matches_torch_on_a_product():
    rng = np.random.default_rng(4)
    D = rng.standard_normal((37, 53)) * 3
    bias_f = rng.standard_normal(53).astype(np.float32)
    bias = (bias_f.view(np.uint32) >> 16).astype(np.uint16)      # truncated to BF16 bits
    bias_v = (bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for act, f in ACTS.items():
        ref = f(torch.from_numpy(D + bias_v[None, :])).numpy()
        assert np.allclose(oracle.epilogue(D, bias, act), ref, rtol=1e-14, atol=1e-15)


def test_epilogue_rejects_unknown_activation_and_bad_bias():
    with pytest.raises(ValueError):
        oracle.epilogue(np.zeros((2, 2)), None, 7)
    with pytest.raises(ValueError):
        oracle.epilogue(np.zeros((2, 3)), np.zeros(2, np.uint16), oracle.ACT_NONE)
