"""GPU parity of grouped_bf16_gemm_run (plain and preshuffled weights)
against the FP64 oracle's BF16 grouped GEMM.  Rows of D outside every group
are prefilled with a sentinel and must keep it bit for bit; empty groups own
no rows."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_03_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

SENTINEL_BITS = 0x7F7F


def _inputs(seed, m_sizes, N, K, totM=None, scale=1.0):
    m_sizes = np.asarray(m_sizes, np.int64)
    cover = int(m_sizes.sum())
    totM = cover if totM is None else totM
    X = synth.bf16_bits(synth.normal(seed, (totM, K), scale))
    W = synth.bf16_bits(synth.normal(seed + 1, (len(m_sizes), N, K), scale))
    return m_sizes, X, W, totM


def _run(m_sizes, X, W, totM, N, K, preshuffled):
    from block_scaled_precision_03_amd import mxgemm
    G = len(m_sizes)
    D = torch.full((totM, N), 0, dtype=torch.int16, device=H.DEV)
    D.fill_(SENTINEL_BITS)
    Wd = H.dev(W.view(np.int16))
    if preshuffled:
        Wp = torch.empty_like(Wd)
        mxgemm.grouped_bf16_preshuffle_b(G, Wd, Wp, N, K)
        Wd = Wp
    mxgemm.grouped_bf16_run(G, H.dev(m_sizes), H.dev(X.view(np.int16)), Wd, D, totM, N, K,
                            b_preshuffled=preshuffled)
    torch.cuda.synchronize()
    return D


SPLITS = [
    [37, 0, 150, 3, 64, 1, 99, 30],    # uneven, one empty, not tile aligned
    [0, 0, 300, 0],                    # all rows in one group
    [0, 70, 129, 41],                  # first empty
    [200, 56, 0],                      # last empty
    [256, 256, 512],                   # tile aligned
    [1, 1, 1, 1, 1],                   # single rows
]


@pytest.mark.parametrize("preshuffled", [False, True])
@pytest.mark.parametrize("split", SPLITS)
def test_bf16_grouped_splits(split, preshuffled):
    """N = 192 (three 64-column tiles; one 256-column tile with 64 columns
    past N where the 256 x 256 kernel runs), K = 320 (five 64-value K
    steps): every entry against the oracle, every row written."""
    N, K = 192, 320
    m_sizes, X, W, totM = _inputs(811, split, N, K)
    D = _run(m_sizes, X, W, totM, N, K, preshuffled)
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    ref = oracle.grouped_gemm_bf16(m_sizes, X, W, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16)), ref, "bf16 grouped %s" % split)


def test_bf16_grouped_rows_outside_groups_untouched():
    N, K = 256, 256
    split = [100, 0, 77]
    m_sizes, X, W, totM = _inputs(821, split, N, K, totM=400)
    D = _run(m_sizes, X, W, totM, N, K, True)
    bits = H.bits(D.view(torch.bfloat16))
    assert np.all(bits[177:] == SENTINEL_BITS)
    ref = oracle.grouped_gemm_bf16(m_sizes, X, W, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16))[:177], ref[:177], "bf16 grouped, partial cover")


def _integer_inputs(rng, m_sizes, N, K):
    G, totM = len(m_sizes), int(np.sum(m_sizes))
    vals = synth.bf16_bits(np.array([-2.0, -1.0, 0.0, 1.0, 2.0, 0.5], np.float32))
    X = vals[rng.integers(0, len(vals), (totM, K))]
    W = vals[rng.integers(0, len(vals), (G, N, K))]
    return X, W, totM


# (m_sizes, N, K, kernel): one configuration per kernel the call can run;
# the 128-row streaming kernel runs 128 x 128 tiles (N = 1152: nine tile
# columns) and, where N is an odd multiple of 64 (1216), 128 x 64 tiles
EXACT_CASES = [
    ([30, 0, 47, 1, 60], 576, 1024, "stream64"),
    ([1200, 0, 1017, 1, 900, 1400], 1152, 256, "stream128"),
    ([1200, 0, 1017, 1, 900, 1400], 1216, 128, "stream128"),
    ([1500, 0, 1077, 2100, 1, 700, 2500, 314], 2048, 4096, "tiled"),
]


@pytest.mark.parametrize("preshuffled", [False, True])
@pytest.mark.parametrize("m_sizes,N,K,kernel", EXACT_CASES)
def test_bf16_grouped_integer_valued_bit_exact(m_sizes, N, K, kernel, preshuffled):
    """Values in {0, +-0.5, +-1, +-2}: every FP32 partial sum is exact, so
    each output is the oracle's exact sum rounded once to BF16, bit for bit,
    on each of the three kernels (the 256 x 256 one here with 288 tiles: a
    full round and a last round of 32 tiles handed to the streaming kernel
    on 256 compute units), ragged groups over several tiles.  The streaming
    shapes compare every entry, the 256 x 256 one every entry of 300 rows
    (every group's first and last among them)."""
    from block_scaled_precision_03_amd import mxgemm
    m_sizes = np.array(m_sizes, np.int64)
    X, W, totM = _integer_inputs(np.random.default_rng(99), m_sizes, N, K)
    names = {mxgemm.GROUPED_STREAM64: "stream64", mxgemm.GROUPED_STREAM128: "stream128",
             mxgemm.GROUPED_TILED: "tiled"}
    assert names[mxgemm.grouped_bf16_variant(len(m_sizes), totM, N, K)] == kernel
    D = _run(m_sizes, X, W, totM, N, K, preshuffled)
    bits = H.bits(D.view(torch.bfloat16))
    if kernel != "tiled":
        ref = oracle.grouped_gemm_bf16(m_sizes, X, W, totM, N, K)
        assert np.array_equal(bits, oracle.bf16_rne(ref))
        return
    starts = np.concatenate([[0], np.cumsum(m_sizes)])
    edge = [r for g in range(len(m_sizes)) if m_sizes[g] for r in (starts[g], starts[g + 1] - 1)]
    rows = np.unique(np.concatenate([edge, np.random.default_rng(5).integers(0, totM, 300 - len(edge))]))
    im, inn = np.repeat(rows, N), np.tile(np.arange(N), len(rows))
    ref = oracle.grouped_entries_bf16(m_sizes, X, W, totM, N, K, im, inn)
    assert np.array_equal(bits[im, inn], oracle.bf16_rne(ref))
    assert not np.any(bits == SENTINEL_BITS)


def test_bf16_grouped_preshuffled_equals_plain():
    m_sizes = np.array([513, 0, 260, 1000], np.int64)
    N, K = 448, 1536
    m_sizes, X, W, totM = _inputs(831, m_sizes, N, K)
    a = H.bits(_run(m_sizes, X, W, totM, N, K, False).view(torch.bfloat16))
    b = H.bits(_run(m_sizes, X, W, totM, N, K, True).view(torch.bfloat16))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("preshuffled", [False, True])
def test_bf16_grouped_several_rounds(preshuffled):
    """totM = 16384 over eight uneven groups (one empty), N = 2048,
    K = 1024: more 256 x 256 tiles than compute units (several rounds of the
    persistent grid).  Sampled entries and every group's first and last rows
    against the oracle, every row written."""
    G, N, K = 8, 2048, 1024
    m_sizes = synth.m_sizes_for(16384, G, 4242)
    m_sizes, X, W, totM = _inputs(841, m_sizes, N, K)
    D = _run(m_sizes, X, W, totM, N, K, preshuffled)
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    rng = np.random.default_rng(11)
    im, inn = H.sample_indices(rng, totM, N, 20000)
    starts = np.concatenate([[0], np.cumsum(m_sizes)])
    edge = np.array([r for g in range(G) if m_sizes[g] for r in (starts[g], starts[g + 1] - 1)])
    im = np.concatenate([im, np.repeat(edge, N)])
    inn = np.concatenate([inn, np.tile(np.arange(N), len(edge))])
    ref = oracle.grouped_entries_bf16(m_sizes, X, W, totM, N, K, im, inn)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16))[im, inn], ref, "bf16 grouped, 16384 rows")


def test_bf16_grouped_k_zero_writes_zeros():
    from block_scaled_precision_03_amd import mxgemm
    m_sizes = np.array([5, 0, 9], np.int64)
    totM, N = 20, 128
    D = torch.full((totM, N), 0, dtype=torch.int16, device=H.DEV)
    D.fill_(SENTINEL_BITS)
    mxgemm.grouped_bf16_run(3, H.dev(m_sizes), None, None, D, totM, N, 0)
    torch.cuda.synchronize()
    bits = H.bits(D.view(torch.bfloat16))
    assert np.all(bits[:14] == 0) and np.all(bits[14:] == SENTINEL_BITS)


def test_bf16_grouped_1024_groups():
    """MXG_GROUPED_MAX_G = 1024 groups of 0..40 rows (every fifth empty):
    the group table over all of them; every entry against the oracle."""
    G, N, K = 1024, 128, 128
    rng = np.random.default_rng(1026)
    split = rng.integers(0, 41, G)
    split[::5] = 0
    m_sizes, X, W, totM = _inputs(851, split, N, K)
    D = _run(m_sizes, X, W, totM, N, K, True)
    assert not np.any(H.bits(D.view(torch.bfloat16)) == SENTINEL_BITS)
    ref = oracle.grouped_gemm_bf16(m_sizes, X, W, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16)), ref, "bf16 grouped, 1024 groups")
