"""GPU parity of grouped_fp8_gemm_run (plain and preshuffled weights) against
the FP64 oracle.  Rows of D outside every group are prefilled with a
sentinel and must keep it bit for bit; empty groups own no rows."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_03_amd import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

SENTINEL_BITS = 0x7F7F   # a large finite BF16 value no GEMM row here produces


def _inputs(seed, m_sizes, N, K, totM=None):
    m_sizes = np.asarray(m_sizes, np.int64)
    G = len(m_sizes)
    cover = int(m_sizes.sum())
    totM = cover if totM is None else totM
    x = synth.normal(seed, (totM, K))
    w = synth.normal(seed + 1, (G, N, K), 0.02)
    XQ, xs = synth.quant_group_act(x[:cover], m_sizes)
    if totM > cover:   # rows beyond every group: any codes, unit scales
        XQ = np.concatenate([XQ, np.full((totM - cover, K), 0x38, np.uint8)])
        xs = np.concatenate([xs, np.ones((totM - cover) * (K // 128), np.float32)])
    WQ, ws = synth.quant_group_weight(w)
    return m_sizes, XQ, xs, WQ, ws, totM


def _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled):
    from block_scaled_precision_03_amd import mxgemm
    G = len(m_sizes)
    D = torch.full((totM, N), 0, dtype=torch.int16, device=H.DEV)
    D.fill_(SENTINEL_BITS)
    W = H.dev(WQ)
    if preshuffled:
        Wp = torch.empty_like(W)
        mxgemm.grouped_preshuffle_b(G, W, Wp, N, K)
        W = Wp
    mxgemm.grouped_run(G, H.dev(m_sizes), H.dev(XQ), H.dev(xs), W, H.dev(ws), D, totM, N, K,
                       b_preshuffled=preshuffled)
    torch.cuda.synchronize()
    return D


def _run_forced(tmp_path, variant, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled):
    """_run with grouped_run made to launch `variant` (tune-cache entries for
    this key), whichever kernel the table or the estimate would pick."""
    from block_scaled_precision_03_amd import mxgemm
    _force_variant(mxgemm, tmp_path / "forced.txt", len(m_sizes), totM, N, K, variant)
    try:
        return _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    finally:
        mxgemm.tune_cache_clear()


SPLITS = [
    [37, 0, 150, 3, 64, 1, 99, 30],    # uneven, one empty, not tile aligned
    [0, 0, 300, 0],                    # all rows in one group
    [0, 70, 129, 41],                  # first empty
    [200, 56, 0],                      # last empty
    [128, 128, 256],                   # tile aligned
    [1, 1, 1, 1, 1],                   # single rows
]


@pytest.mark.parametrize("preshuffled", [False, True])
@pytest.mark.parametrize("split", SPLITS)
def test_grouped_splits(split, preshuffled):
    N, K = 256, 640              # G > 1, K > 128: per-group scale addressing matters
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(700 + len(split), split, N, K)
    D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16)), ref, "grouped %s" % split)


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_rows_outside_groups_untouched(preshuffled):
    N, K = 128, 384
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(801, [40, 0, 77], N, K, totM=200)
    D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    bits = H.bits(D.view(torch.bfloat16))
    assert np.all(bits[117:] == SENTINEL_BITS)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    H.assert_close(H.bf16_to_f64(D[:117].view(torch.bfloat16)), ref[:117], "covered rows")


def test_grouped_integer_valued_bit_exact():
    """Codes in {-2..2}, power-of-two scales: every partial sum is an exact
    FP32 integer, so group boundaries and scale addressing must be exact."""
    rng = np.random.default_rng(5)
    m_sizes = np.array([33, 0, 190, 7, 100], np.int64)
    totM, N, K, G = int(m_sizes.sum()), 256, 1024, 5
    vals = np.array([0xC0, 0xB8, 0x00, 0x38, 0x40], np.uint8)
    XQ = vals[rng.integers(0, 5, (totM, K))]
    WQ = vals[rng.integers(0, 5, (G, N, K))]
    xs = (2.0 ** rng.integers(0, 3, totM * K // 128)).astype(np.float32)
    ws = (2.0 ** rng.integers(0, 3, (G, N // 128, K // 128))).astype(np.float32)
    for pre in (False, True):
        D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, pre)
        ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
        assert np.array_equal(H.bits(D.view(torch.bfloat16)), oracle.bf16_rne(ref))


def test_grouped_scale_addressing_distinct_groups():
    """Distinct per-group activation scales: a kernel that reads another
    group's scales (the global-transpose mistake) fails this test."""
    rng = np.random.default_rng(9)
    m_sizes = np.array([20, 50, 0, 35], np.int64)
    totM, N, K, G = int(m_sizes.sum()), 128, 512, 4
    XQ = np.full((totM, K), 0x38, np.uint8)
    WQ = np.full((G, N, K), 0x38, np.uint8)
    xs = rng.integers(1, 9, totM * K // 128).astype(np.float32)
    ws = np.ones((G, 1, K // 128), np.float32)
    D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, False)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    assert np.array_equal(H.bits(D.view(torch.bfloat16)), oracle.bf16_rne(ref))


def test_grouped_precondition_violation_is_contained():
    """sum(m_sizes) > totM: groups are clamped to [0, totM); nothing outside
    D is touched and covered rows still match the clamped oracle."""
    N, K = 128, 256
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(901, [30, 50], N, K)
    bad = np.array([30, 500], np.int64)
    guard = torch.full((totM + 64, N), 0, dtype=torch.int16, device=H.DEV)
    guard.fill_(SENTINEL_BITS)
    from block_scaled_precision_03_amd import mxgemm
    mxgemm.grouped_run(2, H.dev(bad), H.dev(XQ), H.dev(xs), H.dev(WQ), H.dev(ws), guard[:totM],
                       totM, N, K)
    torch.cuda.synchronize()
    bits = H.bits(guard.view(torch.bfloat16))
    assert np.all(bits[totM:] == SENTINEL_BITS)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    H.assert_close(H.bf16_to_f64(guard[:30].view(torch.bfloat16)), ref[:30], "group 0")


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_long_k(preshuffled):
    """K = 2304 (18 steps of 128): the persistent kernel's DMA ring wraps
    many times within a tile and across tiles, and its stages past the last
    K step read nothing."""
    N, K = 384, 2304
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(911, [90, 7, 0, 160, 33], N, K)
    D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16)), ref, "grouped long K")


def _edge_samples(rng, m_sizes, N, count):
    """Random entries plus every group's first and last row (8 columns each)."""
    totM = int(np.sum(m_sizes))
    im, inn = H.sample_indices(rng, totM, N, count)
    starts = np.concatenate([[0], np.cumsum(m_sizes)])
    edge = np.array([r for g in range(len(m_sizes)) if m_sizes[g] for r in (starts[g], starts[g + 1] - 1)])
    return (np.concatenate([im, np.repeat(edge, 8)]),
            np.concatenate([inn, rng.integers(0, N, 8 * len(edge))]))


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_tiled_kernel(preshuffled, tmp_path):
    """Shapes for which the matrix-core kernel (256 x 256 tiles on the dense
    pipeline) runs: uneven groups, one empty, none tile aligned, 38 K steps.
    Every row written; sampled entries and every group's edge rows."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 2048, 4864
    split = [1500, 0, 1077, 2100, 1, 700, 2500, 314]
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(921, split, N, K)
    D = _run_forced(tmp_path, mxgemm.GROUPED_TILED, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    assert not np.any(H.bits(D.view(torch.bfloat16)) == SENTINEL_BITS)
    im, inn = _edge_samples(np.random.default_rng(7), m_sizes, N, 20000)
    ref = oracle.grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, im, inn)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16))[im, inn], ref, "grouped tiled kernel")


def test_grouped_small_shapes_take_the_streaming_kernels():
    """The parity cases above with few rows run the persistent 64 x 64
    kernel (the 128 x 128 one has its own test below), and so does the
    benchmark's 128 x 2048 x 7168 call (at 128 x 7168 x 2304 the table lists
    the 128 x 128 kernel, faster there warm and cold)."""
    from block_scaled_precision_03_amd import mxgemm
    got = {mxgemm.grouped_variant(len(split), int(sum(split)), 256, 640) for split in SPLITS}
    assert got == {mxgemm.GROUPED_STREAM64}
    assert mxgemm.grouped_variant(8, 128, 2048, 7168) == mxgemm.GROUPED_STREAM64
    assert mxgemm.grouped_variant(8, 128, 2048, 7168, False) == mxgemm.GROUPED_STREAM64


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_stream128_kernel(preshuffled, tmp_path):
    """The persistent kernel with 128 x 128 tiles: uneven groups (one empty,
    none tile aligned) and five tile columns (the preshuffled weights' 64-
    column groups in pairs), sampled entries and every group's first and
    last rows against the oracle, every row written."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 640, 2048
    split = [700, 0, 1, 1157, 129, 1013]
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(941, split, N, K)
    D = _run_forced(tmp_path, mxgemm.GROUPED_STREAM128, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    d = H.bf16_to_f64(D.view(torch.bfloat16))
    assert not np.any(H.bits(D.view(torch.bfloat16)) == SENTINEL_BITS)
    rng = np.random.default_rng(5)
    im, inn = H.sample_indices(rng, totM, N, 4000)
    starts = np.concatenate([[0], np.cumsum(m_sizes)])
    edge = np.array([r for g in range(len(split)) if split[g] for r in (starts[g], starts[g + 1] - 1)])
    im = np.concatenate([im, np.repeat(edge, N)])
    inn = np.concatenate([inn, np.tile(np.arange(N), len(edge))])
    ref = oracle.grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, im, inn)
    H.assert_close(d[im, inn], ref, "grouped 128-row tiles")


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_many_groups_several_rounds(preshuffled, tmp_path):
    """200 small groups (some empty): the persistent 64 x 64 kernel walks more
    real tiles than it has workgroups (on 256 compute units three whole
    rounds of 512 and a last round of 314 tiles, which do not split evenly
    over the eight XCD bands).
    Every row written, all entries against the oracle."""
    from block_scaled_precision_03_amd import mxgemm
    G, N, K = 200, 640, 256
    rng = np.random.default_rng(100)
    split = rng.integers(0, 41, G)
    split[::17] = 0
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(960, split, N, K)
    real_tiles = int(sum((m + 63) // 64 for m in split)) * (N // 64)
    P = min(((totM + 63) // 64 + G - 1) * (N // 64),
            2 * torch.cuda.get_device_properties(0).multi_processor_count)
    assert real_tiles // P >= 2 and (real_tiles % P) % 8 != 0
    D = _run_forced(tmp_path, mxgemm.GROUPED_STREAM64, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    assert not np.any(H.bits(D.view(torch.bfloat16)) == SENTINEL_BITS)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16)), ref, "grouped, 200 groups")


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_tiled_half_last_column_tile(preshuffled, tmp_path):
    """The matrix-core kernel's 256-column tiles with N = 1152 (the last tile
    of each group holds 128 real columns; its weight rows and block scales
    past N belong to the next group, or lie past the end for the last one),
    uneven groups (one empty, none tile aligned) and rows past the last
    group, which keep the sentinel.  Every entry of the last column tile,
    sampled entries and the groups' edge rows against the oracle."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 1152, 2048
    split = [1900, 0, 1077, 2100, 1, 700, 2500, 2622]
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(931, split, N, K, totM=11000)
    D = _run_forced(tmp_path, mxgemm.GROUPED_TILED, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    cover = int(sum(split))
    bits = H.bits(D.view(torch.bfloat16))
    assert np.all(bits[cover:] == SENTINEL_BITS)
    assert not np.any(bits[:cover] == SENTINEL_BITS)
    rng = np.random.default_rng(8)
    im, inn = _edge_samples(rng, m_sizes, N, 20000)
    rows = rng.integers(0, cover, 64)
    im = np.concatenate([im, np.repeat(rows, 128)])
    inn = np.concatenate([inn, np.tile(np.arange(1024, 1152), len(rows))])
    ref = oracle.grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, im, inn)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16))[im, inn], ref, "grouped N=1152")


@pytest.mark.parametrize("preshuffled", [False, True])
@pytest.mark.parametrize("variant", ["stream64", "stream128"])
def test_grouped_1024_groups_streaming(preshuffled, variant, tmp_path):
    """MXG_GROUPED_MAX_G = 1024 groups of 0..8 rows on each streaming kernel
    (64 x 64 and 128 x 128 tiles): the group table spans sixteen 64-group
    chunks.  Every entry against the oracle, every row written."""
    from block_scaled_precision_03_amd import mxgemm
    G, N, K = 1024, 256, 256
    split = np.random.default_rng(1024).integers(0, 9, G)
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(970, split, N, K)
    v = mxgemm.GROUPED_STREAM64 if variant == "stream64" else mxgemm.GROUPED_STREAM128
    D = _run_forced(tmp_path, v, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    assert not np.any(H.bits(D.view(torch.bfloat16)) == SENTINEL_BITS)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16)), ref, "grouped, 1024 groups")


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_1024_groups_tiled(preshuffled, tmp_path):
    """MXG_GROUPED_MAX_G = 1024 groups of 0..512 rows (every seventh empty)
    on the matrix-core kernel: its group table and binary search over all of
    them, eight rounds of persistent tiles.  Integer-valued codes with
    power-of-two scales, so sampled entries and every group's edge rows must
    match the oracle bit for bit."""
    from block_scaled_precision_03_amd import mxgemm
    G, N, K = 1024, 256, 4096
    rng = np.random.default_rng(1025)
    split = rng.integers(0, 513, G)
    split[::7] = 0
    m_sizes = split.astype(np.int64)
    totM = int(m_sizes.sum())
    vals = np.array([0xC0, 0xB8, 0x00, 0x38, 0x40], np.uint8)
    XQ = vals[rng.integers(0, 5, (totM, K), dtype=np.uint8)]
    WQ = vals[rng.integers(0, 5, (G, N, K), dtype=np.uint8)]
    xs = (2.0 ** rng.integers(0, 3, totM * K // 128)).astype(np.float32)
    ws = (2.0 ** rng.integers(0, 3, (G, N // 128, K // 128))).astype(np.float32)
    D = _run_forced(tmp_path, mxgemm.GROUPED_TILED, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    im, inn = _edge_samples(np.random.default_rng(6), m_sizes, N, 20000)
    ref = oracle.grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, im, inn)
    assert np.array_equal(bits[im, inn], oracle.bf16_rne(ref))


def test_grouped_autotune_records_the_fastest_and_the_run_uses_it():
    """The tuner times all three kernels on the caller's buffers, records the
    fastest under (G, nextPow2(totM), N, K, preshuffled), leaves a correct
    result in D, and every later call with that key launches the recorded
    kernel; under graph capture it refuses and enqueues nothing."""
    from block_scaled_precision_03_amd import mxgemm
    m_sizes = synth.m_sizes_for(1024, 8, 9301)
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(9302, m_sizes, 2048, 1024)
    N, K, G = 2048, 1024, 8
    W = H.dev(WQ)
    Wp = torch.empty_like(W)
    mxgemm.grouped_preshuffle_b(G, W, Wp, N, K)
    dm, dx, dxs, dws = H.dev(m_sizes), H.dev(XQ), H.dev(xs), H.dev(ws)
    ref = oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K)
    mxgemm.tune_cache_clear()
    try:
        D = torch.full((totM, N), float("nan"), dtype=torch.bfloat16, device=H.DEV)
        v, us = mxgemm.grouped_autotune(G, dm, dx, dxs, Wp, dws, D, totM, N, K, True, reps=5)
        torch.cuda.synchronize()
        assert v in (mxgemm.GROUPED_STREAM64, mxgemm.GROUPED_STREAM128, mxgemm.GROUPED_TILED)
        assert all(u > 0 for u in us) and us[v] == min(us)
        assert mxgemm.tune_cache_size() == 1
        assert mxgemm.grouped_variant(G, totM, N, K, True) == v
        assert mxgemm.grouped_variant(G, 700, N, K, True) == v          # same nextPow2(totM)
        H.assert_close(H.bf16_to_f64(D), ref, "grouped after autotune")
        D2 = torch.full((totM, N), float("nan"), dtype=torch.bfloat16, device=H.DEV)
        mxgemm.grouped_run(G, dm, dx, dxs, Wp, dws, D2, totM, N, K, b_preshuffled=True)
        torch.cuda.synchronize()
        H.assert_close(H.bf16_to_f64(D2), ref, "grouped with the tuned kernel")
        # the tuner waits on events: refused while the stream is captured
        lib = mxgemm.lib()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rc = lib.grouped_fp8_gemm_autotune(G, dm.data_ptr(), dx.data_ptr(), dxs.data_ptr(), Wp.data_ptr(),
                                               dws.data_ptr(), D2.data_ptr(), totM, N, K, 1, 5, None, None,
                                               torch.cuda.current_stream().cuda_stream)
        assert rc == -1
    finally:
        mxgemm.tune_cache_clear()


def _force_variant(mxgemm, path, G, totM, N, K, variant):
    """Tune-cache entries (plain and preshuffled) that make grouped_run launch
    `variant` for this key."""
    lg = max(0, int(totM - 1).bit_length())
    with open(path, "w") as f:
        for pre in (0, 1):
            f.write("grouped %d %d %d %d %d %d\n" % (G, lg, N, K, pre, variant))
    mxgemm.tune_cache_clear()
    mxgemm.tune_cache_load(str(path))
    assert mxgemm.grouped_variant(G, totM, N, K) == variant


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_tiled_tail_pieces(preshuffled, tmp_path):
    """The 256 x 256 kernel's last, partial round goes to the streaming kernel
    in 128 x 64 pieces.  N = 1152 gives five tile columns, the last one half
    real, and the groups give 60 row tiles: 300 tiles, of which (on 256
    compute units) 256 run in one full round and 44 as 352 pieces, among
    them column quarters past N and the empty half of the last group's
    82-row last tile.  The result must equal bit for bit those of the 128 x 128
    and 64 x 64 streaming kernels over the whole problem (the same
    per-element arithmetic), every row must be written, and sampled entries,
    the groups' edge rows and every entry of the last group's last 300 rows
    must match the oracle."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 1152, 1024
    split = [2000, 0, 3000, 1, 5000, 4690]
    G = len(split)
    row_tiles = sum((m + 255) // 256 for m in split)
    assert row_tiles == 60
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nb = row_tiles * 5
    if cus == 256:
        pieces = (16 if 16 * 44 <= cus else 8) * 44      # the tail kernel: one workgroup per CU
        assert nb % cus == 44 and (pieces + cus - 1) // cus <= 2
    m_sizes, XQ, xs, WQ, ws, totM = _inputs(951, split, N, K)
    try:
        _force_variant(mxgemm, tmp_path / "tiled.txt", G, totM, N, K, mxgemm.GROUPED_TILED)
        D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
        _force_variant(mxgemm, tmp_path / "s128.txt", G, totM, N, K, mxgemm.GROUPED_STREAM128)
        D128 = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
        _force_variant(mxgemm, tmp_path / "s64.txt", G, totM, N, K, mxgemm.GROUPED_STREAM64)
        D64 = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    finally:
        mxgemm.tune_cache_clear()
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    assert np.array_equal(bits, H.bits(D128.view(torch.bfloat16)))
    assert np.array_equal(bits, H.bits(D64.view(torch.bfloat16)))
    rng = np.random.default_rng(9)
    im, inn = _edge_samples(rng, m_sizes, N, 20000)
    last = np.arange(totM - 300, totM)
    im = np.concatenate([im, np.repeat(last, N)])
    inn = np.concatenate([inn, np.tile(np.arange(N), len(last))])
    ref = oracle.grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, im, inn)
    H.assert_close(H.bf16_to_f64(D.view(torch.bfloat16))[im, inn], ref, "grouped tail pieces")


def test_grouped_tiled_tail_pieces_integer_valued_bit_exact(tmp_path):
    """The split as above with integer-valued codes and power-of-two scales
    (every partial sum exact in FP32): every entry of the last group, whose
    rows the tail pieces hold, equals the oracle's bit for bit."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 1152, 1024
    split = [2000, 0, 3000, 1, 5000, 4690]
    G = len(split)
    m_sizes = np.asarray(split, np.int64)
    totM = int(m_sizes.sum())
    rng = np.random.default_rng(1152)
    vals = np.array([0xC0, 0xB8, 0x00, 0x38, 0x40], np.uint8)
    XQ = vals[rng.integers(0, 5, (totM, K), dtype=np.uint8)]
    WQ = vals[rng.integers(0, 5, (G, N, K), dtype=np.uint8)]
    xs = (2.0 ** rng.integers(0, 3, totM * K // 128)).astype(np.float32)
    ws = (2.0 ** rng.integers(0, 3, (G, N // 128, K // 128))).astype(np.float32)
    try:
        _force_variant(mxgemm, tmp_path / "tiled.txt", G, totM, N, K, mxgemm.GROUPED_TILED)
        D = _run(m_sizes, XQ, xs, WQ, ws, totM, N, K, True)
    finally:
        mxgemm.tune_cache_clear()
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    last = np.arange(totM - split[-1], totM)
    im, inn = np.repeat(last, N), np.tile(np.arange(N), len(last))
    ref = oracle.grouped_entries(m_sizes, XQ, xs, WQ, ws, totM, N, K, im, inn)
    assert np.array_equal(bits[im, inn], oracle.bf16_rne(ref))


@pytest.mark.parametrize("preshuffled", [False, True])
def test_grouped_tiled_tail_64_row_pieces_bit_exact(preshuffled, tmp_path):
    """A last round of 12 tiles of the 256 x 256 kernel (on 256 compute
    units; N = 256, 268 row tiles): sixteen 64 x 64 pieces per tile, the
    lower half of each tail tile empty, groups ending inside a piece and one
    single-row group.  Integer-valued codes and power-of-two scales (every
    partial sum exact in FP32): every entry equals the oracle's bit for
    bit, and every row is written."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 256, 256
    split = [20000, 1, 0, 30030, 17800]
    G = len(split)
    m_sizes = np.asarray(split, np.int64)
    totM = int(m_sizes.sum())
    row_tiles = sum((m + 255) // 256 for m in split)
    assert row_tiles == 268
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        r = row_tiles % cus
        assert r == 12 and 16 * r <= cus      # the tail grid is one workgroup per CU
    rng = np.random.default_rng(268)
    vals = np.array([0xC0, 0xB8, 0x00, 0x38, 0x40], np.uint8)
    XQ = vals[rng.integers(0, 5, (totM, K), dtype=np.uint8)]
    WQ = vals[rng.integers(0, 5, (G, N, K), dtype=np.uint8)]
    xs = (2.0 ** rng.integers(0, 3, totM * K // 128)).astype(np.float32)
    ws = (2.0 ** rng.integers(0, 3, (G, N // 128, K // 128))).astype(np.float32)
    D = _run_forced(tmp_path, mxgemm.GROUPED_TILED, m_sizes, XQ, xs, WQ, ws, totM, N, K, preshuffled)
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    if "tail64" not in _ORACLE_CACHE:         # the same inputs for both weight layouts
        _ORACLE_CACHE["tail64"] = oracle.bf16_rne(oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K))
    assert np.array_equal(bits, _ORACLE_CACHE["tail64"])


_ORACLE_CACHE = {}


@pytest.mark.parametrize("variant", ["stream64", "stream128", "tiled"])
def test_grouped_single_k_step_every_kernel(variant, tmp_path):
    """K = 128, one K step, on each kernel: the 64 x 64 kernel's two-step
    stages and the tail kernel's hold one live step and one that reads
    zeros.  N = 384 (the 256 x 256 kernel's last column tile half real),
    uneven groups (one empty, one single row); on 256 compute units the
    256 x 256 kernel has 276 tiles and hands a last round of 20 to the tail
    kernel.  Integer-valued codes and power-of-two scales: every entry
    equals the oracle's bit for bit, every row written."""
    from block_scaled_precision_03_amd import mxgemm
    N, K = 384, 128
    split = [10000, 0, 1, 14000, 10500]
    G = len(split)
    m_sizes = np.asarray(split, np.int64)
    totM = int(m_sizes.sum())
    rng = np.random.default_rng(128)
    vals = np.array([0xC0, 0xB8, 0x00, 0x38, 0x40], np.uint8)
    XQ = vals[rng.integers(0, 5, (totM, K), dtype=np.uint8)]
    WQ = vals[rng.integers(0, 5, (G, N, K), dtype=np.uint8)]
    xs = (2.0 ** rng.integers(0, 3, totM * K // 128)).astype(np.float32)
    ws = (2.0 ** rng.integers(0, 3, (G, N // 128, K // 128))).astype(np.float32)
    v = {"stream64": mxgemm.GROUPED_STREAM64, "stream128": mxgemm.GROUPED_STREAM128,
         "tiled": mxgemm.GROUPED_TILED}[variant]
    D = _run_forced(tmp_path, v, m_sizes, XQ, xs, WQ, ws, totM, N, K, True)
    bits = H.bits(D.view(torch.bfloat16))
    assert not np.any(bits == SENTINEL_BITS)
    if "k1" not in _ORACLE_CACHE:             # the same inputs for every kernel
        _ORACLE_CACHE["k1"] = oracle.bf16_rne(oracle.grouped_gemm(m_sizes, XQ, xs, WQ, ws, totM, N, K))
    assert np.array_equal(bits, _ORACLE_CACHE["k1"])


def test_grouped_tiled_random_shapes_match_streaming(tmp_path):
    """Random group counts (1..64) and sizes (some empty), N an odd or even
    multiple of 128, K from 256 to 1024, rows past the last group, sized so
    that the 256 x 256 kernel has more tiles than compute units: with its
    partial last round split off to the streaming kernel or not (the tile
    count decides; both occur here), its output equals the 128 x 128
    streaming kernel's over the whole problem bit for bit, and rows outside
    every group keep the sentinel."""
    from block_scaled_precision_03_amd import mxgemm
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(4242)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)   # every E4M3 value but NaN
    split_seen = {True: 0, False: 0}
    for case in range(8):
        G = int(rng.integers(1, 65))
        N = 128 * int(rng.integers(5, 17))
        K = 128 * int(rng.integers(2, 9))
        tiles_n = (N + 255) // 256
        target = int(rng.integers(cus + 1, 3 * cus)) // tiles_n + G   # 256-row tiles wanted
        sizes = rng.integers(0, 2 * 256 * target // G + 1, G)
        sizes[rng.random(G) < 0.2] = 0
        m_sizes = sizes.astype(np.int64)
        cover = int(m_sizes.sum())
        totM = cover + int(rng.integers(0, 300))
        row_tiles = int(sum((m + 255) // 256 for m in m_sizes))
        nb = row_tiles * tiles_n
        grid = min(((totM + 255) // 256 + G - 1) * tiles_n, cus)
        r = nb % grid
        pieces = (16 if 16 * r <= cus else 8) * r
        split = nb > grid and r > 0 and (pieces + cus - 1) // cus <= 2
        if nb <= grid:
            continue
        split_seen[split] += 1
        XQ = codes[rng.integers(0, len(codes), (totM, K))]
        WQ = codes[rng.integers(0, len(codes), (G, N, K))]
        xs = (2.0 ** rng.integers(-12, -4, totM * K // 128) * rng.uniform(1, 2, totM * K // 128)).astype(np.float32)
        ws = (2.0 ** rng.integers(-12, -4, (G, N // 128, K // 128))).astype(np.float32)
        out = {}
        for pre in (False, True):
            try:
                for v in (mxgemm.GROUPED_TILED, mxgemm.GROUPED_STREAM128):
                    _force_variant(mxgemm, tmp_path / "v.txt", G, totM, N, K, v)
                    out[(pre, v)] = H.bits(_run(m_sizes, XQ, xs, WQ, ws, totM, N, K, pre).view(torch.bfloat16))
            finally:
                mxgemm.tune_cache_clear()
            what = "case %d: G=%d totM=%d N=%d K=%d tiles=%d split=%s pre=%s" % (case, G, totM, N, K, nb, split, pre)
            assert np.array_equal(out[(pre, mxgemm.GROUPED_TILED)], out[(pre, mxgemm.GROUPED_STREAM128)]), what
            assert np.all(out[(pre, mxgemm.GROUPED_TILED)][cover:] == SENTINEL_BITS), what
            assert not np.any(out[(pre, mxgemm.GROUPED_TILED)][:cover] == SENTINEL_BITS), what
    assert split_seen[True] >= 2 and split_seen[False] >= 1, split_seen
