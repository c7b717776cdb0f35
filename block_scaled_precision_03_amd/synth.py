"""Seeded synthetic inputs: FP32 data drawn from a seeded generator and
encoded into element codes plus scales.

This module prepares inputs only.  It holds none of the GEMM's arithmetic:
it never decodes a code, never forms a product and never accumulates.  Both
the GPU library's tests/benchmark and the CPU oracle receive the codes and
scales it returns; the quantization recipe is an input recipe, not part of
the computed path.

Recipes (the pages fix only the formats and block sizes; the rules below are
this project's stated readings):

* MX (E8M0 per 32 K values): for each block, X = floor(log2(amax / fmt_max))
  evaluated exactly, clamped to [-127, 127]; scale code = X + 127; elements
  q = RNE_sat(x / 2^X).  fmt_max = 448 (E4M3), 57344 (E5M2), 6 (E2M1).
* Tensor-wise: s = amax / fmt_max (FP32) is the dequant multiplier;
  q = RNE_sat(x / s).
* Groupwise: per 1x128 activation block and per 128x128 weight block,
  s = amax / 448 (FP32; 1.0 for an all-zero block), q = RNE_sat(x / s).
  Activation scales are laid out per group: group g's block starts at
  start_g * (K/128) and holds (local row i, k-block kb) at i + kb * M_g.
* m_sizes (G groups): one seeded group is empty, the other G-1 sizes come
  from G-2 distinct seeded cut points in [1, totM-1].

Element rounding is round-to-nearest-even with saturation to +-fmt_max.
E4M3/E5M2 encoding goes through torch's CPU float8 casts after clamping;
E2M1 is encoded here by comparing against the midpoints of its value grid.
"""
from __future__ import annotations

import numpy as np
import torch

FMT_MAX = {"e4m3": 448.0, "e5m2": 57344.0, "e2m1": 6.0}


def normal(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _encode_fp8(y: torch.Tensor, elem: str) -> np.ndarray:
    m = FMT_MAX[elem]
    y = torch.clamp(y, -m, m)
    dt = torch.float8_e4m3fn if elem == "e4m3" else torch.float8_e5m2
    return y.to(dt).view(torch.uint8).numpy()


def _encode_e2m1(y: torch.Tensor) -> np.ndarray:
    """E2M1 nibble codes (unpacked, one per element), RNE with saturation."""
    a = torch.clamp(y.abs(), max=6.0)
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).to(torch.uint8)
    code = code | ((y < 0).to(torch.uint8) << 3)
    return code.numpy()


def pack_e2m1(nibbles: np.ndarray) -> np.ndarray:
    """Pack nibble codes two per byte along the last axis; even index -> low nibble."""
    n = np.asarray(nibbles, dtype=np.uint8)
    assert n.shape[-1] % 2 == 0
    return (n[..., 0::2] & 15) | ((n[..., 1::2] & 15) << 4)


def transpose_e2m1(packed: np.ndarray) -> np.ndarray:
    """Packed E2M1 codes [rows, K/2] (two per byte along K) -> the same codes
    stored [K, rows/2], two per byte along rows (even index -> low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    n = np.empty((p.shape[0], 2 * p.shape[1]), np.uint8)
    n[:, 0::2] = p & 15
    n[:, 1::2] = p >> 4
    return pack_e2m1(np.ascontiguousarray(n.T))


def _e8m0_exponent(amax: np.ndarray, fmt_max: float) -> np.ndarray:
    """X = floor(log2(amax / fmt_max)) exactly, clamped to [-127, 127]."""
    a = amax.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        x0 = np.floor(np.log2(a / fmt_max))
    x0 = np.where(a > 0, x0, -127.0)
    x0 = np.clip(x0, -200, 200)
    # exact corrections: fmt_max * 2^X <= amax < fmt_max * 2^(X+1)
    x0 = np.where((a > 0) & (fmt_max * np.exp2(x0) > a), x0 - 1, x0)
    x0 = np.where((a > 0) & (fmt_max * np.exp2(x0 + 1) <= a), x0 + 1, x0)
    return np.clip(x0, -127, 127).astype(np.int32)


def quant_mx(x: np.ndarray, elem: str):
    """x: FP32 [rows, K] -> (codes, scales).

    codes: uint8 [rows, K] (E4M3/E5M2) or packed uint8 [rows, K/2] (E2M1);
    scales: uint8 E8M0 [rows, K/32]."""
    rows, K = x.shape
    assert K % 32 == 0
    t = torch.from_numpy(np.ascontiguousarray(x)).view(rows, K // 32, 32)
    amax = t.abs().amax(dim=-1).numpy()
    X = _e8m0_exponent(amax, FMT_MAX[elem])
    inv = torch.from_numpy(np.exp2(-X.astype(np.float64)).astype(np.float32))
    y = (t * inv.unsqueeze(-1)).view(rows, K)
    if elem == "e2m1":
        codes = pack_e2m1(_encode_e2m1(y))
    else:
        codes = _encode_fp8(y, elem)
    return codes, (X + 127).astype(np.uint8)


def quant_tensor(x: np.ndarray, elem: str):
    """Per-tensor FP8: (codes uint8 same shape as x, FP32 dequant scale s)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = np.float32(amax) / np.float32(FMT_MAX[elem]) if amax > 0 else np.float32(1.0)
    y = torch.from_numpy(np.ascontiguousarray(x)) / torch.tensor(s, dtype=torch.float32)
    return _encode_fp8(y, elem), np.float32(s)


def _block_scale(amax: np.ndarray) -> np.ndarray:
    s = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quant_group_act(x: np.ndarray, m_sizes) -> tuple:
    """E4M3 with one FP32 scale per row per 128-K block, per-group block layout.

    Returns (codes uint8 [totM, K], xs float32 [totM*K/128])."""
    totM, K = x.shape
    assert K % 128 == 0
    t = torch.from_numpy(np.ascontiguousarray(x)).view(totM, K // 128, 128)
    s = _block_scale(t.abs().amax(dim=-1).numpy())          # [totM, K/128]
    y = (t / torch.from_numpy(s).unsqueeze(-1)).view(totM, K)
    codes = _encode_fp8(y, "e4m3")
    xs = np.empty(totM * (K // 128), dtype=np.float32)
    start = 0
    for mg in (int(v) for v in m_sizes):
        blk = s[start:start + mg, :].T                       # [K/128, mg]
        xs[start * (K // 128):(start + mg) * (K // 128)] = blk.reshape(-1)
        start += mg
    assert start == totM
    return codes, xs


def quant_group_weight(w: np.ndarray):
    """E4M3 with one FP32 scale per 128x128 block.  w: [G, N, K] ->
    (codes uint8 [G, N, K], ws float32 [G, N/128, K/128])."""
    G, N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    t = torch.from_numpy(np.ascontiguousarray(w)).view(G, N // 128, 128, K // 128, 128)
    amax = t.abs().amax(dim=(2, 4)).numpy()                  # [G, N/128, K/128]
    s = _block_scale(amax)
    st = torch.from_numpy(s).view(G, N // 128, 1, K // 128, 1)
    y = (t / st).view(G, N, K)
    return _encode_fp8(y, "e4m3"), s


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """FP32 data -> BF16 bit patterns (uint16), rounded to nearest even by
    torch's conversion: the BF16 operands of the BF16 grouped GEMM."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def m_sizes_for(totM: int, G: int, seed: int) -> np.ndarray:
    """Uneven group sizes summing to totM with exactly one empty group."""
    rng = np.random.default_rng(seed)
    assert G >= 2 and totM >= G - 1
    cuts = np.sort(rng.choice(np.arange(1, totM), size=G - 2, replace=False))
    sizes = np.diff(np.concatenate([[0], cuts, [totM]])).astype(np.int64)
    empty = int(rng.integers(0, G))
    out = np.insert(sizes, empty, 0).astype(np.int64)
    assert out.sum() == totM and len(out) == G
    return out


def seed_for(config: int, tensor: int, shape_index: int = 0) -> int:
    """Seed of tensor t (1 A/X, 2 B/W, 3 dY, 4 m_sizes) of config c."""
    return 1000 * config + 10 * shape_index + tensor
