"""Seeded synthetic inputs shared by the GPU path's callers and the oracle.

This module holds no attention arithmetic: only random draws, the bf16
storage format (round-to-nearest-even from fp32, exact widening back), the
deterministic generator that the "FlashAttention" deep-dive page uses in its
self-test (section "Code"), and the choice of sampled heads.

Workloads follow the pages' shapes: Q, K, V (and dO) are i.i.d. N(0, 1), drawn
in fp32 with numpy's PCG64 ``standard_normal`` in the order Q, K, V, dO from one
generator, then stored as bf16 (RNE) for the bf16 workloads.  The oracle reads
the exact fp64 widening of the very values the GPU receives.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns the
    raw uint16 bit patterns.  NaN stays NaN (quiet)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)
    return rounded.reshape(f.shape)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).reshape(b.shape)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


@dataclass
class Tensors:
    """One seeded draw.  ``bits`` holds the stored representation (uint16 bf16
    patterns, float32 for fp32 workloads, uint8 e4m3 bytes for fp8); ``f64``
    the exact real values; ``descale`` the fp8 dequantisation factors."""
    names: tuple
    dtype: str
    bits: dict
    f64: dict
    descale: dict = field(default_factory=dict)


def normal_qkv(B, H, N, d, seed, dtype="bf16", with_dout=False) -> Tensors:
    """Q, K, V (and dO) of shape [B, H, N, d], i.i.d. N(0,1) from
    ``numpy.random.default_rng(seed)``, drawn in fp32 in the order Q, K, V, dO."""
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    rng = np.random.default_rng(seed)
    names = ("q", "k", "v", "do") if with_dout else ("q", "k", "v")
    bits, f64 = {}, {}
    for n in names:
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if dtype == "bf16":
            bits[n] = bf16_bits(x)
            f64[n] = bf16_to_f64(bits[n])
        else:
            bits[n] = x
            f64[n] = x.astype(np.float64)
    return Tensors(names, dtype, bits, f64)


def normal_gqa(B, Hq, Hkv, N, d, seed, with_dout=False) -> Tensors:
    """Grouped heads: Q (and dO) [B, Hq, N, d], K, V [B, Hkv, N, d], i.i.d.
    N(0,1) from ``numpy.random.default_rng(seed)`` in the order Q, K, V, dO,
    stored as bf16."""
    rng = np.random.default_rng(seed)
    names = ("q", "k", "v", "do") if with_dout else ("q", "k", "v")
    bits, f64 = {}, {}
    for n in names:
        heads = Hkv if n in ("k", "v") else Hq
        bits[n] = bf16_bits(rng.standard_normal((B, heads, N, d), dtype=np.float32))
        f64[n] = bf16_to_f64(bits[n])
    return Tensors(names, "bf16", bits, f64)


def _e4m3_values() -> np.ndarray:
    """The 256 OCP fp8 e4m3 codes as float64 (sign, 4 exponent bits with bias
    7, 3 mantissa bits; exponent 0 is subnormal; 0x7F and 0xFF are NaN)."""
    codes = np.arange(256)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    mant = (codes & 7).astype(np.float64)
    val = np.where(e == 0, mant / 8.0 * 2.0 ** -6, (1.0 + mant / 8.0) * 2.0 ** (e - 7.0))
    val = sign * val
    val[(codes & 0x7F) == 0x7F] = np.nan
    return val


_E4M3 = _e4m3_values()


def e4m3_to_f64(bits) -> np.ndarray:
    """Exact value of OCP e4m3 bytes."""
    return _E4M3[np.asarray(bits, dtype=np.uint8)]


def e4m3_bits(x) -> np.ndarray:
    """Round values to OCP e4m3 (nearest, ties to the even code), saturating
    at +-448; returns the bytes."""
    x = np.asarray(x, dtype=np.float64)
    pos = _E4M3[:0x7F]  # codes 0x00 .. 0x7E, ascending
    a = np.minimum(np.abs(x), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 1, len(pos) - 1)
    lo = hi - 1
    d_lo, d_hi = a - pos[lo], pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == 0, 0, code).astype(np.uint8)
    return (code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def fp8_qkv(B, Hq, Hkv, N, d, seed) -> Tensors:
    """Q [B, Hq, N, d], K, V [B, Hkv, N, d]: i.i.d. N(0,1) fp32 draws from
    ``numpy.random.default_rng(seed)`` (order Q, K, V), each tensor quantised
    to OCP e4m3 with one factor per tensor, descale = max|x| / 448 rounded to
    fp32.  ``bits`` holds the e4m3 bytes, ``f64`` the exact real values
    descale * e4m3, and ``descale`` the three factors."""
    rng = np.random.default_rng(seed)
    bits, f64, descale = {}, {}, {}
    for n, heads in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((B, heads, N, d), dtype=np.float32)
        ds = float(np.float32(np.max(np.abs(x)) / 448.0))
        bits[n] = e4m3_bits(x.astype(np.float64) / ds)
        f64[n] = ds * e4m3_to_f64(bits[n])
        descale[n] = ds
    return Tensors(("q", "k", "v"), "fp8", bits, f64, descale)


def decode_qkv(B, Hq, Hkv, Nk, d, seed, with_f64=True) -> Tensors:
    """Decode step: Q [B, Hq, d] (one query row per head), K, V cache
    [B, Hkv, Nk, d], i.i.d. N(0,1) from ``numpy.random.default_rng(seed)`` in
    the order Q, K, V, stored as bf16 (``f64`` left empty unless with_f64)."""
    rng = np.random.default_rng(seed)
    bits, f64 = {}, {}
    for n, shape in (("q", (B, Hq, d)), ("k", (B, Hkv, Nk, d)), ("v", (B, Hkv, Nk, d))):
        bits[n] = bf16_bits(rng.standard_normal(shape, dtype=np.float32))
        if with_f64:
            f64[n] = bf16_to_f64(bits[n])
    return Tensors(("q", "k", "v"), "bf16", bits, f64)


def page_generator(n, d, seed) -> np.ndarray:
    """The deterministic fp32 generator of the deep-dive page's self-test:
    element i (row-major over n x d) is ((i * 7919 + seed) mod 1000) / 500 - 1."""
    i = np.arange(n * d, dtype=np.int64)
    return (((i * 7919 + seed) % 1000).astype(np.float32) / np.float32(500.0)
            - np.float32(1.0)).reshape(n, d)


def default_scale(d) -> float:
    """1/sqrt(d) rounded to fp32, the value both sides receive."""
    return float(np.float32(1.0 / math.sqrt(d)))


def sample_heads(bh_total, count, seed) -> list:
    """A seeded sample of ``count`` distinct flat (b*H + h) head indices that
    always contains head 0; sorted."""
    if count >= bh_total:
        return list(range(bh_total))
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, bh_total), size=count - 1, replace=False)
    return sorted([0] + [int(x) for x in rest])


# The five workloads (shapes, dtype, mask) and their seeds.
WORKLOADS = {
    "c1_f32_n256_d64": dict(B=1, H=1, N=256, d=64, dtype="f32", causal=False, seed=20261),
    "c2_bf16_n2048_d64": dict(B=4, H=16, N=2048, d=64, dtype="bf16", causal=False, seed=20262),
    "c3_bf16_causal_n8192_d128": dict(B=2, H=32, N=8192, d=128, dtype="bf16", causal=True,
                                      seed=20263),
    "c4_bf16_n18000_d128": dict(B=1, H=16, N=18000, d=128, dtype="bf16", causal=False,
                                seed=20264),
    "c5_bf16_causal_fwdbwd_n4096_d128": dict(B=4, H=16, N=4096, d=128, dtype="bf16",
                                             causal=True, seed=20265, backward=True),
}
