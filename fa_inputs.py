"""Seeded synthetic inputs for exact attention, shared by the tests, the bench and
the CPU oracle's callers.

This module holds no attention arithmetic: it only draws i.i.d. N(0, 1) samples
from a seeded NumPy generator and, for bf16 workloads, rounds them to bf16 with
round-to-nearest-even so that the device path and the oracle read identical
values. The pages run attention on activations of these shapes; no dataset or
trained weight is involved, so standard-normal data stands in for them.

Draw order is fixed: q, k, v, then dO (backward only), each with
``rng.standard_normal(shape, dtype=float32)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "bf16_round_bits",
    "bf16_bits_to_f32",
    "bf16_round",
    "make_inputs",
    "make_block_mask",
]


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN stays NaN (quiet bit set); +-inf and overflow to inf follow IEEE RNE.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    is_nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if is_nan.any():
        out[is_nan] = ((u[is_nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal fp32 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded (RNE) to the nearest bf16, returned as fp32."""
    return bf16_bits_to_f32(bf16_round_bits(x))


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, mask, scale and seed."""

    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    seed: int
    backward: bool = False
    scale: float = field(default=float("nan"))

    def __post_init__(self):
        if math.isnan(self.scale):
            object.__setattr__(self, "scale", 1.0 / math.sqrt(self.d))

    @property
    def q_shape(self):
        return (self.B, self.Hq, self.N, self.d)

    @property
    def kv_shape(self):
        return (self.B, self.Hkv, self.N, self.d)


# The five workloads the attention path is measured and checked on.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_f32_b1h1n256d64", 1, 1, 1, 256, 64, "f32", False, seed=0),
        Workload("fwd_bf16_b4h16n2048d64", 4, 16, 16, 2048, 64, "bf16", False, seed=1),
        Workload("fwd_causal_bf16_b2h16n4096d128", 2, 16, 16, 4096, 128, "bf16", True, seed=2),
        Workload("fwd_causal_gqa_bf16_b2hq64hkv8n4096d128", 2, 64, 8, 4096, 128, "bf16", True, seed=3),
        Workload("bwd_causal_bf16_b2h16n4096d128", 2, 16, 16, 4096, 128, "bf16", True, seed=4, backward=True),
    ]
}


def make_inputs(B, Hq, Hkv, N, d, dtype="bf16", seed=0, backward=False, q_mult=1.0):
    """Draw q, k, v (and dO) as fp32 arrays holding exactly the values the device reads.

    For ``dtype == "bf16"`` every array is rounded to bf16 (RNE) and the bit
    patterns are returned alongside under ``<name>_bits``. ``q_mult`` scales q
    before rounding (a peaky-softmax variant used only for correctness checks).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.default_rng(seed)
    shapes = {"q": (B, Hq, N, d), "k": (B, Hkv, N, d), "v": (B, Hkv, N, d)}
    if backward:
        shapes["dO"] = (B, Hq, N, d)
    out = {}
    for name, shape in shapes.items():
        x = rng.standard_normal(shape, dtype=np.float32)
        if name == "q" and q_mult != 1.0:
            x = (x * np.float32(q_mult)).astype(np.float32)
        if dtype == "bf16":
            bits = bf16_round_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
        else:
            out[name] = x
    return out


def make_workload_inputs(w: Workload, q_mult=1.0):
    return make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, w.seed, w.backward, q_mult)


def make_block_mask(kind, B, Hq, N, seed=0, block=128):
    """A block mask [B, Hq, n_blk, n_blk] (uint8, 1 = the query block sees the key block), n_blk = ceil(N / block).

    kinds: "all" (every block), "diag" (block i sees block i), "band" (blocks
    i-1, i, i+1 and the first block: a sliding window plus one global block),
    "random" (each entry 1 with probability 1/2, seeded, differing per batch
    and head), "holes" ("random" with every third query block seeing nothing).
    """
    n = -(-N // block)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    if kind == "all":
        m = np.ones((n, n), bool)
    elif kind == "diag":
        m = i == j
    elif kind == "band":
        m = (np.abs(i - j) <= 1) | (j == 0)
    elif kind in ("random", "holes"):
        m = np.random.default_rng(seed).random((B, Hq, n, n)) < 0.5
        if kind == "holes":
            m[:, :, ::3, :] = False
        return m.astype(np.uint8)
    else:
        raise ValueError(f"unknown block mask kind {kind!r}")
    return np.ascontiguousarray(np.broadcast_to(m, (B, Hq, n, n))).astype(np.uint8)
