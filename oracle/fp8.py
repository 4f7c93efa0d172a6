"""FP8 (e4m3) block-wise quantisation and attention on dequantised inputs, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the library.

Followed: "Flash Attention V3技术解析" (mlqm.cn), sections 1.3 ("低精度计算的工程
实践": block-wise quantisation of the inputs of Q K^T, fused with the rotary
embedding that acts on Q and K) and 3.2 ("块级缩放因子": one scale per block,
scale = max|block| / (largest code), code = round(block / scale)); and "4.3
FlashAttention-2与FlashAttention-3演进" (aiknowledge.cn), FlashAttention-3
section 2 (FP8 for the cheap steps, BF16 where precision matters).

Readings where the pages are silent or garbled:
* format: e4m3 as defined by the OCP 8-bit floating point specification (the
  format the gfx950 matrix unit reads): 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits; exponent 0 is subnormal (m / 8 * 2^-6); the code with
  all exponent and mantissa bits set is NaN; no infinities; largest finite
  value 448. The page's "/127.0" is read as "/ largest code value", i.e. 448
  for e4m3 (127 is the int8 maximum).
* rounding: to nearest, ties to the even code; values beyond 448 saturate to
  448 (they do not occur: x / scale <= 448 by construction, up to one
  rounding of the division). The sign is kept as in IEEE 754 rounding, so a
  negative value whose magnitude rounds to zero gives -0 (code 0x80).
* block: 64 consecutive rows of one (batch, head) across the whole head dim
  (the page's 64 x 64 block with d = 64); a block of zeros gets scale 1.
* the scale is formed and applied in float32, as the kernels do:
  scale = fp32(amax) / fp32(448) and code = e4m3(fp32(x) / scale), each a
  correctly rounded float32 division.
* only Q and K are quantised; V and the probabilities stay bf16 (the pages'
  mixed precision: the quantisation is fused with the rotary embedding, which
  touches Q and K only, and the P V step is where the pages keep BF16).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fwd

__all__ = ["E4M3_MAX", "e4m3_values", "e4m3_decode", "e4m3_encode", "quantize_blockwise_e4m3",
           "dequantize_blockwise_e4m3", "attention_fwd_fp8"]

E4M3_MAX = 448.0


def e4m3_values():
    """Value of each of the 256 codes (float64; NaN for 0x7F and 0xFF), from the bit fields."""
    vals = np.empty(256)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_VALUES = e4m3_values()
_POS_CODES = np.arange(0x7F)          # 0x00 .. 0x7E: the non-negative finite codes, increasing
_POS_VALUES = _VALUES[_POS_CODES]


def e4m3_decode(codes):
    """uint8 codes -> float64 values."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y):
    """float values -> uint8 codes: nearest e4m3 value, ties to the even code, saturating at 448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # index of the largest code value <= a, then pick it or the next one
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, len(_POS_VALUES) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def quantize_blockwise_e4m3(x, block=64):
    """x [B, H, N, d] -> (codes uint8 [B, H, N, d], scale float32 [B, H, ceil(N / block)]).

    x ~= e4m3_decode(codes) * scale[row // block].
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = -(-N // block)
    codes = np.zeros((B, H, N, d), np.uint8)
    scale = np.ones((B, H, nb), np.float32)
    for i in range(nb):
        r = slice(i * block, min(N, (i + 1) * block))
        blk = x[:, :, r, :]
        amax = np.abs(blk).max(axis=(2, 3))                       # exact in float32
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scale[:, :, i] = s
        codes[:, :, r, :] = e4m3_encode((blk / s[:, :, None, None]).astype(np.float32))
    return codes, scale


def dequantize_blockwise_e4m3(codes, scale, block=64):
    """The float64 values the codes and scales stand for."""
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[2]
    rows = np.arange(N) // block
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, :, rows, None]


def attention_fwd_fp8(q_codes, q_scale, k_codes, k_scale, v, causal, scale, block=64):
    """The attention definition on the dequantised Q and K (float64) and V: (O, lse) like attention_fwd."""
    q = dequantize_blockwise_e4m3(q_codes, q_scale, block)
    k = dequantize_blockwise_e4m3(k_codes, k_scale, block)
    return attention_fwd(q, k, np.asarray(v, dtype=np.float64), causal, scale)
