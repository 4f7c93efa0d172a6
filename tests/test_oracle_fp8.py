"""Pins of the FP8 oracle (CPU only): e4m3 code values from the format's definition,
round-to-nearest-even encoding, block-wise quantisation bounds, and attention on
exactly representable inputs. See oracle/fp8.py for the passages followed."""
import numpy as np
import pytest

from oracle import (E4M3_MAX, attention_fwd, attention_fwd_fp8, dequantize_blockwise_e4m3, e4m3_decode,
                    e4m3_encode, e4m3_values, quantize_blockwise_e4m3)


def test_code_values_named_by_the_format():
    v = e4m3_values()
    # (code, value) pairs that follow from 1 sign, 4 exponent (bias 7), 3 mantissa bits
    for code, val in ((0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                      (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0)):
        assert v[code] == val, hex(code)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..0x7E increase
    assert np.isfinite(v).sum() == 254 and E4M3_MAX == pos.max()
    # spacing: 2^-9 in the subnormals and the first binade, relative 1/8 above
    assert np.all(np.diff(pos[:16]) == 2.0 ** -9)


def test_encode_round_trip_and_ties_to_even():
    v = e4m3_values()
    finite = np.array([c for c in range(256) if np.isfinite(v[c]) and c != 0x80])
    assert np.array_equal(e4m3_encode(v[finite]), finite.astype(np.uint8))
    pos = v[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2                       # exact in float64
    codes = e4m3_encode(mid)
    lower = np.arange(0x7E)
    expect = np.where(lower % 2 == 0, lower, lower + 1)  # the even neighbour
    assert np.array_equal(codes, expect.astype(np.uint8))
    step = np.diff(pos)
    assert np.array_equal(e4m3_encode(mid - step / 8), lower.astype(np.uint8))
    assert np.array_equal(e4m3_encode(mid + step / 8), (lower + 1).astype(np.uint8))
    assert e4m3_encode(np.array([1e6, -500.0, 460.0]))[0] == 0x7E
    assert list(e4m3_encode(np.array([-500.0, 460.0]))) == [0xFE, 0x7E]
    # the sign survives rounding to zero (IEEE 754): -0 is code 0x80
    assert list(e4m3_encode(np.array([-1e-30, -0.0, 0.0, 1e-30]))) == [0x80, 0x80, 0x00, 0x00]


@pytest.mark.parametrize("N,d", [(64, 8), (130, 16), (1, 4)])
def test_blockwise_quantisation_bounds(N, d):
    rng = np.random.default_rng(N)
    x = (rng.standard_normal((2, 3, N, d)) * rng.uniform(0.01, 100, (2, 3, 1, 1))).astype(np.float32)
    x[0, 0, : min(N, 64)] = 0.0                          # an all-zero block: scale 1, codes 0
    codes, scale = quantize_blockwise_e4m3(x)
    assert scale.shape == (2, 3, -(-N // 64)) and scale.dtype == np.float32
    assert scale[0, 0, 0] == 1.0 and np.all(codes[0, 0, : min(N, 64)] == 0)
    deq = dequantize_blockwise_e4m3(codes, scale)
    s_row = scale.astype(np.float64)[:, :, np.arange(N) // 64, None]
    err = np.abs(deq - x)
    # half a unit in the last place: 2^-4 relative for normal codes, 2^-10 * scale below 2^-6 * scale
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, s_row * 2.0 ** -10) * (1 + 1e-6))
    # each non-zero block's largest magnitude lands on the largest code
    for b in range(2):
        for h in range(3):
            for i in range(scale.shape[2]):
                blk = codes[b, h, i * 64:(i + 1) * 64]
                if np.abs(x[b, h, i * 64:(i + 1) * 64]).max() > 0:
                    assert (blk & 0x7F).max() == 0x7E


def test_power_of_two_rescaling_of_a_block_keeps_its_codes():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 2, 128, 8)).astype(np.float32)
    c1, s1 = quantize_blockwise_e4m3(x)
    y = x.copy()
    y[:, :, 64:] *= np.float32(8.0)
    c2, s2 = quantize_blockwise_e4m3(y)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2[:, :, 1], s1[:, :, 1] * 8) and np.array_equal(s2[:, :, 0], s1[:, :, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_attention_on_representable_inputs_is_the_definition(causal):
    # codes drawn at random (finite, moderate) with scale 1: the dequantised values are exact
    rng = np.random.default_rng(5)
    B, Hq, Hkv, N, d = 1, 4, 2, 100, 16
    v = e4m3_values()
    ok = np.array([c for c in range(256) if np.isfinite(v[c]) and abs(v[c]) <= 4])
    qc = rng.choice(ok, (B, Hq, N, d)).astype(np.uint8)
    kc = rng.choice(ok, (B, Hkv, N, d)).astype(np.uint8)
    vv = rng.standard_normal((B, Hkv, N, d))
    ones_q = np.ones((B, Hq, 2), np.float32)
    ones_k = np.ones((B, Hkv, 2), np.float32)
    O, L = attention_fwd_fp8(qc, ones_q, kc, ones_k, vv, causal, 0.25)
    O2, L2 = attention_fwd(e4m3_decode(qc), e4m3_decode(kc), vv, causal, 0.25)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    # a block scale of 2 on q is the same as doubling the softmax scale for those rows
    two = ones_q.copy()
    two[:, :, 1] = 2.0
    O3, L3 = attention_fwd_fp8(qc, two, kc, ones_k, vv, causal, 0.25)
    Oa, La = attention_fwd(e4m3_decode(qc), e4m3_decode(kc), vv, causal, 0.5)
    np.testing.assert_allclose(O3[:, :, 64:], Oa[:, :, 64:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L3[:, :, 64:], La[:, :, 64:], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(O3[:, :, :64], O[:, :, :64])
