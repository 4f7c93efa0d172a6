"""The seeded input generator: determinism and bit-exact bf16 round-to-nearest-even."""
import numpy as np
import pytest

from fa_inputs import WORKLOADS, bf16_bits_to_f32, bf16_round_bits, make_inputs


def test_same_seed_same_inputs_and_draw_order():
    a = make_inputs(1, 2, 1, 5, 4, "f32", seed=3, backward=True)
    b = make_inputs(1, 2, 1, 5, 4, "f32", seed=3, backward=True)
    for n in ("q", "k", "v", "dO"):
        np.testing.assert_array_equal(a[n], b[n])
    rng = np.random.default_rng(3)
    np.testing.assert_array_equal(a["q"], rng.standard_normal((1, 2, 5, 4), dtype=np.float32))
    np.testing.assert_array_equal(a["k"], rng.standard_normal((1, 1, 5, 4), dtype=np.float32))


def test_bf16_rounding_matches_torch_bit_for_bit():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000, dtype=np.float32) * np.float32(10) ** rng.integers(-40, 38, 100000).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3.4e38, 1.17549435e-38], dtype=np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_round_bits(x), want)


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to the even mantissa (1.0)
    x = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8)], dtype=np.float32)
    got = bf16_bits_to_f32(bf16_round_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0 + 2.0**-6, -1.0], dtype=np.float32))


def test_bf16_nan_stays_nan():
    x = np.array([np.nan], dtype=np.float32)
    assert np.isnan(bf16_bits_to_f32(bf16_round_bits(x))).all()


def test_bf16_inputs_are_exact_bf16_values():
    w = make_inputs(2, 2, 2, 7, 8, "bf16", seed=1)
    for n in ("q", "k", "v"):
        assert w[n].dtype == np.float32
        np.testing.assert_array_equal(bf16_round_bits(w[n]), w[n + "_bits"])
        assert (w[n].view(np.uint32) & 0xFFFF == 0).all()


def test_workload_table():
    assert len(WORKLOADS) == 5
    w = WORKLOADS["fwd_causal_bf16_b2h16n4096d128"]
    assert (w.B, w.Hq, w.Hkv, w.N, w.d, w.causal) == (2, 16, 16, 4096, 128, True)
    assert abs(w.scale - 128 ** -0.5) < 1e-15
    g = WORKLOADS["fwd_causal_gqa_bf16_b2hq64hkv8n4096d128"]
    assert (g.Hq, g.Hkv) == (64, 8)
    assert WORKLOADS["fwd_f32_b1h1n256d64"].scale == 0.125
    assert WORKLOADS["bwd_causal_bf16_b2h16n4096d128"].backward
