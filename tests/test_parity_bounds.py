"""CPU checks of the derived parity bounds themselves (no GPU): the bf16 row-sum term of the lse bound is the
largest change that rounding the probabilities to bf16 (round to nearest even) can make to log(sum p), it is
nearly reached, and the bound carries it only at the head dim where the forward sums rounded probabilities."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from fa_inputs import bf16_round  # noqa: E402
from fa_testlib import LSE_BF16_ROWSUM, LSE_REL, ROWSUM_ON_MATRIX_D, lse_bound, lse_bound_rows  # noqa: E402

U_BF16 = 2.0 ** -8  # unit roundoff of an 8-bit significand


def test_bf16_rounding_moves_each_positive_value_by_at_most_the_unit_roundoff():
    rng = np.random.default_rng(11)
    x = np.ldexp(rng.uniform(1.0, 2.0, 200_000), rng.integers(-60, 2, 200_000)).astype(np.float32)
    # values just below and above the halfway points between neighbouring bf16 numbers
    half = np.ldexp(1.0 + (2 * rng.integers(0, 128, 4096) + 1) * 2.0 ** -8, rng.integers(-30, 1, 4096))
    x = np.concatenate([x, np.nextafter(half, 0).astype(np.float32), np.nextafter(half, 4).astype(np.float32),
                        half.astype(np.float32)])
    r = bf16_round(x).astype(np.float64)
    rel = np.abs(r - x.astype(np.float64)) / x.astype(np.float64)
    assert rel.max() <= U_BF16
    assert rel.max() > 0.99 * U_BF16  # the halfway cases come close


def test_lse_rowsum_term_bounds_the_rounded_sum_and_is_nearly_reached():
    assert np.isclose(LSE_BF16_ROWSUM, -np.log1p(-U_BF16))
    rng = np.random.default_rng(5)
    worst = 0.0
    for n in (1, 7, 64, 4096):
        for _ in range(50):
            p = np.exp2(np.minimum(rng.normal(0.0, 3.0, n), 0.0)).astype(np.float32)  # 2^(s - m) with s <= m
            d = abs(np.log(bf16_round(p).astype(np.float64).sum()) - np.log(p.astype(np.float64).sum()))
            assert d <= LSE_BF16_ROWSUM
            worst = max(worst, d)
    # adversarial row: every probability just under a halfway point rounds down by nearly 2^-8 of itself
    p = np.full(4096, np.nextafter(np.float32(1.0 + 2.0 ** -8), np.float32(0)), np.float32)
    d = abs(np.log(bf16_round(p).astype(np.float64).sum()) - np.log(p.astype(np.float64).sum()))
    assert 0.99 * LSE_BF16_ROWSUM < d <= LSE_BF16_ROWSUM
    assert worst < d


def test_lse_bound_adds_the_term_only_at_the_rowsum_head_dim():
    rng = np.random.default_rng(3)
    for d in (64, 128, 256):
        q = rng.normal(size=(1, 2, 16, d))
        k = rng.normal(size=(1, 1, 16, d))
        s = d ** -0.5
        base = LSE_REL * (1.0 + s * (np.abs(q[0, 0]) @ np.abs(k[0, 0]).T).max(axis=1))
        extra = LSE_BF16_ROWSUM if d == ROWSUM_ON_MATRIX_D else 0.0
        np.testing.assert_allclose(lse_bound(q, k, s)[0, 0], base + extra, rtol=1e-12)
        np.testing.assert_allclose(lse_bound_rows(q[0, 0], k[0, 0], s), base + extra, rtol=1e-12)
