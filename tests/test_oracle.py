"""Pins for the CPU oracle: each test checks it against something other than itself.

Sources of truth: hand-derived closed forms (tests/golden), identities of the
definition softmax(scale * Q K^T) V, brute-force central finite differences, the
two online-softmax recurrences of the pages, and torch's CPU float64 softmax and
autograd (a library routine, used only here).
"""
import json
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import (
    attention_bwd,
    attention_bwd_head,
    attention_fwd,
    attention_fwd_rows,
    attention_probs,
    causal_tile_count,
    online_fwd_deferred,
    online_fwd_normalise_each_block,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_examples.json")

_TERM = re.compile(r"^\s*(-?\d+(?:/\d+)?)?\s*(\*)?\s*(ln\((\d+)\))?\s*$")


def _value(text):
    """Parse 'p/q', 'ln(n)', 'p/q*ln(n)' into a float."""
    m = _TERM.match(text)
    if not m or (m.group(1) is None and m.group(3) is None):
        raise ValueError(f"bad golden value {text!r}")
    coef = Fraction(m.group(1)) if m.group(1) else Fraction(1)
    if m.group(3):
        return float(coef) * math.log(int(m.group(4)))
    return float(coef)


def _arr(rows):
    return np.array([[_value(x) for x in row] for row in rows], dtype=np.float64)


def _vec(xs):
    return np.array([_value(x) for x in xs], dtype=np.float64)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- golden, by hand
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["forward"], ids=lambda c: c["name"])
@pytest.mark.parametrize("causal", [False, True])
def test_golden_forward(case, causal):
    q, k, v = (_arr(case[n])[None, None] for n in ("q", "k", "v"))
    want = case["causal" if causal else "noncausal"]
    O, lse = attention_fwd(q, k, v, causal, _value(case["scale"]))
    np.testing.assert_allclose(O[0, 0], _arr(want["O"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], _vec(want["lse"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", _golden()["backward"], ids=lambda c: c["name"])
@pytest.mark.parametrize("causal", [False, True])
def test_golden_backward(case, causal):
    q, k, v, dO = (_arr(case[n])[None, None] for n in ("q", "k", "v", "dO"))
    want = case["causal" if causal else "noncausal"]
    scale = _value(case["scale"])
    O, _ = attention_fwd(q, k, v, causal, scale)
    np.testing.assert_allclose(O[0, 0], _arr(want["O"]), atol=1e-14)
    dQ, dK, dV = attention_bwd(q, k, v, dO, causal, scale)
    for got, name in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        np.testing.assert_allclose(got[0, 0], _arr(want[name]), rtol=0, atol=1e-14, err_msg=name)


# ---------------------------------------------------------------- identities
shapes = st.tuples(st.integers(1, 2), st.integers(1, 3), st.integers(1, 9), st.integers(1, 5))


@settings(max_examples=40, deadline=None)
@given(shapes, st.booleans(), st.integers(0, 2**31 - 1))
def test_values_all_one_give_output_one(shape, causal, seed):
    B, H, N, d = shape
    rng = np.random.default_rng(seed)
    q, k = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    O, _ = attention_fwd(q, k, np.ones((B, H, N, d)), causal, 0.7)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-14)


@settings(max_examples=40, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1))
def test_zero_queries_give_mean_of_values(shape, seed):
    B, H, N, d = shape
    rng = np.random.default_rng(seed)
    k, v = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    q = np.zeros((B, H, N, d))
    O, lse = attention_fwd(q, k, v, False, 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(N), atol=1e-14)
    O, lse = attention_fwd(q, k, v, True, 0.5)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(O, prefix_mean, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), atol=1e-14)


@settings(max_examples=40, deadline=None)
@given(shapes, st.booleans(), st.integers(0, 2**31 - 1))
def test_probability_rows_sum_to_one_and_respect_mask(shape, causal, seed):
    B, H, N, d = shape
    rng = np.random.default_rng(seed)
    P = attention_probs(_rand(rng, B, H, N, d) * 3, _rand(rng, B, H, N, d), causal, 1.0)
    np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-14)
    assert (P >= 0).all()
    if causal:
        assert (P[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0).all()


def test_single_key_gives_value_and_score():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 3, 1, 4), _rand(rng, 2, 3, 1, 4), _rand(rng, 2, 3, 1, 4)
    for causal in (False, True):
        O, lse = attention_fwd(q, k, v, causal, 0.3)
        np.testing.assert_allclose(O, v, atol=1e-15)
        np.testing.assert_allclose(lse, 0.3 * np.sum(q * k, axis=-1), atol=1e-15)


def test_two_keys_closed_form_sigmoid():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 1, 2, 3), _rand(rng, 1, 1, 2, 3), _rand(rng, 1, 1, 2, 3)
    scale = 0.9
    s = scale * np.einsum("id,jd->ij", q[0, 0], k[0, 0])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    want = np.stack([sig(s[i, 0] - s[i, 1]) * v[0, 0, 0] + sig(s[i, 1] - s[i, 0]) * v[0, 0, 1] for i in range(2)])
    O, lse = attention_fwd(q, k, v, False, scale)
    np.testing.assert_allclose(O[0, 0], want, atol=1e-14)
    want_lse = [max(s[i]) + math.log1p(math.exp(-abs(s[i, 0] - s[i, 1]))) for i in range(2)]
    np.testing.assert_allclose(lse[0, 0], want_lse, atol=1e-14)


@settings(max_examples=25, deadline=None)
@given(st.integers(1, 2), st.sampled_from([(2, 1), (4, 2), (6, 3), (8, 1)]), st.integers(1, 7), st.integers(1, 4),
       st.booleans(), st.integers(0, 2**31 - 1))
def test_grouped_heads_equal_repeated_heads(B, heads, N, d, causal, seed):
    Hq, Hkv = heads
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    q, k, v, dO = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hq, N, d)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    O, lse = attention_fwd(q, k, v, causal, 0.6)
    Or, lser = attention_fwd(q, kr, vr, causal, 0.6)
    np.testing.assert_allclose(O, Or, atol=1e-14)
    np.testing.assert_allclose(lse, lser, atol=1e-14)
    dQ, dK, dV = attention_bwd(q, k, v, dO, causal, 0.6)
    dQr, dKr, dVr = attention_bwd(q, kr, vr, dO, causal, 0.6)
    np.testing.assert_allclose(dQ, dQr, atol=1e-13)
    np.testing.assert_allclose(dK, dKr.reshape(B, Hkv, G, N, d).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dV, dVr.reshape(B, Hkv, G, N, d).sum(axis=2), atol=1e-13)


def test_permutations():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4)
    O, lse = attention_fwd(q, k, v, False, 0.8)
    perm = rng.permutation(9)
    O2, lse2 = attention_fwd(q, k[:, :, perm], v[:, :, perm], False, 0.8)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)
    O3, lse3 = attention_fwd(q[:, :, perm], k, v, False, 0.8)
    np.testing.assert_allclose(O3, O[:, :, perm], atol=1e-14)
    np.testing.assert_allclose(lse3, lse[:, :, perm], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 2, 2, 8, 5), _rand(rng, 2, 2, 8, 5), _rand(rng, 2, 2, 8, 5)
    c = _rand(rng, 5)
    O, lse = attention_fwd(q, k, v, causal, 0.4)
    O2, lse2 = attention_fwd(q, k + c, v, causal, 0.4)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 0.4 * np.einsum("bhnd,d->bhn", q, c), atol=1e-13)


def test_rows_variant_matches_full():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 2, 4, 13, 3), _rand(rng, 2, 2, 13, 3), _rand(rng, 2, 2, 13, 3)
    for causal in (False, True):
        O, lse = attention_fwd(q, k, v, causal, 0.5)
        rows = np.array([0, 5, 12, 7])
        Or, lser = attention_fwd_rows(q, k, v, causal, 0.5, 1, 3, rows)
        np.testing.assert_allclose(Or, O[1, 3, rows], atol=1e-15)
        np.testing.assert_allclose(lser, lse[1, 3, rows], atol=1e-15)


def test_empty_sequence():
    z = np.zeros((1, 2, 0, 4))
    O, lse = attention_fwd(z, z, z, True, 1.0)
    assert O.shape == (1, 2, 0, 4) and lse.shape == (1, 2, 0)


def test_peaky_scores_are_finite_and_pick_the_argmax():
    # max subtraction: scores near 1e4 would overflow exp() without it
    q = np.array([[[[100.0, 0.0]]]])
    k = np.array([[[[100.0, 0.0], [99.0, 0.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    O, lse = attention_fwd(np.repeat(q, 2, axis=2), k, v, False, 1.0)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    w = 1.0 / (1.0 + math.exp(-100.0))
    np.testing.assert_allclose(O[0, 0, 0], [w, 1 - w], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 1e4 + math.log1p(math.exp(-100.0)), rtol=1e-15)


# ---------------------------------------------------------------- online recurrences (the pages' algorithm)
@settings(max_examples=30, deadline=None)
@given(st.integers(1, 2), st.sampled_from([(1, 1), (2, 1), (4, 2)]), st.integers(1, 12), st.integers(1, 5),
       st.booleans(), st.sampled_from([1, 2, 3, 5, 64]), st.sampled_from([1, 2, 3, 5, 64]), st.integers(0, 2**31 - 1))
def test_online_recurrences_equal_the_definition(B, heads, N, d, causal, bq, bk, seed):
    Hq, Hkv = heads
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, B, Hq, N, d) * 2, _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    O, lse = attention_fwd(q, k, v, causal, 0.7)
    vmax = np.abs(v).max()
    for fn in (online_fwd_normalise_each_block, online_fwd_deferred):
        O2, lse2 = fn(q, k, v, causal, 0.7, bq, bk)
        np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12 * vmax, err_msg=fn.__name__)
        np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12, err_msg=fn.__name__)


# ---------------------------------------------------------------- backward: finite differences, invariants
def _loss(q, k, v, dO, causal, scale):
    return float(np.sum(dO * attention_fwd(q, k, v, causal, scale)[0]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 2), (5, 3), (8, 4)])
def test_backward_matches_finite_differences(causal, N, d):
    rng = np.random.default_rng(100 + N)
    q, k, v, dO = (_rand(rng, 1, 1, N, d) for _ in range(4))
    scale = 0.8
    dQ, dK, dV = attention_bwd(q, k, v, dO, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], dO, causal, scale)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], dO, causal, scale)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=name)


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 10), st.integers(1, 5), st.booleans(), st.integers(0, 2**31 - 1))
def test_backward_invariants(N, d, causal, seed):
    rng = np.random.default_rng(seed)
    q, k, v, dO = (_rand(rng, 1, 1, N, d) for _ in range(4))
    dQ, dK, dV = attention_bwd(q, k, v, dO, causal, 0.9)
    # shifting every key by one vector leaves every softmax row unchanged -> keys' gradients sum to 0
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    # each probability row sums to one -> dV summed over keys equals dO summed over queries
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=2), atol=1e-12)
    if causal:
        # row 0 sees only key 0: dP - D = dO.v_0 - dO.O_0 with O_0 = v_0, zero up to the
        # rounding of two d-term fp64 dot products
        tol = 8 * d * np.finfo(np.float64).eps * float(np.abs(dO[0, 0, 0]).sum() * np.abs(v[0, 0, 0]).max() + 1)
        np.testing.assert_allclose(dQ[0, 0, 0], 0.0, atol=tol * float(np.abs(k[0, 0, 0]).max() + 1))
        P = attention_probs(q, k, True, 0.9)[0, 0]
        np.testing.assert_allclose(dV[0, 0, N - 1], P[N - 1, N - 1] * dO[0, 0, N - 1], atol=1e-13)
    # equal value rows -> output independent of q and k
    v_eq = np.broadcast_to(v[:, :, :1], v.shape).copy()
    dQ2, dK2, _ = attention_bwd(q, k, v_eq, dO, causal, 0.9)
    np.testing.assert_allclose(dQ2, 0.0, atol=1e-12)
    np.testing.assert_allclose(dK2, 0.0, atol=1e-12)


def test_row_term_identity():
    # sum_c dO_ic O_ic == sum_j P_ij dP_ij, dP = dO V^T
    rng = np.random.default_rng(11)
    q, k, v, dO = (_rand(rng, 1, 1, 7, 3) for _ in range(4))
    for causal in (False, True):
        P = attention_probs(q, k, causal, 1.1)[0, 0]
        O = attention_fwd(q, k, v, causal, 1.1)[0][0, 0]
        dP = dO[0, 0] @ v[0, 0].T
        np.testing.assert_allclose(np.sum(dO[0, 0] * O, axis=1), np.sum(P * dP, axis=1), atol=1e-13)


def test_bwd_head_matches_batched():
    rng = np.random.default_rng(12)
    q, k, v, dO = (_rand(rng, 2, 2, 6, 3) for _ in range(4))
    dQ, dK, dV = attention_bwd(q, k, v, dO, True, 0.5)
    g = attention_bwd_head(q[1, 0], k[1, 0], v[1, 0], dO[1, 0], True, 0.5)
    for a, b in zip(g, (dQ[1, 0], dK[1, 0], dV[1, 0])):
        np.testing.assert_allclose(a, b, atol=1e-15)


# ---------------------------------------------------------------- library cross-check (torch CPU float64)
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_cpu_float64(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    B, Hq, Hkv, N, d = 2, 4, 2, 11, 6
    q, k, v, dO = _rand(rng, B, Hq, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hq, N, d)
    scale = 0.37
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    kk, vv = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    lse_t = torch.logsumexp(s, dim=-1)
    o_t = torch.matmul(torch.softmax(s, dim=-1), vv)
    o_t.backward(torch.tensor(dO))
    O, lse = attention_fwd(q, k, v, causal, scale)
    np.testing.assert_allclose(O, o_t.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(lse, lse_t.detach().numpy(), atol=1e-13)
    dQ, dK, dV = attention_bwd(q, k, v, dO, causal, scale)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------- causal tile skipping count
def test_causal_tile_count_closed_form_and_skip_share():
    # square tiles: T(T+1)/2 of T^2 tiles hold a visible entry
    for T in (1, 2, 5, 16, 32):
        assert causal_tile_count(64 * T, 64, 64) == T * (T + 1) // 2
    # T = 16: skipped share (T-1)/(2T) = 46.9 %, the page's "about 47 %" (Flash Attention V3技术解析, 2.1)
    skipped = 1 - causal_tile_count(1024, 64, 64) / 16**2
    assert abs(skipped - 0.46875) < 1e-12
    # ragged: N = 100 with 64-tiles: tiles (0,0), (1,0), (1,1)
    assert causal_tile_count(100, 64, 64) == 3
    # rectangular 128 x 64 tiles on N = 4096: query tile t covers key tiles 0..2t+1
    assert causal_tile_count(4096, 128, 64) == sum(2 * t + 2 for t in range(32))
