"""Backward parity: libfa dQ, dK, dV on the GPU against the fp64 CPU oracle."""
import sys

import numpy as np
import pytest

from fa_inputs import WORKLOADS, make_inputs, make_workload_inputs
from fa_testlib import assert_bf16_close, to_device, to_f64, torch_mod, zero_grad_bounds
from oracle import attention_bwd

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(inp, causal, scale):
    import tiled_online_softmax_fa_amd as fa

    q, k, v, dO = (to_device(inp, n, "bf16") for n in ("q", "k", "v", "dO"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dO, causal=causal, scale=scale)
    torch_mod().cuda.synchronize()
    return dq, dk, dv


def _check_grads(got, ref, what, inp=None, scale=None):
    worst = []
    zero_bounds = None
    for name, gt, rf in zip(("dQ", "dK", "dV"), got, ref):
        s = float(np.abs(rf).max())
        if s == 0.0:  # an exactly-zero gradient (e.g. a single key): fp32 rounding of dP - D only
            assert inp is not None, f"{what} {name}: zero reference needs the inputs for its bound"
            if zero_bounds is None:
                zero_bounds = zero_grad_bounds(inp, scale)
            bound = zero_bounds[0] if name == "dQ" else zero_bounds[1]
            assert name != "dV" and np.all(np.abs(gt) <= bound), (
                f"{what} {name}: |got| up to {np.abs(gt).max():.3e} where the exact gradient is 0 "
                f"(bound {bound.max():.3e})")
            worst.append(f"{name} {np.abs(gt).max():.1e} (exact 0)")
            continue
        mx, mean = assert_bf16_close(gt, rf, f"{what} {name}", scale=s)
        worst.append(f"{name} max {mx / s:.1e} mean {mean / s:.1e}")
    _say("  " + ", ".join(worst))


SMALL = [
    (1, 2, 2, 300, 64, False),
    (1, 2, 2, 300, 64, True),
    (1, 2, 2, 300, 128, False),
    (1, 2, 2, 300, 128, True),
    (2, 4, 2, 257, 128, True),
    (1, 4, 1, 200, 64, True),
    (1, 8, 1, 130, 128, False),
    (1, 1, 1, 1, 128, True),
    (1, 2, 2, 17, 64, False),
    (1, 2, 2, 1000, 128, True),
    # head dim 256 (64-key and 32-query tiles in dK/dV, 128-query tiles in dQ)
    (1, 2, 2, 300, 256, False),
    (1, 2, 2, 300, 256, True),
    (2, 4, 2, 257, 256, True),
    (1, 4, 1, 130, 256, False),
    (1, 1, 1, 1, 256, True),
    (1, 2, 2, 65, 256, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", SMALL)
def test_bwd_small(B, Hq, Hkv, N, d, causal):
    _say(f"bwd B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=N + 3 * d, backward=True)
    scale = d ** -0.5
    got = [to_f64(t) for t in _run(inp, causal, scale)]
    ref = attention_bwd(inp["q"], inp["k"], inp["v"], inp["dO"], causal, scale)
    _check_grads(got, ref, "bwd", inp, scale)


def test_bwd_peaky():
    _say("bwd peaky q x 8")
    inp = make_inputs(1, 4, 2, 500, 128, "bf16", seed=21, backward=True, q_mult=8.0)
    got = [to_f64(t) for t in _run(inp, True, 128 ** -0.5)]
    ref = attention_bwd(inp["q"], inp["k"], inp["v"], inp["dO"], True, 128 ** -0.5)
    _check_grads(got, ref, "bwd peaky")


def full_grad_check(got, inp, causal, scale, what):
    """Every element of dQ, dK, dV against the oracle, one (batch, K/V group) at a time.

    Bars per tensor, relative to that tensor's largest reference magnitude:
    max |g - ref| <= 2e-2 max|ref| and the mean over all elements <= 2e-3 max|ref|.
    """
    dq, dk, dv = got
    for t in got:
        assert np.isfinite(t).all(), f"{what}: non-finite gradient"
    B, Hq, N, d = dq.shape
    Hkv = dk.shape[1]
    G = Hq // Hkv
    err_max = [0.0, 0.0, 0.0]
    err_sum = [0.0, 0.0, 0.0]
    ref_max = [0.0, 0.0, 0.0]
    for b in range(B):
        for hk in range(Hkv):
            qs = (slice(b, b + 1), slice(hk * G, (hk + 1) * G))
            ks = (slice(b, b + 1), slice(hk, hk + 1))
            ref = attention_bwd(inp["q"][qs], inp["k"][ks], inp["v"][ks], inp["dO"][qs], causal, scale)
            for i, (g, r) in enumerate(zip((dq[qs], dk[ks], dv[ks]), ref)):
                e = np.abs(g - r)
                err_max[i] = max(err_max[i], float(e.max()))
                err_sum[i] += float(e.sum())
                ref_max[i] = max(ref_max[i], float(np.abs(r).max()))
    parts = []
    for i, name in enumerate(("dQ", "dK", "dV")):
        n = (dq, dk, dv)[i].size
        rel_max, rel_mean = err_max[i] / ref_max[i], err_sum[i] / n / ref_max[i]
        parts.append(f"{name} max {rel_max:.1e} mean {rel_mean:.1e}")
        assert rel_max <= 2e-2 and rel_mean <= 2e-3, f"{what} {name}: max {rel_max:.3e} mean {rel_mean:.3e} (relative)"
    _say(f"  {what} whole tensors: " + ", ".join(parts))


def test_bwd_workload_causal_4096():
    w = WORKLOADS["bwd_causal_bf16_b2h16n4096d128"]
    _say(f"workload {w.name}: every element of dQ, dK, dV")
    inp = make_workload_inputs(w)
    got = [to_f64(t) for t in _run(inp, w.causal, w.scale)]
    full_grad_check(got, inp, w.causal, w.scale, w.name)
    # extra invariants at any size: keys' gradients sum to zero (softmax is shift
    # invariant) and sum_j dV_j = sum_i dO_i (probability rows sum to one)
    dq, dk, dv = got
    dO = inp["dO"].astype(np.float64)
    sdv = dv.sum(axis=2)
    np.testing.assert_allclose(sdv, dO.sum(axis=2), atol=2e-2 * np.abs(sdv).max() + 0.25)
    assert np.abs(dk.sum(axis=2)).max() <= 2e-2 * np.abs(dk).max() * 64


def test_bwd_d256_causal_4096():
    # B2 H16 N4096 d256 causal: every element of the three gradients
    from fa_inputs import Workload

    w = Workload("bwd_causal_bf16_b2h16n4096d256", 2, 16, 16, 4096, 256, "bf16", True, backward=True, seed=61)
    _say(f"workload {w.name}: every element of dQ, dK, dV")
    inp = make_workload_inputs(w)
    got = [to_f64(t) for t in _run(inp, w.causal, w.scale)]
    full_grad_check(got, inp, w.causal, w.scale, w.name)


@pytest.mark.parametrize("B,Hq,Hkv,N,causal", [(1, 16, 2, 1024, True), (4, 16, 4, 2048, False)])
def test_bwd_gqa_group_parts(B, Hq, Hkv, N, causal):
    # B1 Hq16 Hkv2 N1024: 16 dK/dV workgroups, so the 8 query heads of each K/V head are split into 8 parts whose
    # fp32 partial sums a reduction adds up; B4 Hq16 Hkv4: 256 workgroups, no split. Every element checked.
    _say(f"bwd GQA B{B} Hq{Hq} Hkv{Hkv} N{N} d128 causal={causal}: every element")
    inp = make_inputs(B, Hq, Hkv, N, 128, "bf16", seed=N + Hq + B, backward=True)
    scale = 128 ** -0.5
    got = [to_f64(t) for t in _run(inp, causal, scale)]
    full_grad_check(got, inp, causal, scale, f"GQA B{B} Hq{Hq} Hkv{Hkv} N{N}")


def test_bwd_gqa_medium():
    _say("bwd GQA B1 Hq8 Hkv2 N777 d128 causal")
    inp = make_inputs(1, 8, 2, 777, 128, "bf16", seed=31, backward=True)
    got = [to_f64(t) for t in _run(inp, True, 128 ** -0.5)]
    ref = attention_bwd(inp["q"], inp["k"], inp["v"], inp["dO"], True, 128 ** -0.5)
    _check_grads(got, ref, "bwd gqa")


@pytest.mark.parametrize("d", [128, 256])
def test_bwd_bitwise_repeatable(d):
    # no atomics anywhere in the backward: every output is bitwise repeatable
    inp = make_inputs(1, 4, 4, 600, d, "bf16", seed=41, backward=True)
    a = _run(inp, True, d ** -0.5)
    b = _run(inp, True, d ** -0.5)
    torch = torch_mod()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_autograd_function():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    inp = make_inputs(1, 2, 2, 150, 64, "bf16", seed=51, backward=True)
    q, k, v, dO = (to_device(inp, n, "bf16").requires_grad_(n != "dO") for n in ("q", "k", "v", "dO"))
    o = fa.flash_attn(q, k, v, causal=True)
    o.backward(dO)
    torch.cuda.synchronize()
    ref = attention_bwd(inp["q"], inp["k"], inp["v"], inp["dO"], True, 64 ** -0.5)
    _check_grads([to_f64(t.grad) for t in (q, k, v)], ref, "autograd")


def test_bwd_errors():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    x = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros((1, 2, 8), dtype=torch.float32, device="cuda:0")
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ValueError):
        fa.bwd(x, x, x, x, lse, x, workspace=small_ws)
    z = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    zl = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = fa.bwd(z, z, z, z, zl, z)
    assert dq.shape == z.shape


@pytest.mark.parametrize("scale,causal,d", [(0.37, True, 128), (1.0, False, 64), (0.02, True, 256)])
def test_bwd_other_scales(scale, causal, d):
    # scale enters both the exponent and the dQ / dK factor: a mix-up shows only away from 1/sqrt(d)
    _say(f"bwd scale {scale} causal={causal} d{d}")
    inp = make_inputs(1, 4, 2, 300, d, "bf16", seed=71, backward=True)
    got = [to_f64(t) for t in _run(inp, causal, scale)]
    ref = attention_bwd(inp["q"], inp["k"], inp["v"], inp["dO"], causal, scale)
    _check_grads(got, ref, f"bwd scale {scale}")
