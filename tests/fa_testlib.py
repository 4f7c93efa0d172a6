"""Shared helpers for the GPU parity tests (not a test module).

Inputs come from the seeded generator; expected values only from the CPU
oracle; the GPU side only through the libfa binding.
"""
from __future__ import annotations

import numpy as np

from fa_inputs import make_inputs

# Parity bars.
# bf16 storage, fp32 accumulation: max |gpu - oracle| <= 2e-2 and mean <= 2e-3
# on O (and on each gradient, relative to that gradient's max magnitude).
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
# fp32 storage and arithmetic: max |gpu - oracle| <= 1e-5 on O.
F32_MAX_ABS = 1e-5
# lse: each score is an fp32 sum of d exact products, which errs by up to about
# d * 2^-24 of the sum of the products' magnitudes, scale * sum_c |q_ic k_jc|
# (d <= 2^8: at most 2^-16 of it); lse moves by at most the largest score
# error of its row, and the fp32 row sum and the hardware exp2 / log2 add a
# few ulps more. Per row i:
#   |lse_i - LSE_i| <= 2^-16 * (1 + scale * max_j sum_c |q_ic| |k_jc|)
# (about 1.7e-4 for N(0,1) inputs at scale 1/sqrt(d), growing with the scores).
LSE_REL = 2.0 ** -16
# At head dim 64 the bf16 forward sums the probabilities after their rounding
# to bf16 (the values that also weight V), on the matrix unit. Round to
# nearest even changes each positive term by at most its unit roundoff 2^-8,
# so the row sum by at most a factor 1 -/+ 2^-8 and lse by -log(1 - 2^-8)
# (3.9e-3) more. Only the bf16 (and FP8) lse checks use lse_bound.
LSE_BF16_ROWSUM = -float(np.log1p(-(2.0 ** -8)))
ROWSUM_ON_MATRIX_D = 64


def _rowsum_term(d):
    return LSE_BF16_ROWSUM if d == ROWSUM_ON_MATRIX_D else 0.0


def lse_bound(q, k, scale):
    """Per-row lse bound [B, Hq, N] for q [B, Hq, N, d], k [B, Hkv, N, d] (query head h reads h // (Hq // Hkv))."""
    q = np.abs(np.asarray(q, np.float64))
    k = np.abs(np.asarray(k, np.float64))
    B, Hq, N, _ = q.shape
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            out[b, h] = (q[b, h] @ k[b, h // G].T).max(axis=1) if N else 0.0
    return LSE_REL * (1.0 + scale * out) + _rowsum_term(q.shape[-1])


def lse_bound_rows(q_rows, k_head, scale):
    """Per-row lse bound for selected query rows [R, d] of one head against its keys [N, d]."""
    a = np.abs(np.asarray(q_rows, np.float64)) @ np.abs(np.asarray(k_head, np.float64)).T
    return LSE_REL * (1.0 + scale * a.max(axis=1)) + _rowsum_term(np.asarray(q_rows).shape[-1])


def assert_lse_close(got, ref, bound, what="lse"):
    """|got - ref| <= bound per row; rows whose reference is -inf (no visible key) must be -inf too."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), dead), f"{what}: rows without keys differ"
    err = np.where(dead, 0.0, np.abs(np.where(dead, 0.0, got) - np.where(dead, 0.0, ref)))
    bound = np.broadcast_to(bound, err.shape)
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: error {err[i]:.3e} > bound {bound[i]:.3e} (|lse| {abs(ref[i]):.3f})")
    return float(err.max()) if err.size else 0.0


def torch_mod():
    import torch

    return torch


def to_device(inputs, name, dtype):
    """Upload one generated array (exact bf16 bits or fp32 values) to cuda:0."""
    torch = torch_mod()
    if dtype == "bf16":
        bits = inputs[name + "_bits"]
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(inputs[name])).to("cuda:0")


def to_f64(t):
    torch = torch_mod()
    return t.detach().to(torch.float64).cpu().numpy()


def errors(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_bf16_close(got, ref, what, scale=1.0):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    mx, mean = errors(got, ref)
    assert mx <= BF16_MAX_ABS * scale and mean <= BF16_MEAN_ABS * scale, (
        f"{what}: max {mx:.3e} (bar {BF16_MAX_ABS * scale:.3e}) mean {mean:.3e} (bar {BF16_MEAN_ABS * scale:.3e})")
    return mx, mean


def run_fwd(B, Hq, Hkv, N, d, causal, dtype="bf16", seed=0, q_mult=1.0, scale=None):
    """Generate inputs, run the libfa forward on cuda:0. Returns (inputs, o, lse) as fp64 numpy."""
    import tiled_online_softmax_fa_amd as fa

    inp = make_inputs(B, Hq, Hkv, N, d, dtype, seed, q_mult=q_mult)
    q, k, v = (to_device(inp, n, dtype) for n in ("q", "k", "v"))
    scale = scale if scale is not None else 1.0 / np.sqrt(d)
    fn = fa.fwd if dtype == "bf16" else fa.fwd_f32
    o, lse = fn(q, k, v, causal=causal, scale=scale)
    torch_mod().cuda.synchronize()
    return inp, to_f64(o), to_f64(lse), scale


def zero_grad_bounds(inp, scale):
    """Bounds on |dQ| and |dK| where the exact gradient is zero (e.g. one key).

    There dS = P o (dP - D) is exactly 0, and the kernels form dP - D as an fp32
    matrix product whose accumulator starts at -D, i.e. the difference of two
    fp32 sums of the same d products dO_ic v_jc (D from the stored O). Each sum
    errs by at most d 2^-24 times its sum of magnitudes, so
    |dS_ij| <= E_ij = 2 d 2^-24 sum_c |dO_ic| (|v_jc| + max_j' |v_j'c|) (P <= 1, |O| <= max |V|),
    and dQ = scale dS K, dK = scale dS^T Q carry it to
    |dQ_ic| <= scale sum_j E_ij |k_jc|,  |dK_jc| <= scale sum_i E_ij |q_ic|
    (per batch and head; grouped heads sum dK over the group; all heads are
    bounded with the group's K/V head).
    """
    q, k, v, dO = (np.abs(inp[n].astype(np.float64)) for n in ("q", "k", "v", "dO"))
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    bq, bk = np.zeros_like(q), np.zeros_like(k)
    for b in range(B):
        for h in range(Hq):
            vv, kk = v[b, h // G], k[b, h // G]
            E = 2 * d * 2.0 ** -24 * (dO[b, h] @ (vv + vv.max(axis=0)).T)  # [N queries, N keys]
            bq[b, h] = scale * E @ kk
            bk[b, h // G] += scale * E.T @ q[b, h]
    return bq, bk
