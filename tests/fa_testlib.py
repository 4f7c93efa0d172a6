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
# lse is computed from fp32 scores of exact bf16/fp32 inputs and an fp32 row
# sum that never goes through bf16: its error is a few fp32 ulps of |scale*s|
# (|scale*s| < 40 here) plus the 1-2 ulp error of the hardware exp2/log2, far
# below this bound, which is kept well above that and well below any real bug.
LSE_MAX_ABS = 1e-4


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
