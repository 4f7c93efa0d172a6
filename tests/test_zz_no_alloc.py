"""The allocation-free backward (fa_bwd_noalloc, for callers that cannot allocate device
memory) against fa_bwd on the same inputs: two calls in a row, the second smaller, so
the second reuses the scratch the first left behind."""
import sys

import numpy as np
import pytest

from fa_inputs import make_inputs
from fa_testlib import to_device, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(B, Hq, Hkv, N, d, causal, seed):
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=seed, backward=True)
    q, k, v, dO = (to_device(inp, n, "bf16") for n in ("q", "k", "v", "dO"))
    scale = d ** -0.5
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    ref = fa.bwd(q, k, v, o, lse, dO, causal=causal, scale=scale)
    # outputs start as NaN so that an element the call does not write shows up
    got = tuple(torch.full_like(t, float("nan")) for t in ref)
    torch.cuda.synchronize()
    before = (torch.cuda.memory_allocated(), torch.cuda.memory_reserved())
    fa.bwd_noalloc(q, k, v, o, lse, dO, *got, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert (torch.cuda.memory_allocated(), torch.cuda.memory_reserved()) == before
    return ref, got


def test_bwd_noalloc_matches_bwd_on_two_calls():
    torch = torch_mod()
    import tiled_online_softmax_fa_amd as fa

    cases = [
        # grouped heads on a small grid: 16 parts of fp32 partial dK/dV sums, 24 MiB of the scratch
        (1, 16, 2, 768, 128, True, 5),
        # smaller, no split parts: the row terms only, over stale scratch from the first call
        (1, 4, 4, 300, 64, False, 6),
    ]
    for B, Hq, Hkv, N, d, causal, seed in cases:
        need = fa.bwd_workspace_bytes(B, Hq, Hkv, N, d)
        assert need <= fa.BWD_NOALLOC_SCRATCH_BYTES
        _say(f"bwd_noalloc B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}: scratch {need} bytes")
        ref, got = _case(B, Hq, Hkv, N, d, causal, seed)
        for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(r, g), f"{name} differs from fa_bwd (max {float((r.float() - g.float()).abs().max()):.3e})"
        _say("  dQ, dK, dV bit-identical to fa_bwd")


def test_bwd_noalloc_rejects_oversized_problems_before_launch():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    # 16 query heads on 1 K/V head at N = 8192: the split dK/dV partial sums need more than the scratch
    q = torch.zeros((1, 16, 8192, 128), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 1, 8192, 128), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros((1, 16, 8192), dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.bwd_noalloc(q, k, k, q, lse, q, q.clone(), k.clone(), k.clone(), causal=True)
    assert e.value.status == fa.FA_ERR_TOO_LARGE
