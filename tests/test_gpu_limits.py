"""The largest tensors the ABI accepts (just under 2^31 elements): per-head base offsets beyond
2^32 bytes, checked against the fp64 oracle on the first, middle and last heads."""
import sys

import numpy as np
import pytest

from fa_testlib import assert_bf16_close, assert_lse_close, errors, lse_bound_rows, torch_mod
from oracle import attention_bwd, attention_fwd_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_fwd_bwd_largest_tensors_grouped_causal():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    B, Hq, Hkv, N, d = 1, 4095, 1365, 4096, 128  # q, o, dO, dq: 2^31 - 2^19 elements each
    assert 2 ** 31 - 2 ** 20 < B * Hq * N * d < 2 ** 31
    G = Hq // Hkv
    scale = d ** -0.5
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(2024)  # seeded synthetic N(0, 1) inputs, drawn on the device (4 GiB each)
    q = torch.randn((B, Hq, N, d), generator=gen, device="cuda:0", dtype=torch.bfloat16)
    k = torch.randn((B, Hkv, N, d), generator=gen, device="cuda:0", dtype=torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), generator=gen, device="cuda:0", dtype=torch.bfloat16)
    dO = torch.randn((B, Hq, N, d), generator=gen, device="cuda:0", dtype=torch.bfloat16)
    _say("inputs drawn; forward")
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    _say("backward")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, dO, causal=True, scale=scale)
    torch.cuda.synchronize()
    _say("checking")
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    for h in (0, 1, 2047, Hq - 3, Hq - 1):
        rows = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.integers(0, N, 12)]))
        qh, kh, vh = host(q[:, h:h + 1]), host(k[:, h // G:h // G + 1]), host(v[:, h // G:h // G + 1])
        Or, Lr = attention_fwd_rows(qh, kh, vh, True, scale, 0, 0, rows)
        assert errors(host(o[0, h])[rows], Or)[0] <= 2e-2, f"head {h}"
        assert_lse_close(lse[0, h].cpu().numpy().astype(np.float64)[rows], Lr,
                         lse_bound_rows(qh[0, 0][rows], kh[0, 0], scale), f"lse head {h}")
    # the last key/value head and its three query heads (the end of every tensor): full gradients
    hs = slice(Hq - G, Hq)
    ref = attention_bwd(host(q[:, hs]), host(k[:, Hkv - 1:]), host(v[:, Hkv - 1:]), host(dO[:, hs]), True, scale)
    for name, got, rf in zip(("dQ", "dK", "dV"), (host(dq[:, hs]), host(dk[:, Hkv - 1:]), host(dv[:, Hkv - 1:])), ref):
        s = float(np.abs(rf).max())
        mx, mean = assert_bf16_close(got, rf, f"last group {name}", scale=s)
        _say(f"  last group {name}: max {mx / s:.1e} mean {mean / s:.1e}")
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
