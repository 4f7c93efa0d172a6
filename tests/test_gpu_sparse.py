"""Block-sparse forward parity: libfa on the GPU against the fp64 block-mask oracle."""
import sys

import numpy as np
import pytest

from fa_inputs import make_block_mask, make_inputs
from fa_testlib import assert_bf16_close, assert_lse_close, lse_bound, to_device, to_f64, torch_mod
from oracle import attention_fwd, attention_fwd_blockmask

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(inp, mask, causal, scale, mask_form="4d"):
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    if mask_form == "2d":
        m = torch.from_numpy(np.ascontiguousarray(mask[0, 0])).to("cuda:0")
    elif mask_form == "3d":
        m = torch.from_numpy(np.ascontiguousarray(mask[0])).to("cuda:0")
    else:
        m = torch.from_numpy(mask).to("cuda:0")
    o, lse = fa.fwd_blocksparse(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), m, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def _compare(o, lse, O, LSE, what, bound):
    dead = np.isneginf(LSE)
    assert np.array_equal(np.isneginf(lse), dead), f"{what}: rows without keys differ"
    assert np.all(o[dead] == 0), f"{what}: rows without keys must be 0"
    mx, mean = assert_bf16_close(o, O, what)
    lmx = assert_lse_close(lse, LSE, bound, f"{what} lse")
    _say(f"  {what}: O max {mx:.2e} mean {mean:.2e}, lse max {lmx:.2e}, rows without keys {int(dead.sum())}")


CASES = [
    # B, Hq, Hkv, N, d, causal, kind, mask form
    (1, 2, 2, 300, 64, False, "random", "4d"),
    (1, 2, 2, 300, 128, True, "random", "4d"),
    (2, 4, 2, 513, 128, False, "holes", "4d"),
    (2, 4, 2, 513, 128, True, "holes", "4d"),
    (1, 4, 1, 1000, 64, True, "band", "2d"),
    (1, 3, 3, 640, 128, False, "diag", "3d"),
    (1, 2, 2, 2048, 128, True, "random", "4d"),
    (1, 2, 2, 2048, 128, False, "band", "2d"),
    (1, 1, 1, 1, 64, False, "all", "2d"),
    (1, 2, 2, 129, 128, True, "random", "4d"),
    (1, 2, 2, 300, 256, True, "random", "4d"),
    (1, 2, 1, 700, 256, False, "holes", "4d"),
    (1, 2, 2, 1024, 256, True, "band", "2d"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,kind,form", CASES)
def test_fwd_blocksparse_small(B, Hq, Hkv, N, d, causal, kind, form):
    _say(f"block-sparse B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal} mask={kind} ({form})")
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=N + d + 7)
    mask = make_block_mask(kind, B, Hq, N, seed=N)
    scale = d ** -0.5
    o, lse = _run(inp, mask, causal, scale, form)
    O, LSE = attention_fwd_blockmask(inp["q"], inp["k"], inp["v"], mask, causal, scale)
    _compare(o, lse, O, LSE, kind, lse_bound(inp["q"], inp["k"], scale))


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_blocksparse_all_blocks_equals_dense(causal):
    # every block on: the same answer as the dense oracle
    inp = make_inputs(2, 4, 2, 777, 128, "bf16", seed=3)
    mask = make_block_mask("all", 2, 4, 777)
    o, lse = _run(inp, mask, causal, 128 ** -0.5)
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], causal, 128 ** -0.5)
    _compare(o, lse, O, LSE, "all blocks", lse_bound(inp["q"], inp["k"], 128 ** -0.5))


def test_fwd_blocksparse_peaky():
    inp = make_inputs(1, 4, 2, 900, 128, "bf16", seed=12, q_mult=8.0)
    mask = make_block_mask("holes", 1, 4, 900, seed=5)
    o, lse = _run(inp, mask, True, 128 ** -0.5)
    O, LSE = attention_fwd_blockmask(inp["q"], inp["k"], inp["v"], mask, True, 128 ** -0.5)
    assert_bf16_close(o, O, "peaky")
    assert_lse_close(lse, LSE, lse_bound(inp["q"], inp["k"], 128 ** -0.5), "peaky lse")


@pytest.mark.parametrize("kind,causal", [("band", True), ("random", False)])
def test_fwd_blocksparse_workload_4096(kind, causal):
    # B2 H16 N4096 d128: a sliding window of 3 blocks plus the first block (causal), and a random half of the
    # blocks per head (not causal); every element of O and lse, one head at a time
    B, H, N, d = 2, 16, 4096, 128
    inp = make_inputs(B, H, H, N, d, "bf16", seed=9)
    mask = make_block_mask(kind, B, H, N, seed=4)
    o, lse = _run(inp, mask, causal, d ** -0.5, "2d" if kind == "band" else "4d")
    assert np.isfinite(o).all() and not np.isnan(lse).any()
    worst, total, lworst = 0.0, 0.0, 0.0
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            O, LSE = attention_fwd_blockmask(inp["q"][sl], inp["k"][sl], inp["v"][sl], mask[sl], causal, d ** -0.5)
            dead = np.isneginf(LSE)
            assert np.array_equal(np.isneginf(lse[sl]), dead) and np.all(o[sl][dead] == 0)
            e = np.abs(o[sl] - O)
            worst = max(worst, float(e.max()))
            total += float(e.sum())
            assert worst <= 2e-2, f"{kind} head ({b},{h}): max {worst:.3e}"
            lworst = max(lworst, assert_lse_close(lse[sl], LSE, lse_bound(inp["q"][sl], inp["k"][sl], d ** -0.5)))
    mean = total / o.size
    _say(f"  {kind}: whole tensor O max {worst:.2e} mean {mean:.2e}, lse max {lworst:.2e}")
    assert mean <= 2e-3


def test_fwd_blocksparse_errors():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    q = torch.zeros((1, 2, 200, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        fa.fwd_blocksparse(q, q, q, torch.ones((3, 3), dtype=torch.uint8, device="cuda:0"))  # n_blk is 2
    with pytest.raises(TypeError):
        fa.fwd_blocksparse(q, q, q, torch.ones((2, 2), dtype=torch.float32, device="cuda:0"))
    o, lse = fa.fwd_blocksparse(q, q, q, torch.zeros((2, 2), dtype=torch.bool, device="cuda:0"))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
