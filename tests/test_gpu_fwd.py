"""Forward parity: libfa on the GPU against the fp64 CPU oracle, same seeded inputs."""
import sys

import numpy as np
import pytest

from fa_inputs import WORKLOADS, make_inputs, make_workload_inputs
from fa_testlib import (F32_MAX_ABS, assert_bf16_close, assert_lse_close, errors, lse_bound, lse_bound_rows,
                        run_fwd, to_device, to_f64, torch_mod)
from oracle import attention_fwd, attention_fwd_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = [
    # B, Hq, Hkv, N, d, causal  -- several tiles, ragged tails, grouped heads
    (1, 2, 2, 300, 64, False),
    (1, 2, 2, 300, 64, True),
    (1, 2, 2, 300, 128, False),
    (1, 2, 2, 300, 128, True),
    (2, 8, 2, 513, 128, True),
    (1, 4, 1, 1000, 64, True),
    (1, 3, 3, 640, 128, False),
    (2, 2, 1, 257, 64, False),
    (1, 2, 2, 255, 128, True),
    (1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 128, True),
    (1, 2, 2, 17, 128, True),
    (1, 2, 2, 64, 64, True),
    (1, 1, 1, 2048, 128, True),
    # head dim 256 (32-key tiles, 128-query tiles)
    (1, 2, 2, 300, 256, False),
    (1, 2, 2, 300, 256, True),
    (2, 4, 2, 513, 256, True),
    (1, 2, 1, 129, 256, False),
    (1, 1, 1, 1, 256, True),
    (1, 2, 2, 31, 256, True),
    (1, 1, 1, 1024, 256, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", SMALL)
def test_fwd_bf16_small(B, Hq, Hkv, N, d, causal):
    _say(f"fwd bf16 B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
    inp, o, lse, scale = run_fwd(B, Hq, Hkv, N, d, causal, "bf16", seed=N + d)
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], causal, scale)
    mx, mean = assert_bf16_close(o, O, "O")
    lmx = assert_lse_close(lse, LSE, lse_bound(inp["q"], inp["k"], scale))
    _say(f"  O max {mx:.2e} mean {mean:.2e}  lse max {lmx:.2e}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwd_bf16_peaky_scores(causal, d):
    # q scaled by 8: softmax rows are dominated by a few keys and the running
    # maximum moves often, exercising the rescale path
    _say(f"fwd bf16 peaky d{d} causal={causal}")
    inp, o, lse, scale = run_fwd(1, 4, 2, 700, d, causal, "bf16", seed=11, q_mult=8.0)
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_bf16_close(o, O, "O")
    assert_lse_close(lse, LSE, lse_bound(inp["q"], inp["k"], scale))


def test_fwd_bf16_increasing_keys_force_rescales():
    # keys whose scores grow along the sequence: the reference maximum must move
    # on nearly every tile
    torch = torch_mod()
    import tiled_online_softmax_fa_amd as fa
    from fa_inputs import bf16_round_bits, bf16_bits_to_f32

    N, d = 777, 128
    rng = np.random.default_rng(5)
    q = np.ones((1, 1, N, d), np.float32)
    k = (np.linspace(0, 6, N, dtype=np.float32)[None, None, :, None] * np.ones((1, 1, 1, d), np.float32))
    v = rng.standard_normal((1, 1, N, d), dtype=np.float32)
    inp = {}
    for n, x in (("q", q), ("k", k), ("v", v)):
        inp[n + "_bits"] = bf16_round_bits(x)
        inp[n] = bf16_bits_to_f32(inp[n + "_bits"])
    for causal in (False, True):
        o, lse = fa.fwd(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), causal=causal, scale=0.05)
        torch.cuda.synchronize()
        O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], causal, 0.05)
        assert_bf16_close(to_f64(o), O, f"O causal={causal}")
        assert_lse_close(to_f64(lse), LSE, lse_bound(inp["q"], inp["k"], 0.05))


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [(1, 1, 1, 256, 64, False), (1, 2, 2, 300, 64, True),
                                                 (2, 2, 1, 77, 128, False), (1, 1, 1, 1, 64, True)])
def test_fwd_f32_small(B, Hq, Hkv, N, d, causal):
    _say(f"fwd f32 B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
    inp, o, lse, scale = run_fwd(B, Hq, Hkv, N, d, causal, "f32", seed=N)
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], causal, scale)
    mx, _ = errors(o, O)
    lmx, _ = errors(lse, LSE)
    _say(f"  O max {mx:.2e} lse max {lmx:.2e}")
    assert np.isfinite(o).all() and mx <= F32_MAX_ABS and lmx <= F32_MAX_ABS


def test_fwd_f32_workload_single_head_256():
    w = WORKLOADS["fwd_f32_b1h1n256d64"]
    _say(f"workload {w.name}")
    inp = make_workload_inputs(w)
    import tiled_online_softmax_fa_amd as fa

    o, lse = fa.fwd_f32(*(to_device(inp, n, "f32") for n in ("q", "k", "v")), causal=w.causal, scale=w.scale)
    torch_mod().cuda.synchronize()
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], w.causal, w.scale)
    mx, _ = errors(to_f64(o), O)
    lmx, _ = errors(to_f64(lse), LSE)
    _say(f"  O max {mx:.2e} lse max {lmx:.2e}")
    assert mx <= F32_MAX_ABS and lmx <= F32_MAX_ABS


def test_fwd_bf16_workload_multihead_2048_full():
    w = WORKLOADS["fwd_bf16_b4h16n2048d64"]
    _say(f"workload {w.name} (full oracle)")
    inp = make_workload_inputs(w)
    import tiled_online_softmax_fa_amd as fa

    o, lse = fa.fwd(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), causal=w.causal, scale=w.scale)
    torch_mod().cuda.synchronize()
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], w.causal, w.scale)
    mx, mean = assert_bf16_close(to_f64(o), O, "O")
    _say(f"  O max {mx:.2e} mean {mean:.2e}")
    assert_lse_close(to_f64(lse), LSE, lse_bound(inp["q"], inp["k"], w.scale))


def _sampled_check(w, n_full_heads=2, rows_per_head=48, seed=123):
    """Long or large workloads: every head checked on sampled rows, a few heads in full."""
    import tiled_online_softmax_fa_amd as fa

    inp = make_workload_inputs(w)
    o, lse = fa.fwd(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), causal=w.causal, scale=w.scale)
    torch_mod().cuda.synchronize()
    o, lse = to_f64(o), to_f64(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(seed)
    worst = 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            rows = np.unique(np.concatenate([[0, 1, w.N - 1], rng.integers(0, w.N, rows_per_head)]))
            Or, Lr = attention_fwd_rows(inp["q"], inp["k"], inp["v"], w.causal, w.scale, b, h, rows)
            mx, _ = errors(o[b, h, rows], Or)
            worst = max(worst, mx)
            assert mx <= 2e-2, f"head ({b},{h}) sampled rows: max {mx:.3e}"
            assert_lse_close(lse[b, h, rows], Lr,
                             lse_bound_rows(inp["q"][b, h][rows], inp["k"][b, h // (w.Hq // w.Hkv)], w.scale))
    G = w.Hq // w.Hkv
    for i in range(n_full_heads):
        b, h = i % w.B, (7 * i + 3) % w.Hq
        O, LSE = attention_fwd(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h // G:h // G + 1],
                               inp["v"][b:b + 1, h // G:h // G + 1], w.causal, w.scale)
        assert_bf16_close(o[b:b + 1, h:h + 1], O, f"full head ({b},{h})")
        assert_lse_close(lse[b:b + 1, h:h + 1], LSE,
                         lse_bound(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h // G:h // G + 1], w.scale))
    _say(f"  sampled worst max {worst:.2e}")


def full_tensor_check(o, lse, inp, causal, scale, what):
    """Every element of o [B, Hq, N, d] and lse [B, Hq, N] against the oracle, one head at a time.

    The bf16 bars apply to the whole tensor: max |O - ref| <= 2e-2 and the
    mean over all B * Hq * N * d elements <= 2e-3; lse within its per-row bound.
    """
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    B, Hq, N, _ = o.shape
    G = Hq // inp["k"].shape[1]
    worst, total, lworst = 0.0, 0.0, 0.0
    for b in range(B):
        for h in range(Hq):
            sl = (slice(b, b + 1), slice(h, h + 1))
            kv = (slice(b, b + 1), slice(h // G, h // G + 1))
            O, LSE = attention_fwd(inp["q"][sl], inp["k"][kv], inp["v"][kv], causal, scale)
            d = np.abs(o[sl] - O)
            worst = max(worst, float(d.max()))
            total += float(d.sum())
            assert worst <= 2e-2, f"{what}: head ({b},{h}) max {worst:.3e}"
            lworst = max(lworst, assert_lse_close(lse[sl], LSE, lse_bound(inp["q"][sl], inp["k"][kv], scale),
                                                  f"{what} lse head ({b},{h})"))
    mean = total / o.size
    _say(f"  {what}: whole tensor O max {worst:.2e} mean {mean:.2e}, lse max {lworst:.2e}")
    assert mean <= 2e-3, f"{what}: mean {mean:.3e} over the whole tensor"


def _full_workload(w):
    import tiled_online_softmax_fa_amd as fa

    inp = make_workload_inputs(w)
    o, lse = fa.fwd(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), causal=w.causal, scale=w.scale)
    torch_mod().cuda.synchronize()
    full_tensor_check(to_f64(o), to_f64(lse), inp, w.causal, w.scale, w.name)


def test_fwd_bf16_workload_causal_4096():
    w = WORKLOADS["fwd_causal_bf16_b2h16n4096d128"]
    _say(f"workload {w.name} (every element of O and lse)")
    _full_workload(w)


def test_fwd_bf16_workload_causal_gqa_4096():
    w = WORKLOADS["fwd_causal_gqa_bf16_b2hq64hkv8n4096d128"]
    _say(f"workload {w.name} (every element of O and lse)")
    _full_workload(w)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", [(4, 32, 8, 1100, 128, True), (4, 32, 8, 1100, 128, False),
                                                  (4, 32, 32, 1037, 64, False), (2, 64, 64, 777, 128, False)])
def test_fwd_bf16_full_grid_ragged(B, Hq, Hkv, N, d, causal):
    # grids of at least two 256-row workgroups per compute unit with N > 512 (and not causal d = 64) take the
    # 256-row tiles; ragged lengths cut their last query tile and last key tile
    from fa_inputs import Workload

    w = Workload(f"fwd_grid_b{B}hq{Hq}hkv{Hkv}n{N}d{d}", B, Hq, Hkv, N, d, "bf16", causal, seed=N + d)
    _say(f"{w.name} causal={causal} (every element)")
    _full_workload(w)


@pytest.mark.parametrize("Hq,Hkv,d,causal", [(4, 2, 128, True), (2, 2, 64, False), (2, 1, 256, True)])
def test_fwd_bf16_long_sequence_16384(Hq, Hkv, d, causal):
    # 64 (causal: 1 to 256) key tiles per query tile: sampled rows against the oracle
    from fa_inputs import Workload

    w = Workload(f"long_b1hq{Hq}hkv{Hkv}n16384d{d}", 1, Hq, Hkv, 16384, d, "bf16", causal, seed=77)
    _say(f"workload {w.name} (sampled rows)")
    _sampled_check(w, n_full_heads=0, rows_per_head=24)


SPLITKV = [
    # B, Hq, Hkv, N, d, causal, n_splits  -- including more parts than key tiles (empty parts)
    (1, 2, 2, 300, 64, False, 2),
    (1, 2, 2, 300, 128, True, 3),
    (2, 8, 2, 513, 128, True, 4),
    (1, 4, 1, 1000, 64, True, 7),
    (1, 1, 1, 2048, 128, True, 16),
    (1, 2, 2, 2048, 64, False, 5),
    (1, 2, 2, 17, 128, True, 5),
    (1, 1, 1, 1, 64, False, 2),
    (1, 2, 2, 300, 256, True, 3),
    (1, 2, 2, 2048, 128, True, 0),   # n_splits = 0: the library's choice
    (1, 2, 1, 1500, 256, False, 0),
    (1, 1, 1, 300, 64, False, 0),
    (1, 2, 1, 1000, 256, False, 4),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,n_splits", SPLITKV)
def test_fwd_splitkv_small(B, Hq, Hkv, N, d, causal, n_splits):
    import tiled_online_softmax_fa_amd as fa

    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=N + 13 * n_splits)
    scale = d ** -0.5
    o, lse = fa.fwd_splitkv(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), n_splits, causal=causal,
                            scale=scale)
    torch_mod().cuda.synchronize()
    O, LSE = attention_fwd(inp["q"], inp["k"], inp["v"], causal, scale)
    mx, mean = assert_bf16_close(to_f64(o), O, f"split-KV x{n_splits} O")
    assert_lse_close(to_f64(lse), LSE, lse_bound(inp["q"], inp["k"], scale))
    _say(f"  split-KV x{n_splits}: O max {mx:.2e} mean {mean:.2e}")


def test_fwd_splitkv_one_part_is_the_plain_forward():
    import tiled_online_softmax_fa_amd as fa

    inp = make_inputs(1, 8, 8, 4096, 128, "bf16", seed=17)
    q, k, v = (to_device(inp, n, "bf16") for n in ("q", "k", "v"))
    torch = torch_mod()
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd_splitkv(q, k, v, 1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_splitkv_long_sequence_16384():
    from fa_inputs import Workload
    import tiled_online_softmax_fa_amd as fa

    w = Workload("long_split_b1hq4hkv2n16384d128", 1, 4, 2, 16384, 128, "bf16", True, seed=78)
    inp = make_workload_inputs(w)
    o, lse = fa.fwd_splitkv(*(to_device(inp, n, "bf16") for n in ("q", "k", "v")), 8, causal=True, scale=w.scale)
    torch_mod().cuda.synchronize()
    o, lse = to_f64(o), to_f64(lse)
    rng = np.random.default_rng(5)
    for h in range(w.Hq):
        rows = np.unique(np.concatenate([[0, 1, 255, 256, w.N - 1], rng.integers(0, w.N, 24)]))
        Or, Lr = attention_fwd_rows(inp["q"], inp["k"], inp["v"], True, w.scale, 0, h, rows)
        assert errors(o[0, h, rows], Or)[0] <= 2e-2
        assert_lse_close(lse[0, h, rows], Lr, lse_bound_rows(inp["q"][0, h][rows], inp["k"][0, h // 2], w.scale))


def test_fwd_bf16_is_bitwise_repeatable():
    import tiled_online_softmax_fa_amd as fa

    inp_shape = (2, 8, 2, 1500, 128)
    from fa_inputs import make_inputs

    inp = make_inputs(*inp_shape, "bf16", seed=9)
    q, k, v = (to_device(inp, n, "bf16") for n in ("q", "k", "v"))
    torch = torch_mod()
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_empty_and_errors():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    z = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    o, lse = fa.fwd(z, z, z, causal=True)
    assert o.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)
    q = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros((1, 2, 8, 256), dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fwd_f32(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros((1, 3, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, k, k)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    flat = torch.zeros(2 * 8 * 64 + 1, dtype=torch.bfloat16, device="cuda:0")
    mis = flat[1:].view(1, 2, 8, 64)  # 2-byte offset: misaligned base pointer
    with pytest.raises(fa.FaError) as e:
        fa.fwd(mis, mis, mis)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
