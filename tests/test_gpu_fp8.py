"""FP8 parity: libfa's block-wise e4m3 quantiser (bit-exact codes and scales) and FP8
forward (against the fp64 definition on the dequantised Q, K) on the GPU."""
import sys

import numpy as np
import pytest

from fa_inputs import bf16_bits_to_f32, bf16_round_bits, make_inputs
from fa_testlib import assert_bf16_close, assert_lse_close, errors, lse_bound, to_device, to_f64, torch_mod
from oracle import attention_fwd, attention_fwd_fp8, dequantize_blockwise_e4m3, quantize_blockwise_e4m3

pytestmark = pytest.mark.gpu

# lse of the FP8 path: the same derived per-row bound as the bf16 path (fa_testlib.lse_bound), taken on the
# dequantised Q and K that the oracle uses: the FP8 instruction's sums err in proportion to the sum of the
# products' magnitudes, like the bf16 ones.


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16_tensor(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _quantise_on_gpu(x_bits):
    import tiled_online_softmax_fa_amd as fa

    codes, scale = fa.quantize_fp8(_bf16_tensor(x_bits))
    torch_mod().cuda.synchronize()
    return codes.cpu().numpy(), scale.cpu().numpy()


@pytest.mark.parametrize("B,H,N,d", [(1, 2, 300, 128), (2, 3, 64, 64), (1, 1, 1, 256), (1, 2, 1000, 256),
                                     (2, 2, 129, 128)])
def test_quantize_fp8_bit_exact(B, H, N, d):
    rng = np.random.default_rng(N + d)
    x = rng.standard_normal((B, H, N, d), dtype=np.float32)
    x *= rng.uniform(1e-3, 50.0, (B, H, 1, 1)).astype(np.float32)  # per-head magnitudes
    x[0, 0, :64] = 0.0                                                 # a zero block: scale 1
    if N > 64:
        x[0, -1, 64:128] *= np.float32(1e-6)                           # tiny block values (subnormal codes)
    bits = bf16_round_bits(x)
    codes, scale = _quantise_on_gpu(bits)
    want_codes, want_scale = quantize_blockwise_e4m3(bf16_bits_to_f32(bits))
    assert np.array_equal(scale.view(np.uint32), want_scale.view(np.uint32)), "scales differ"
    bad = codes != want_codes
    assert not bad.any(), f"{int(bad.sum())} codes differ, e.g. gpu {codes[bad][:5]} oracle {want_codes[bad][:5]}"
    _say(f"  quantise B{B} H{H} N{N} d{d}: codes and scales bit-exact")


def _fp8_inputs(B, Hq, Hkv, N, d, seed):
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=seed)
    qc, qs = quantize_blockwise_e4m3(inp["q"])
    kc, ks = quantize_blockwise_e4m3(inp["k"])
    return inp, qc, qs, kc, ks


def _run_fp8(qc, qs, kc, ks, inp, causal, scale):
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    o, lse = fa.fwd_fp8(dev(qc), dev(qs), dev(kc), dev(ks), to_device(inp, "v", "bf16"), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


CASES = [
    (1, 2, 2, 300, 128, False),
    (1, 2, 2, 300, 128, True),
    (2, 8, 2, 513, 128, True),
    (1, 3, 3, 640, 128, False),
    (1, 1, 1, 1, 128, True),
    (1, 2, 2, 17, 128, True),
    (1, 2, 2, 300, 256, True),
    (1, 2, 1, 700, 256, False),
    (1, 1, 1, 2048, 128, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", CASES)
def test_fwd_fp8_small(B, Hq, Hkv, N, d, causal):
    _say(f"fwd fp8 B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
    inp, qc, qs, kc, ks = _fp8_inputs(B, Hq, Hkv, N, d, seed=N + d + 1)
    scale = d ** -0.5
    o, lse = _run_fp8(qc, qs, kc, ks, inp, causal, scale)
    O, LSE = attention_fwd_fp8(qc, qs, kc, ks, inp["v"], causal, scale)
    mx, mean = assert_bf16_close(o, O, "O (fp8 inputs)")
    lmx = assert_lse_close(lse, LSE, lse_bound(dequantize_blockwise_e4m3(qc, qs), dequantize_blockwise_e4m3(kc, ks), scale))
    # the quantisation itself, against the unquantised inputs (reported; loose sanity bound)
    O0, _ = attention_fwd(inp["q"], inp["k"], inp["v"], causal, scale)
    qmx, qmean = errors(o, O0)
    _say(f"  vs dequantised: O max {mx:.2e} mean {mean:.2e} lse {lmx:.2e}; vs bf16 inputs: max {qmx:.2e} "
         f"mean {qmean:.2e}")
    assert qmx <= 0.25 and qmean <= 2e-2


def test_fwd_fp8_peaky_with_gpu_quantised_inputs():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    inp = make_inputs(1, 4, 2, 900, 128, "bf16", seed=12, q_mult=8.0)
    qc, qs = fa.quantize_fp8(to_device(inp, "q", "bf16"))
    kc, ks = fa.quantize_fp8(to_device(inp, "k", "bf16"))
    o, lse = fa.fwd_fp8(qc, qs, kc, ks, to_device(inp, "v", "bf16"), causal=True)
    torch.cuda.synchronize()
    O, LSE = attention_fwd_fp8(qc.cpu().numpy(), qs.cpu().numpy(), kc.cpu().numpy(), ks.cpu().numpy(), inp["v"],
                               True, 128 ** -0.5)
    assert_bf16_close(to_f64(o), O, "peaky fp8")
    qd = dequantize_blockwise_e4m3(qc.cpu().numpy(), qs.cpu().numpy())
    kd = dequantize_blockwise_e4m3(kc.cpu().numpy(), ks.cpu().numpy())
    assert_lse_close(to_f64(lse), LSE, lse_bound(qd, kd, 128 ** -0.5))


def test_fwd_fp8_workload_causal_4096():
    # B2 H16 N4096 d128 causal: every element of O and lse against the dequantised definition
    B, H, N, d = 2, 16, 4096, 128
    inp, qc, qs, kc, ks = _fp8_inputs(B, H, H, N, d, seed=2)
    o, lse = _run_fp8(qc, qs, kc, ks, inp, True, d ** -0.5)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    qd = dequantize_blockwise_e4m3(qc, qs)
    kd = dequantize_blockwise_e4m3(kc, ks)
    worst, total, lworst = 0.0, 0.0, 0.0
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            O, LSE = attention_fwd(qd[sl], kd[sl], inp["v"][sl], True, d ** -0.5)
            e = np.abs(o[sl] - O)
            worst = max(worst, float(e.max()))
            total += float(e.sum())
            assert worst <= 2e-2, f"head ({b},{h}): max {worst:.3e}"
            lworst = max(lworst, assert_lse_close(lse[sl], LSE, lse_bound(qd[sl], kd[sl], d ** -0.5)))
    mean = total / o.size
    _say(f"  whole tensor O max {worst:.2e} mean {mean:.2e}, lse max {lworst:.2e}")
    assert mean <= 2e-3


def test_fwd_fp8_errors():
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    c = torch.zeros((1, 2, 8, 64), dtype=torch.uint8, device="cuda:0")
    s = torch.ones((1, 2, 1), dtype=torch.float32, device="cuda:0")
    v = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fwd_fp8(c, s, c, s, v)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        fa.fwd_fp8(c, torch.ones((1, 2, 2), dtype=torch.float32, device="cuda:0"), c, s, v)


def test_fwd_fp8_other_scale_ragged_causal():
    inp, qc, qs, kc, ks = _fp8_inputs(1, 4, 2, 333, 128, seed=5)
    o, lse = _run_fp8(qc, qs, kc, ks, inp, True, 0.3)
    O, LSE = attention_fwd_fp8(qc, qs, kc, ks, inp["v"], True, 0.3)
    assert_bf16_close(o, O, "fp8 scale 0.3")
    assert_lse_close(lse, LSE, lse_bound(dequantize_blockwise_e4m3(qc, qs), dequantize_blockwise_e4m3(kc, ks), 0.3))
