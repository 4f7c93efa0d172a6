"""Race and ordering checks ("FlashAttention技术解析" section 7 lists missing synchronisation among the
pitfalls): the checking builds of libfa must give the same bits as libfa.so on every entry point.

* libfa_revgrid.so: every kernel maps workgroup i of n to the tile that workgroup n-1-i takes in the normal
  build, so workgroups run in the opposite order and meet different neighbours on each compute unit and XCD;
* libfa_sync.so: every wait for the asynchronous global -> LDS copies waits for all of them.

Identical bits show that no result depends on the order or timing of workgroups or copies (no kernel here
uses atomics or cross-workgroup communication; each output element is written by one workgroup)."""
import ctypes
import os
import sys

import numpy as np
import pytest

from fa_inputs import make_block_mask, make_inputs
from fa_testlib import to_device, torch_mod

pytestmark = pytest.mark.gpu

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tiled_online_softmax_fa_amd")
CHECKS = ["revgrid", "sync"]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _libs(name):
    import tiled_online_softmax_fa_amd as fa

    return fa.open_library(os.path.join(PKG, "libfa.so")), fa.open_library(os.path.join(PKG, f"libfa_{name}.so"))


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch_mod().cuda.current_stream().cuda_stream)


def _same(outs_a, outs_b, what):
    torch = torch_mod()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs_a, outs_b)):
        assert torch.equal(a, b), f"{what}: output {i} differs (max {float((a.float() - b.float()).abs().max()):.3e})"


FWD = [(2, 8, 2, 1500, 128, 1), (1, 4, 4, 777, 64, 0), (1, 4, 2, 700, 256, 1), (4, 16, 16, 300, 128, 1),
       (1, 2, 2, 4096, 128, 1), (2, 16, 16, 4096, 128, 1), (2, 4, 4, 1000, 64, 1)]


@pytest.mark.parametrize("check", CHECKS)
@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", FWD)
def test_forward_bits_match(check, B, Hq, Hkv, N, d, causal):
    torch = torch_mod()
    base, chk = _libs(check)
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=N + d)
    q, k, v = (to_device(inp, n, "bf16") for n in ("q", "k", "v"))
    outs = []
    for lib in (base, chk):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda:0")
        assert lib.fa_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Hq, Hkv, N, d, causal, d ** -0.5, _stream()) == 0
        outs.append((o, lse))
    _same(*outs, f"{check} fwd B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("check", CHECKS)
def test_other_forwards_bits_match(check):
    torch = torch_mod()
    base, chk = _libs(check)
    B, Hq, Hkv, N, d = 1, 4, 2, 2048, 128
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=5)
    q, k, v = (to_device(inp, n, "bf16") for n in ("q", "k", "v"))
    mask = torch.from_numpy(make_block_mask("random", B, Hq, N, seed=3)).to("cuda:0")
    nb = -(-N // 64)
    outs = []
    for lib in (base, chk):
        res = []
        # split-KV, 3 parts
        ws_bytes = lib.fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, N, d, 3)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda:0")
        assert lib.fa_fwd_splitkv(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(ws), ws_bytes, B, Hq, Hkv, N, d, 1,
                                  d ** -0.5, 3, _stream()) == 0
        res += [o, lse]
        # block-sparse, a random mask per batch and head
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda:0")
        assert lib.fa_fwd_blocksparse(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(mask), mask.stride(0),
                                      mask.stride(1), B, Hq, Hkv, N, d, 1, d ** -0.5, _stream()) == 0
        res += [o, lse]
        # FP8: quantiser, then the forward
        qc = torch.empty(q.shape, dtype=torch.uint8, device="cuda:0")
        kc = torch.empty(k.shape, dtype=torch.uint8, device="cuda:0")
        qs = torch.empty((B, Hq, nb), dtype=torch.float32, device="cuda:0")
        ks = torch.empty((B, Hkv, nb), dtype=torch.float32, device="cuda:0")
        assert lib.fa_quantize_fp8(_p(q), _p(qc), _p(qs), B, Hq, N, d, _stream()) == 0
        assert lib.fa_quantize_fp8(_p(k), _p(kc), _p(ks), B, Hkv, N, d, _stream()) == 0
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda:0")
        assert lib.fa_fwd_fp8(_p(qc), _p(kc), _p(v), _p(qs), _p(ks), _p(o), _p(lse), B, Hq, Hkv, N, d, 1, d ** -0.5,
                              _stream()) == 0
        res += [qc, qs, kc, ks, o, lse]
        # fp32 storage
        qf, kf, vf = q.float().contiguous(), k.float().contiguous(), v.float().contiguous()
        o = torch.empty_like(qf)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda:0")
        assert lib.fa_fwd_f32(_p(qf), _p(kf), _p(vf), _p(o), _p(lse), B, Hq, Hkv, N, d, 1, d ** -0.5, _stream()) == 0
        res += [o, lse]
        outs.append(res)
    _same(*outs, f"{check} split-KV / block-sparse / FP8 / fp32")


BWD = [(2, 8, 2, 1500, 128, 1), (1, 4, 4, 777, 64, 0), (1, 2, 2, 600, 256, 1), (2, 16, 16, 4096, 128, 1)]


@pytest.mark.parametrize("check", CHECKS)
@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal", BWD)
def test_backward_bits_match(check, B, Hq, Hkv, N, d, causal):
    import tiled_online_softmax_fa_amd as fa

    torch = torch_mod()
    base, chk = _libs(check)
    inp = make_inputs(B, Hq, Hkv, N, d, "bf16", seed=N + d + 1, backward=True)
    q, k, v, dO = (to_device(inp, n, "bf16") for n in ("q", "k", "v", "dO"))
    o, lse = fa.fwd(q, k, v, causal=bool(causal), scale=d ** -0.5)
    ws_bytes = fa.bwd_workspace_bytes(B, Hq, Hkv, N, d)
    outs = []
    for lib in (base, chk):
        ws = torch.full((ws_bytes,), 255, dtype=torch.uint8, device="cuda:0")
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        assert lib.fa_bwd(_p(q), _p(k), _p(v), _p(o), _p(dO), _p(lse), _p(dq), _p(dk), _p(dv), _p(ws), ws_bytes,
                          B, Hq, Hkv, N, d, causal, d ** -0.5, _stream()) == 0
        outs.append((dq, dk, dv))
    _same(*outs, f"{check} bwd B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} causal={causal}")
