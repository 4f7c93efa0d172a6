"""Exact tiled attention for AMD MI355X (gfx950): Python binding of libfa.

Every step of the computation runs in libfa's HIP kernels; this module only
checks tensor metadata, allocates outputs with torch (device memory), and
passes raw pointers and the current stream through the C ABI declared in
include/fa.h. There is no fallback: if libfa.so is missing or cannot be
loaded, importing the ops raises.

    o, lse = fwd(q, k, v, causal=True)              # bf16 [B,H,N,d], d = 64, 128, 256
    o, lse = fwd_f32(q, k, v)                        # float32, d = 64, 128
    o, lse = fwd_splitkv(q, k, v, 4, causal=True)    # keys of each query tile in 4 parts + merge
    o, lse = fwd_blocksparse(q, k, v, mask)          # uint8/bool block mask, 128 x 128 blocks
    qc, qs = quantize_fp8(q); kc, ks = quantize_fp8(k)
    o, lse = fwd_fp8(qc, qs, kc, ks, v, causal=True) # e4m3 Q, K with per-64-row scales
    dq, dk, dv = bwd(q, k, v, o, lse, dout, causal=True)
    o = flash_attn(q, k, v, causal=True)             # autograd.Function
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LIB_PATH",
    "FaError",
    "load_library",
    "open_library",
    "fwd",
    "fwd_f32",
    "fwd_splitkv",
    "splitkv_workspace_bytes",
    "fwd_blocksparse",
    "SPARSE_BLOCK",
    "quantize_fp8",
    "fwd_fp8",
    "FP8_BLOCK",
    "bwd",
    "bwd_workspace_bytes",
    "bwd_noalloc",
    "BWD_NOALLOC_SCRATCH_BYTES",
    "flash_attn",
    "status_string",
    "FA_OK",
    "FA_ERR_INVALID_ARG",
    "FA_ERR_UNSUPPORTED",
    "FA_ERR_DEVICE",
    "FA_ERR_LAUNCH",
    "FA_ERR_INTERNAL",
    "FA_ERR_TOO_LARGE",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_DEVICE = -3
FA_ERR_LAUNCH = -4
FA_ERR_INTERNAL = -5
FA_ERR_TOO_LARGE = -6

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: libfa status {status} ({status_string(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once and declare the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Load a library with libfa's C ABI from `path` (not cached; e.g. a checking build) and declare its
    signatures. Raises if it is missing."""
    if not os.path.exists(path):
        raise ImportError(f"{os.path.basename(path)} not found at {path}; build it with "
                          "`python -m tiled_online_softmax_fa_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_f32.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp, vp]
    lib.fa_bwd_timed.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_splitkv.restype = i
    ll = ctypes.c_longlong
    lib.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, ll, ll, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_blocksparse.restype = i
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.fa_quantize_fp8.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != FA_OK:
        raise FaError(status, what)


def _torch():
    import torch

    return torch


def _stream_ptr(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _guard(*tensors):
    """All tensors on one GPU; the calls below run with that GPU current (the library's device check and
    launches use the current device)."""
    torch = _torch()
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(str(d) for d in devs)}")
    return torch.cuda.device(devs.pop())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, Hq, k.shape[1], N, d


def _require(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fwd_impl(entry, dtype, q, k, v, causal, scale, out, lse):
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, dtype, n)
    B, Hq, Hkv, N, d = _dims(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require(out, dtype, "out")
    _require(lse, torch.float32, "lse")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("out/lse have the wrong shape")
    lib = load_library()
    with _guard(q, k, v, out, lse):
        st = getattr(lib, entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d,
                             int(bool(causal)), float(scale), _stream_ptr(q))
    _check(st, entry)
    return out, lse


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Forward attention on bf16 tensors (q [B,Hq,N,d], k/v [B,Hkv,N,d]). Returns (o, lse)."""
    return _fwd_impl("fa_fwd", _torch().bfloat16, q, k, v, causal, scale, out, lse)


def fwd_f32(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Forward attention on float32 tensors. Returns (o, lse)."""
    return _fwd_impl("fa_fwd_f32", _torch().float32, q, k, v, causal, scale, out, lse)


def splitkv_workspace_bytes(B, Hq, Hkv, N, d, n_splits) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_bytes(B, Hq, Hkv, N, d, n_splits))


def fwd_splitkv(q, k, v, n_splits=0, causal=False, scale=None, out=None, lse=None, workspace=None):
    """Forward attention on bf16 tensors with each query tile's keys split into n_splits ranges
    (separate workgroups, then a merge; 0 = the library's choice for the GPU's 256 compute units).
    Same results as fwd up to rounding. Returns (o, lse)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    B, Hq, Hkv, N, d = _dims(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require(out, torch.bfloat16, "out")
    _require(lse, torch.float32, "lse")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("out/lse have the wrong shape")
    need = splitkv_workspace_bytes(B, Hq, Hkv, N, d, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    lib = load_library()
    with _guard(q, k, v, out, lse, workspace):
        st = lib.fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                B, Hq, Hkv, N, d, int(bool(causal)), float(scale), int(n_splits), _stream_ptr(q))
    _check(st, "fa_fwd_splitkv")
    return out, lse


FP8_BLOCK = 64  # FA_FP8_BLOCK


def quantize_fp8(x, codes=None, scale=None):
    """Block-wise e4m3 quantisation of a bf16 tensor [B, H, N, d]: returns (codes uint8 [B, H, N, d],
    scale float32 [B, H, ceil(N / 64)]) with x ~= e4m3(codes) * scale."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    nb = -(-N // FP8_BLOCK)
    if codes is None:
        codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    _require(codes, torch.uint8, "codes")
    _require(scale, torch.float32, "scale")
    if tuple(codes.shape) != (B, H, N, d) or tuple(scale.shape) != (B, H, nb):
        raise ValueError("codes/scale have the wrong shape")
    with _guard(x, codes, scale):
        st = load_library().fa_quantize_fp8(_ptr(x), _ptr(codes), _ptr(scale), B, H, N, d, _stream_ptr(x))
    _check(st, "fa_quantize_fp8")
    return codes, scale


def fwd_fp8(q_codes, q_scale, k_codes, k_scale, v, causal=False, scale=None, out=None, lse=None):
    """Forward attention with e4m3 q, k (codes uint8 and per-64-row float32 scales, as from quantize_fp8)
    and bf16 v. Returns (o bf16, lse float32)."""
    torch = _torch()
    _require(q_codes, torch.uint8, "q_codes")
    _require(k_codes, torch.uint8, "k_codes")
    _require(v, torch.bfloat16, "v")
    _require(q_scale, torch.float32, "q_scale")
    _require(k_scale, torch.float32, "k_scale")
    B, Hq, Hkv, N, d = _dims(q_codes, k_codes, v)
    nb = -(-N // FP8_BLOCK)
    if tuple(q_scale.shape) != (B, Hq, nb) or tuple(k_scale.shape) != (B, Hkv, nb):
        raise ValueError(f"q_scale/k_scale must be [B, H, {nb}]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=v.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=v.device)
    _require(out, torch.bfloat16, "out")
    _require(lse, torch.float32, "lse")
    if tuple(out.shape) != (B, Hq, N, d) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("out/lse have the wrong shape")
    with _guard(q_codes, k_codes, v, q_scale, k_scale, out, lse):
        st = load_library().fa_fwd_fp8(_ptr(q_codes), _ptr(k_codes), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(out),
                                   _ptr(lse), B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _stream_ptr(v))
    _check(st, "fa_fwd_fp8")
    return out, lse


SPARSE_BLOCK = 128  # FA_SPARSE_BLOCK


def fwd_blocksparse(q, k, v, block_mask, causal=False, scale=None, out=None, lse=None):
    """Forward attention on bf16 tensors restricted by a block mask of 128 x 128 blocks.

    block_mask: uint8 or bool GPU tensor [n_blk, n_blk] (shared by all batches and heads),
    [Hq, n_blk, n_blk] (per query head) or [B, Hq, n_blk, n_blk], n_blk = ceil(N / 128);
    the last two dims contiguous. Rows that see no key get o = 0, lse = -inf. Returns (o, lse).
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    B, Hq, Hkv, N, d = _dims(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n_blk = -(-N // SPARSE_BLOCK)
    m = block_mask
    if not isinstance(m, torch.Tensor) or not m.is_cuda or m.dtype not in (torch.uint8, torch.bool):
        raise TypeError("block_mask must be a uint8 or bool GPU tensor")
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if tuple(m.shape[-2:]) != (n_blk, n_blk) or m.dim() not in (2, 3, 4):
        raise ValueError(f"block_mask must end in [{n_blk}, {n_blk}]")
    if m.stride(-1) != 1 or m.stride(-2) != n_blk:
        raise ValueError("block_mask's last two dims must be contiguous")
    if m.dim() == 2:
        sb, sh = 0, 0
    elif m.dim() == 3:
        if m.shape[0] != Hq:
            raise ValueError("a 3-d block_mask is [Hq, n_blk, n_blk]")
        sb, sh = 0, m.stride(0)
    else:
        if m.shape[0] != B or m.shape[1] != Hq:
            raise ValueError("a 4-d block_mask is [B, Hq, n_blk, n_blk]")
        sb, sh = m.stride(0), m.stride(1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require(out, torch.bfloat16, "out")
    _require(lse, torch.float32, "lse")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("out/lse have the wrong shape")
    lib = load_library()
    with _guard(q, k, v, out, lse, m):
        st = lib.fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(m), sb, sh, B, Hq, Hkv, N, d,
                                    int(bool(causal)), float(scale), _stream_ptr(q))
    _check(st, "fa_fwd_blocksparse")
    return out, lse


def bwd_workspace_bytes(B, Hq, Hkv, N, d) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None, events=None):
    """Backward attention on bf16 tensors. Returns (dq, dk, dv).

    events: optional ctypes array of 3 hipEvent_t handles; when given the call
    goes through fa_bwd_timed, which records them around its two kernels.
    """
    torch = _torch()
    # every shape first: the library sees only pointers, so an output smaller
    # than q (dq) or k (dk, dv) would be written past its end
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (lse, "lse"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv")):
        if t is not None and not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
    B, Hq, Hkv, N, d = _dims(q, k, v)
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o/dout/lse have the wrong shape")
    for t, n, want in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", v.shape)):
        if t is not None and tuple(t.shape) != tuple(want):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(want)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _require(t, torch.bfloat16, n)
    _require(lse, torch.float32, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _require(t, torch.bfloat16, n)
    need = bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace.numel() < need:
        raise ValueError(f"workspace too small: {workspace.numel()} < {need} bytes")
    lib = load_library()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(workspace), workspace.numel(), B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _stream_ptr(q))
    with _guard(q, k, v, o, dout, lse, dq, dk, dv, workspace):
        if events is None:
            _check(lib.fa_bwd(*args), "fa_bwd")
        else:
            _check(lib.fa_bwd_timed(*args, ctypes.cast(events, ctypes.c_void_p)), "fa_bwd_timed")
    return dq, dk, dv


BWD_NOALLOC_SCRATCH_BYTES = 32 << 20  # FA_BWD_NOALLOC_SCRATCH_BYTES


def bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, scale=None):
    """fa_bwd_noalloc: the backward without a workspace, for callers that cannot allocate device memory
    (the C entry point uses the library's fixed per-GPU scratch). The outputs dq, dk, dv are caller-provided
    bf16 tensors shaped like q, k, v; nothing is allocated here either. Calls that overlap on one GPU race.
    Returns (dq, dk, dv)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _dims(q, k, v)
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o/dout/lse have the wrong shape")
    for t, n, want in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", v.shape)):
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(want):
            raise ValueError(f"{n} must be a tensor of shape {tuple(want)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _require(t, torch.bfloat16, n)
    _require(lse, torch.float32, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load_library()
    with _guard(q, k, v, o, dout, lse, dq, dk, dv):
        st = lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _stream_ptr(q))
    _check(st, "fa_bwd_noalloc")
    return dq, dk, dv


def _autograd_function():
    torch = _torch()

    class FlashAttnFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            o, lse = fwd(q, k, v, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale = causal, scale
            return o

        @staticmethod
        def backward(ctx, dout):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = bwd(q, k, v, o, lse, dout.contiguous(), causal=ctx.causal, scale=ctx.scale)
            return dq, dk, dv, None, None

    return FlashAttnFunction


_FN = None


def flash_attn(q, k, v, causal=False, scale=None):
    """Differentiable exact attention on bf16 tensors (libfa forward and backward)."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _FN.apply(q, k, v, causal, scale)
