"""Throughput of the libfa attention path on one MI355X.

One step = forward + backward of exact causal attention on the workload
B=2, H=16, N=4096, d=128, bf16 storage, fp32 accumulation: fa_fwd (O, lse)
followed by fa_bwd (dQ, dK, dV recomputed from lse), on seeded i.i.d. N(0,1)
inputs already resident in device memory.

Prints one JSON line. `value` is the step's algorithmic TFLOP/s:
forward 4*B*H*N^2*d / 2 (causal) plus backward 2.5x that (five N^2*d matrix
products instead of two), divided by the measured step time. Each kernel is
also timed on its own with HIP events on the launch stream; `roofline`
describes the kernel with the largest time per step.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS  # MI355X dense fp8 (e4m3) MFMA
# FP8 forward: half its FLOP (S = Q K^T) at the fp8 rate, half (P V) at the bf16 rate
PEAK_FP8_BF16_MIX_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
WORKLOAD = dict(B=2, H=16, N=4096, d=128, causal=True, seed=4)
WARMUP_MIN_S = 2.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """Raw HIP events through the runtime library (same stream the kernels use)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value


def flops(B, H, N, d, causal):
    fwd = 4.0 * B * H * N * N * d / (2.0 if causal else 1.0)
    return fwd, 2.5 * fwd


# the sources each timed kernel is compiled from (its own file and the shared headers)
KERNEL_SOURCES = {
    "fa_fwd_bf16_kernel": ("fa_fwd_bf16.hip", "fa_common.hpp", "fa_launch.hpp"),
    "fa_bwd_dq_kernel": ("fa_bwd_bf16.hip", "fa_common.hpp", "fa_launch.hpp"),
    "fa_bwd_dkdv_kernel": ("fa_bwd_bf16.hip", "fa_common.hpp", "fa_launch.hpp"),
}


def source_digest(names=None):
    """sha256 (16 hex digits) of the named files under csrc/, or of all of them."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_online_softmax_fa_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed PMC summary, if it was taken on the kernel's current sources.

    Returns (bytes or None, provenance text)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    digest = source_digest(KERNEL_SOURCES[kernel_key])
    if not os.path.exists(path):
        return None, "no profiles/traffic.json"
    with open(path) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(kernel_key)
    if k is None:
        return None, f"profiles/traffic.json has no entry for {kernel_key}"
    if k.get("source_digest") != digest:
        return None, (f"profiles/traffic.json was taken on sources {k.get('source_digest')}, the kernel's sources "
                      f"are now {digest}: stale, not reported")
    cal = t.get("calibration", {})
    return k.get("hbm_bytes_per_launch"), (
        f"profiles/traffic.json (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE of bench.py, two runs, KiB per dispatch "
        f"scaled by the copy calibration x{cal.get('fetch_factor', float('nan')):.4f} / "
        f"x{cal.get('write_factor', float('nan')):.4f}), source digest {digest} = current sources")


PEAK_F32_TFLOPS = 157.3  # MI355X dense fp32 MFMA


def time_configs(torch, min_warmup_s):
    """Forward time of each forward workload (seeded inputs resident on the GPU, HIP events on the launch stream)."""
    import numpy as np

    import tiled_online_softmax_fa_amd as fa
    from fa_inputs import WORKLOADS, make_workload_inputs

    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    for w in WORKLOADS.values():
        if w.backward:
            continue
        inp = make_workload_inputs(w)
        if w.dtype == "bf16":
            dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
                   for n in ("q", "k", "v")}
            call, elt, peak = fa.fwd, 2, PEAK_BF16_TFLOPS
        else:
            dev = {n: torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to("cuda:0")
                   for n in ("q", "k", "v")}
            call, elt, peak = fa.fwd_f32, 4, PEAK_F32_TFLOPS
        o, lse = call(dev["q"], dev["k"], dev["v"], causal=w.causal)
        t0 = time.perf_counter()
        n = 0
        while n < 20 or time.perf_counter() - t0 < min_warmup_s:
            call(dev["q"], dev["k"], dev["v"], causal=w.causal, out=o, lse=lse)
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        K = 50
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(K):
            call(dev["q"], dev["k"], dev["v"], causal=w.causal, out=o, lse=lse)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        us = hip.ms(e0, e1) / K * 1e3
        f_fwd, _ = flops(w.B, w.Hq, w.N, w.d, w.causal)
        nbytes = (2 * w.B * w.Hq + 2 * w.B * w.Hkv) * w.N * w.d * elt + 4 * w.B * w.Hq * w.N
        tflops = f_fwd / (us * 1e-6) / 1e12
        print(json.dumps({"workload": w.name, "dtype": w.dtype, "causal": w.causal,
                          "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "avg_us": us,
                          "tflops": tflops, "frac_of_peak": tflops / peak, "peak_tflops": peak,
                          "compulsory_bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
                          "source_digest": source_digest()}), flush=True)

    time_short_sequences(torch, min_warmup_s)

    # head dim 256, and split-KV on shapes with few query tiles (seeded N(0,1) inputs, bf16): plain forward
    # vs key-range parts
    from fa_inputs import Workload

    for B, H, N, d, causal, split_list in ((2, 16, 4096, 128, False, (0,)),
                                          (2, 16, 4096, 256, True, (0,)), (2, 16, 4096, 256, False, (0,)),
                                          (1, 8, 16384, 128, True, (0, 2, 4, 8, "auto")),
                                          (1, 4, 8192, 128, False, (0, 2, 4, 8, "auto"))):
        w = Workload(f"{'splitkv_' if len(split_list) > 1 else 'fwd_'}b{B}h{H}n{N}d{d}{'_causal' if causal else ''}",
                     B, H, H, N, d, "bf16", causal, seed=9)
        inp = make_workload_inputs(w)
        dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
               for n in ("q", "k", "v")}
        o = torch.empty_like(dev["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        f_fwd, _ = flops(B, H, N, d, causal)
        for splits in split_list:
            if splits:
                ns = 0 if splits == "auto" else splits
                ws = torch.empty(fa.splitkv_workspace_bytes(B, H, H, N, d, ns), dtype=torch.uint8, device="cuda:0")
                run = lambda: fa.fwd_splitkv(dev["q"], dev["k"], dev["v"], ns, causal=causal, out=o, lse=lse,
                                             workspace=ws)
            else:
                run = lambda: fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, out=o, lse=lse)
            t0 = time.perf_counter()
            n = 0
            while n < 10 or time.perf_counter() - t0 < min(min_warmup_s, 0.5):
                run()
                n += 1
                if n % 8 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            for _ in range(20):
                run()
            hip.record(e1, stream)
            torch.cuda.synchronize()
            us = hip.ms(e0, e1) / 20 * 1e3
            tflops = f_fwd / (us * 1e-6) / 1e12
            print(json.dumps({"workload": w.name, "entry": "fa_fwd_splitkv" if splits else "fa_fwd", "n_splits": splits,
                              "avg_us": us, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
                              "source_digest": source_digest()}), flush=True)

    # block-sparse forward (128 x 128 mask blocks): work counted over the visible (query, key) pairs only
    from fa_inputs import make_block_mask

    def visible_pairs(m, N, block, causal):
        """(query, key) pairs a [n_blk, n_blk] block mask lets through (with the causal mask if set)."""
        n = m.shape[0]
        sz = np.array([min(block, N - i * block) for i in range(n)], dtype=np.int64)
        pairs = np.outer(sz, sz)
        if causal:
            lower = np.tril(np.ones((n, n), bool), -1)
            pairs = np.where(lower, pairs, 0) + np.diag(sz * (sz + 1) // 2)
        return int((m.astype(np.int64) * pairs).sum())

    for B, H, N, d, causal, kind in ((2, 16, 4096, 128, True, "band"), (2, 16, 4096, 128, False, "band"),
                                     (2, 16, 4096, 128, False, "random")):
        w = Workload(f"blocksparse_{kind}_b{B}h{H}n{N}d{d}{'_causal' if causal else ''}", B, H, H, N, d, "bf16",
                     causal, seed=9)
        inp = make_workload_inputs(w)
        dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
               for n in ("q", "k", "v")}
        mask = make_block_mask(kind, B, H, N, seed=1)
        visible = sum(visible_pairs(mask[b, h], N, 128, causal) for b in range(B) for h in range(H))
        m_dev = torch.from_numpy(mask).to("cuda:0")
        o = torch.empty_like(dev["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        run = lambda: fa.fwd_blocksparse(dev["q"], dev["k"], dev["v"], m_dev, causal=causal, out=o, lse=lse)
        t0 = time.perf_counter()
        n = 0
        while n < 10 or time.perf_counter() - t0 < min(min_warmup_s, 0.5):
            run()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(20):
            run()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        us = hip.ms(e0, e1) / 20 * 1e3
        f_vis = 4.0 * d * visible
        tflops = f_vis / (us * 1e-6) / 1e12
        print(json.dumps({"workload": w.name, "entry": "fa_fwd_blocksparse", "mask": kind,
                          "visible_fraction": visible / (B * H * N * N), "avg_us": us, "tflops": tflops,
                          "frac_of_peak": tflops / PEAK_BF16_TFLOPS, "source_digest": source_digest()}), flush=True)

    # FP8 forward (e4m3 Q, K with per-64-row scales, bf16 V) and the block-wise quantiser (HBM-bound)
    def timed(run, reps=20):
        t0 = time.perf_counter()
        n = 0
        while n < 10 or time.perf_counter() - t0 < min(min_warmup_s, 0.5):
            run()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for _ in range(reps):
            run()
        hip.record(e1, stream)
        torch.cuda.synchronize()
        return hip.ms(e0, e1) / reps * 1e3

    for B, H, N, d, causal in ((2, 16, 4096, 128, True), (2, 16, 4096, 128, False), (2, 16, 4096, 256, True)):
        w = Workload(f"fwd_fp8_b{B}h{H}n{N}d{d}{'_causal' if causal else ''}", B, H, H, N, d, "bf16", causal, seed=9)
        inp = make_workload_inputs(w)
        dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
               for n in ("q", "k", "v")}
        qc, qs = fa.quantize_fp8(dev["q"])
        kc, ks = fa.quantize_fp8(dev["k"])
        o = torch.empty_like(dev["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        us = timed(lambda: fa.fwd_fp8(qc, qs, kc, ks, dev["v"], causal=causal, out=o, lse=lse))
        f_fwd, _ = flops(B, H, N, d, causal)
        tflops = f_fwd / (us * 1e-6) / 1e12
        print(json.dumps({"workload": w.name, "entry": "fa_fwd_fp8", "avg_us": us, "tflops": tflops,
                          "frac_of_peak": tflops / PEAK_FP8_BF16_MIX_TFLOPS, "peak_tflops": PEAK_FP8_BF16_MIX_TFLOPS,
                          "peak_note": "S = Q K^T on e4m3 MFMA, P V on bf16 MFMA, half the FLOP each",
                          "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS, "source_digest": source_digest()}), flush=True)
        if causal and d == 128:
            us_q = timed(lambda: fa.quantize_fp8(dev["q"], codes=qc, scale=qs))
            qbytes = B * H * N * d * 3 + B * H * (-(-N // 64)) * 4  # read bf16, write codes and scales
            print(json.dumps({"workload": f"quantize_fp8_b{B}h{H}n{N}d{d}", "entry": "fa_quantize_fp8",
                              "avg_us": us_q, "gbs": qbytes / (us_q * 1e-6) / 1e9, "tflops": 0.0,
                              "frac_of_peak": qbytes / (us_q * 1e-6) / 1e9 / PEAK_HBM_GBS,
                              "peak_note": "fraction of HBM bandwidth", "source_digest": source_digest()}), flush=True)

    # backward at head dim 256 (the backward at d = 128 is the headline line): both kernels timed on their own
    for B, H, N, d, causal in ((2, 16, 4096, 256, True),):
        w = Workload(f"bwd_b{B}h{H}n{N}d{d}{'_causal' if causal else ''}", B, H, H, N, d, "bf16", causal, seed=9,
                     backward=True)
        inp = make_workload_inputs(w)
        dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
               for n in ("q", "k", "v", "dO")}
        o, lse = fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
        dq, dk, dv = (torch.empty_like(dev[n]) for n in ("q", "k", "v"))
        ws = torch.empty(fa.bwd_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device="cuda:0")
        K = 20
        evs = [(ctypes.c_void_p * 3)(*[hip.event() for _ in range(3)]) for _ in range(K)]
        run = lambda ev=None: fa.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["dO"], causal=causal, dq=dq, dk=dk,
                                     dv=dv, workspace=ws, events=ev)
        t0 = time.perf_counter()
        n = 0
        while n < 10 or time.perf_counter() - t0 < min(min_warmup_s, 1.0):
            run()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        for i in range(K):
            run(evs[i])
        torch.cuda.synchronize()
        dq_us = sum(hip.ms(e[0], e[1]) for e in evs) / K * 1e3
        dkdv_us = sum(hip.ms(e[1], e[2]) for e in evs) / K * 1e3
        _, f_bwd = flops(B, H, N, d, causal)
        tflops = f_bwd / ((dq_us + dkdv_us) * 1e-6) / 1e12
        print(json.dumps({"workload": w.name, "entry": "fa_bwd", "avg_us": dq_us + dkdv_us, "dq_us": dq_us,
                          "dkdv_us": dkdv_us, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
                          "dkdv_frac_of_peak": f_bwd * 0.8 / (dkdv_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                          "source_digest": source_digest()}), flush=True)
    return 0


SHORT_SEQUENCES = ((64, 16, 128, 128), (32, 16, 256, 128), (16, 16, 512, 128))  # B, H, N, d: 16-32 MiB per tensor


def time_short_sequences(torch, min_warmup_s):
    """bf16 forward on short sequences, where each (batch, head) is one or two query tiles and the work per
    byte is small: compulsory HBM bytes (Q, K, V read, O and lse written, each once) per second, against the
    8 TB/s of HBM, next to the FLOP rate."""
    import numpy as np

    import tiled_online_softmax_fa_amd as fa
    from fa_inputs import Workload, make_workload_inputs

    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    for B, H, N, d in SHORT_SEQUENCES:
        for causal in (False, True):
            w = Workload(f"fwd_short_b{B}h{H}n{N}d{d}{'_causal' if causal else ''}", B, H, H, N, d, "bf16", causal,
                         seed=9)
            inp = make_workload_inputs(w)
            dev = {n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
                   for n in ("q", "k", "v")}
            o = torch.empty_like(dev["q"])
            lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
            t0 = time.perf_counter()
            n = 0
            while n < 20 or time.perf_counter() - t0 < min(min_warmup_s, 0.5):
                fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, out=o, lse=lse)
                n += 1
                if n % 8 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            K = 50
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            for _ in range(K):
                fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, out=o, lse=lse)
            hip.record(e1, stream)
            torch.cuda.synchronize()
            us = hip.ms(e0, e1) / K * 1e3
            f_fwd, _ = flops(B, H, N, d, causal)
            nbytes = 4 * B * H * N * d * 2 + 4 * B * H * N
            gbs = nbytes / (us * 1e-6) / 1e9
            tflops = f_fwd / (us * 1e-6) / 1e12
            print(json.dumps({"workload": w.name, "entry": "fa_fwd", "avg_us": us, "compulsory_bytes": nbytes,
                              "gbs": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS, "tflops": tflops,
                              "frac_of_peak": tflops / PEAK_BF16_TFLOPS, "source_digest": source_digest()}),
                  flush=True)
    return 0


COPY_BYTES = 1 << 29  # 512 MiB read and 512 MiB written per calibration copy
COPY_LAUNCHES = 4


def copy_calibration(torch):
    """A plain device-to-device copy of known size, profiled to scale the byte counters."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(COPY_LAUNCHES):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": COPY_LAUNCHES}), flush=True)
    return 0


def _counter_per_dispatch(path, counter):
    """Mean value of one counter per dispatch, per kernel name, from a rocprofv3 counter_collection CSV."""
    import csv
    from collections import defaultdict

    tot, disp = defaultdict(float), defaultdict(set)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            tot[name] += float(r["Counter_Value"])
            disp[name].add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """profiles/traffic.json: HBM bytes per launch of each kernel (FETCH_SIZE + WRITE_SIZE, KiB per dispatch),
    each counter scaled so that it reads the known size on a plain copy kernel."""
    def copy_reading(path, counter):
        per = _counter_per_dispatch(path, counter)
        name = max(per, key=per.get)  # the copy is by far the largest dispatch of the calibration run
        return name, per[name] * 1024.0

    cname, cf = copy_reading(copy_fetch_csv, "FETCH_SIZE")
    _, cw = copy_reading(copy_write_csv, "WRITE_SIZE")
    f_fetch, f_write = COPY_BYTES / cf, COPY_BYTES / cw
    fetch = _counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _counter_per_dispatch(write_csv, "WRITE_SIZE")
    kernels = {}
    for key in ("fa_fwd_bf16_kernel", "fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"):
        fk = [n for n in fetch if key in n]
        wk = [n for n in write if key in n]
        if not fk or not wk:
            continue
        rd = fetch[fk[0]] * 1024.0 * f_fetch
        wr = write[wk[0]] * 1024.0 * f_write
        kernels[key] = {"hbm_bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                        "source_digest": source_digest(KERNEL_SOURCES[key])}
    out = {
        "source_digest": source_digest(),
        "workload": "causal attention fwd+bwd, B=2 H=16 N=4096 d=128 (bench.py default)",
        "calibration": {"kernel": cname, "copy_bytes": COPY_BYTES, "fetch_factor": f_fetch, "write_factor": f_write},
        "kernels": kernels,
    }
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, with its family and model numbers (else the machine
    type)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break  # the first processor's block is enough
                    continue
                key, val = (x.strip() for x in line.split(":", 1))
                if key in ("model name", "cpu family", "model") and key not in fields:
                    fields[key] = val
    except OSError:
        pass
    if "model name" not in fields:
        return platform.processor() or platform.machine()
    extra = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model") if k in fields)
    return f"{fields['model name']} ({extra})" if extra else fields["model name"]


def cpu_baseline(inputs, budget_s=10.0):
    """Time the fp64 oracle (fwd + bwd per head) on a bounded sample of the same workload, with the BLAS
    thread pool set to the CPUs this process may run on."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention_bwd_head, attention_fwd

    w = WORKLOAD
    scale = w["d"] ** -0.5
    heads = [(b, h) for b in range(w["B"]) for h in range(w["H"])]
    n_cpus = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=n_cpus, user_api="blas"):
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        t0 = time.perf_counter()
        done = 0
        for b, h in heads:
            q, k, v, dO = (inputs[n][b:b + 1, h:h + 1] for n in ("q", "k", "v", "dO"))
            attention_fwd(q, k, v, True, scale)
            attention_bwd_head(q[0, 0], k[0, 0], v[0, 0], dO[0, 0], True, scale)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        secs = time.perf_counter() - t0
    f, b_ = flops(1, done, w["N"], w["d"], True)
    return {
        "value": (f + b_) / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (batch, head) pairs of the same workload, fwd + bwd each, "
                  f"fp64 NumPy with the full N x N matrix, {secs:.1f} s",
        "cpu": cpu_model(),
        "affinity_cpus": n_cpus,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-warmup-s", type=float, default=WARMUP_MIN_S,
                    help="keep warming up until this many seconds have passed (0 for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for scaling the HBM byte counters)")
    ap.add_argument("--short-seq", action="store_true",
                    help="only the short-sequence forward cases of --configs (HBM-rate figures)")
    ap.add_argument("--configs", action="store_true",
                    help="only time the forward on every forward workload of fa_inputs.WORKLOADS, on head dim "
                         "256, split-KV, block-sparse and FP8 shapes, the FP8 quantiser, and the backward at head "
                         "dim 256 (one JSON line each; not the headline line)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs "
                         "of a short bench run and of a --copy-calibration run (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_from:
        return write_traffic(*args.traffic_from)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this library runs a single "
              "MI355X; sharding across GPUs is not built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        return copy_calibration(torch)
    if args.configs:
        return time_configs(torch, args.min_warmup_s)
    if args.short_seq:
        return time_short_sequences(torch, args.min_warmup_s)

    import tiled_online_softmax_fa_amd as fa
    from fa_inputs import make_inputs

    w = WORKLOAD
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    scale = d ** -0.5
    log(f"generating inputs B{B} H{H} N{N} d{d} causal seed {w['seed']}")
    inputs = make_inputs(B, H, H, N, d, "bf16", w["seed"], backward=True)
    dev = {n: torch.from_numpy(inputs[n + "_bits"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
           for n in ("q", "k", "v", "dO")}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = (torch.empty_like(dev[n]) for n in ("q", "k", "v"))
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device="cuda:0")

    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    K = args.steps
    ev_f = [(hip.event(), hip.event()) for _ in range(K)]
    ev_b = [(ctypes.c_void_p * 3)(*[hip.event() for _ in range(3)]) for _ in range(K)]
    ev_all = (hip.event(), hip.event())

    def step(i=None):
        if i is not None:
            hip.record(ev_f[i][0], stream)
        fa.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, out=o, lse=lse)
        if i is not None:
            hip.record(ev_f[i][1], stream)
        fa.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["dO"], causal=causal, scale=scale, dq=dq, dk=dk, dv=dv,
               workspace=ws, events=ev_b[i] if i is not None else None)

    # W steps, then more until the warm-up has run for WARMUP_MIN_S: the
    # GPU clocks ramp up over the first second or so of sustained work
    log(f"warmup {args.warmup} steps (at least {args.min_warmup_s} s)")
    t_w = time.perf_counter()
    n_w = 0
    while n_w < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        step()
        n_w += 1
        if n_w % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"warmup done: {n_w} steps in {time.perf_counter() - t_w:.2f} s")
    log(f"timing {K} steps")
    hip.record(ev_all[0], stream)
    for i in range(K):
        step(i)
    hip.record(ev_all[1], stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(*ev_all)
    ms_step = total_ms / K
    kern_ms = {
        "fa_fwd_bf16_kernel": sum(hip.ms(a, b) for a, b in ev_f) / K,
        "fa_bwd_dq_kernel": sum(hip.ms(e[0], e[1]) for e in ev_b) / K,
        "fa_bwd_dkdv_kernel": sum(hip.ms(e[1], e[2]) for e in ev_b) / K,
    }
    f_fwd, f_bwd = flops(B, H, N, d, causal)
    elt = 2
    qkv_bytes = B * H * N * d * elt
    # algorithmic work per launch of each kernel
    # The backward's algorithmic work is 5 products (S, dP, dV, dK, dQ: 2.5x the
    # forward). The dK/dV kernel does 4 of them; the dQ kernel does the 5th and
    # recomputes S and dP for it (executed, not counted as algorithmic work).
    work = {
        "fa_fwd_bf16_kernel": ("mfma", f_fwd),
        "fa_bwd_dkdv_kernel": ("mfma", f_bwd * 4 / 5),
        "fa_bwd_dq_kernel": ("mfma", f_bwd * 1 / 5),
    }
    executed = {"fa_bwd_dq_kernel": f_bwd * 3 / 5}
    dominant = max(kern_ms, key=kern_ms.get)
    bound, units = work[dominant]
    avg_s = kern_ms[dominant] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = units / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = units / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    traffic, traffic_source = measured_traffic(dominant)
    roofline = {"bound": bound, "kernel": dominant, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic, "traffic_source": traffic_source,
                "avg_launch_us": kern_ms[dominant] * 1e3}
    kernels = {}
    for name, ms in kern_ms.items():
        b_, u_ = work[name]
        if b_ == "mfma":
            kernels[name] = {"avg_us": ms * 1e3, "tflops": u_ / (ms * 1e-3) / 1e12,
                             "frac_of_peak": u_ / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
            if name in executed:
                kernels[name]["executed_tflops"] = executed[name] / (ms * 1e-3) / 1e12
        else:
            kernels[name] = {"avg_us": ms * 1e3, "gbs": u_ / (ms * 1e-3) / 1e9,
                             "frac_of_peak": u_ / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    bwd_ms = kern_ms["fa_bwd_dkdv_kernel"] + kern_ms["fa_bwd_dq_kernel"]
    result = {
        "metric": "attention fwd/bwd TFLOPS and % of MI355X bf16 MFMA peak, d=128 N=4096",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) q, k, v, dO rounded to bf16 (RNE)",
        "config": {"workload": "causal attention fwd+bwd, B=2 H=16 N=4096 d=128, bf16 storage, fp32 accumulation",
                   "B": B, "H": H, "N": N, "d": d, "causal": causal, "scale": scale},
        "pct_of_peak": value / PEAK_BF16_TFLOPS * 100,
        "fwd_tflops": f_fwd / (kern_ms["fa_fwd_bf16_kernel"] * 1e-3) / 1e12,
        "fwd_pct_of_peak": f_fwd / (kern_ms["fa_fwd_bf16_kernel"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS * 100,
        "bwd_tflops": f_bwd / (bwd_ms * 1e-3) / 1e12,
        "bwd_pct_of_peak": f_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS * 100,
        "kernels": kernels,
        "roofline": roofline,
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(inputs)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
