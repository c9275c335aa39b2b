#!/usr/bin/env python3
"""Throughput of the causal attention hot path (forward + backward) on one GPU.

One step = the forward of every layer (0 .. L-1) followed by the backward of
every layer (L-1 .. 0), each layer with its own resident input buffers, on
the GPT-2 124M attention shape: B=12, H=12, T=1024, hs=64, bf16, 12 layers,
q/k/v ~ N(0,1) x 0.5 and dO ~ N(0,1) (seeded, synthetic).

FLOP accounting (the pages' attention term of the MFU estimate, 12 H hs T per
token per layer with the backward at twice the forward, restricted to the
causal pairs j <= i, P_c = T (T + 1) / 2 per (b, h)):
    forward 4 hs P_c B H, backward 8 hs P_c B H.

Prints one JSON line.  `roofline` is for the dominant kernel (the one with the
largest mean duration): its algorithmic FLOP per launch / that mean duration,
measured with HIP events recorded on the launch stream inside the timed steps.
Each timed step brackets the three kernels of one layer with events (layer
s mod L in step s, so every layer is sampled); bracketing every launch would
itself cost about a tenth of the step time.  The events are created with
hipEventDisableSystemFence: timing only, without the cache writeback and
invalidation of a default event, which would slow the kernels they bracket.
Algorithmic FLOP per causal pair and kernel: forward 4 hs (Q K^T and P V);
dK/dV kernel 6 hs (dO V^T, P^T dO, dS^T Q; its Q K^T is recomputation); dQ
kernel 2 hs (dS K; its Q K^T and dO V^T are recomputation).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
Also reported: the forward and backward sequences of a step (events around
the L forward launches and around the L backward pairs: median and minimum
over the timed steps); the throughput under the FlashAttention-style count,
which charges the backward 10 hs per pair (its recomputation of S); and, after
the timed steps, a measured dense bf16 matrix-multiply rate (torch.matmul,
i.e. the vendor GEMM library, on 8192^3) and a measured device-copy bandwidth
at the run's clocks, next to the published peaks.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0
# Workloads (synthetic, seeded; the default is the GPT-2 124M shape the metric
# is quoted on).  bound: what limits the dominant kernel at that shape.
WORKLOADS = {
    "gpt2-124m": dict(B=12, H=12, T=1024, hs=64, layers=12, qkv_scale=0.5, bound="mfma",
                      label="GPT-2 124M causal attention, fwd+bwd, 12 layers"),
    "char-level": dict(B=64, H=6, T=256, hs=64, layers=6, qkv_scale=1.0, bound="hbm",
                       label="char-level GPT causal attention, fwd+bwd, 6 layers"),
    "narrow-t128": dict(B=8, H=12, T=128, hs=32, layers=12, qkv_scale=1.0, bound="hbm",
                        label="narrow-head causal attention (hs 32), fwd+bwd, 12 layers"),
    "narrow-t256": dict(B=8, H=12, T=256, hs=32, layers=12, qkv_scale=1.0, bound="hbm",
                        label="narrow-head causal attention (hs 32), fwd+bwd, 12 layers"),
    "gpt2-xl": dict(B=12, H=25, T=1024, hs=64, layers=48, qkv_scale=1.0, bound="mfma",
                    label="GPT-2 XL-size causal attention (25 heads), fwd+bwd, 48 layers"),
}
CSRC = os.path.join(ROOT, "causal_self_attention_sdpa_amd", "csrc")
# name -> (kernel symbol, source file, algorithmic FLOP per causal pair / hs,
#          algorithmic bytes per launch in units of one (B,H,T,hs) bf16 tensor, and of one
#          (B,H,T) fp32 row vector)
KERNELS = {
    "fwd": ("fwd16_kernel<{E}, {hs}, false, false>", "mfma16_fwd.hip", 4, 4, 1),  # q k v in; o, lse out
    "dq": ("dq16_kernel<{E}, {hs}, false, 0>", "mfma16_bwd.hip", 2, 6, 1),  # q k v o dO lse in; dq out
    "dkdv": ("dkdv16_kernel<{E}, {hs}, false, false>", "mfma16_bwd.hip", 6, 6, 0),  # q k v dO in; dk dv out
}
# With attention dropout (--dropout): the forward kernel, and the backward as
# one call (its dQ and dK/dV kernels back to back), timed as one unit.
DROP_KERNELS = {
    "fwd_dropout": ("fwd16_kernel<{E}, {hs}, false, true>", "mfma16_fwd.hip", 4, 4, 1),
    "bwd_dropout": ("dq16_kernel<{E}, {hs}, false, 2> + dkdv16_kernel<{E}, {hs}, false, true>",
                    "mfma16_bwd.hip", 8, 8, 1),  # q k v o dO lse in; dq dk dv out
}


def flops(B, H, T, hs, bwd_per_pair=8):
    pc = T * (T + 1) // 2
    return 4 * hs * pc * B * H, bwd_per_pair * hs * pc * B * H


def measured_peaks(torch, dev):
    """Dense bf16 GEMM rate (torch.matmul, 8192^3) and device-copy bandwidth
    (1 GiB read + 1 GiB written) at this run's clocks."""
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * reps / (time.perf_counter() - t0) / 1e12
    del a, b
    x = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    copy = 2.0 * x.numel() * 4 * reps / (time.perf_counter() - t0) / 1e9
    del x, y
    # a loop of independent bf16 MFMAs on register operands (the library's probe)
    import causal_self_attention_sdpa_amd as ga
    lib = ga.load_library()
    blocks, iters = 2048, 128
    sink = torch.empty(4 * blocks, dtype=torch.float32, device=dev)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert lib.gattn_probe_mfma_bf16(sink.data_ptr(), blocks, iters, sp) == 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        lib.gattn_probe_mfma_bf16(sink.data_ptr(), blocks, iters, sp)
    torch.cuda.synchronize()
    mfma = blocks * 4 * iters * 8 * 32768 * 5 / (time.perf_counter() - t0) / 1e12
    # the vector ALU beside the matrix core (the library's issue probe): cost of
    # a wave64 vector instruction in MFMA cycles (a saturated 32x32x16 bf16 MFMA,
    # two wavefronts per SIMD, taken as 32), with two or one issuing wavefronts
    # per SIMD, and MFMAs of one wavefront beside v_fma_f32 of another
    pb, mi, vi = 256, 4000, 4000
    sink8 = torch.empty(8 * pb, dtype=torch.float32, device=dev)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def t_issue(m_it, v_it, kind, roles, reps=5):
        # best of `reps` launches, each bracketed by events on the launch stream
        best = float("inf")
        for rep in range(reps + 1):
            ev0.record()
            assert lib.gattn_probe_issue(sink8.data_ptr(), pb, m_it, v_it, kind, roles, sp) == 0
            ev1.record()
            ev1.synchronize()
            if rep:
                best = min(best, ev0.elapsed_time(ev1) * 1e-3)
        return best

    per_mfma = t_issue(mi, 0, 0, 1 | 4) / (2 * mi * 4)
    valu = {}
    for kind, name in ((0, "v_fma_f32"), (1, "v_mul_f32"), (2, "v_exp_f32")):
        two = t_issue(0, vi, kind, 2 | 8) / (2 * vi * 16)
        one = t_issue(0, vi, kind, 2) / (vi * 16)
        valu[name] = {"two_wavefronts": round(32 * two / per_mfma, 2),
                      "one_wavefront": round(32 * one / per_mfma, 2)}
    coexec = {"mfma_alone_ms": round(1e3 * t_issue(mi, 0, 0, 1), 4),
              "fma_alone_ms": round(1e3 * t_issue(0, vi, 0, 8), 4),
              "both_ms": round(1e3 * t_issue(mi, vi, 0, 1 | 8), 4)}
    return {"bf16_gemm_tflops": round(gemm, 1), "copy_gbs": round(copy, 1),
            "mfma_loop_bf16_tflops": round(mfma, 1),
            "valu_cycles_per_instruction": valu, "mfma_beside_valu": coexec,
            "issue_probe": ("gattn_probe_issue: 256 x 8 wavefronts; 4000 x 4 MFMA 32x32x16 or "
                            "4000 x 16 vector instructions per wavefront; cycles in MFMA units "
                            "(32 per MFMA); mfma_beside_valu: MFMAs on wavefronts 0-3, v_fma_f32 "
                            "on 4-7, alone and together"),
            "gemm": "torch.matmul bf16 8192x8192x8192", "copy": "1 GiB device-to-device",
            "mfma_loop": "gattn_probe_mfma_bf16: 2048 x 4 wavefronts x 128 x 8 MFMA 32x32x16"}


def source_digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(name: str, tag: str):
    """HBM bytes per launch of kernel `name` from the committed rocprofv3
    counter summary (profiles/<name>_<tag>_traffic.txt), or None when that
    summary is absent or was taken on a different version of the kernel
    source."""
    path = os.path.join(ROOT, "profiles", f"{name}_{tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    src = {**KERNELS, **DROP_KERNELS}[name][1]
    if not m or not t or m.group(1) != source_digest(os.path.join(CSRC, src)):
        return None
    return float(t.group(1))


def cpu_baseline(host_layers, scale, nslices: int, dropout: float = 0.0):
    """The CPU oracle (as it stands) on the first `nslices` (layer, b, h)
    slices of the workload, all host threads of this process's CPU share (at
    most 16).  With dropout, the oracle's dropout path (numpy, one thread per
    its BLAS) on the same slices with the bench's seed and per-layer offsets."""
    import numpy as np

    import oracle

    B, H, T, hs = host_layers[0]["q"].shape
    idx = [(l, b, h) for l in range(len(host_layers)) for b in range(B) for h in range(H)]
    idx = idx[:nslices]
    sel = {n: np.stack([host_layers[l][n][b, h] for l, b, h in idx])[:, None]
           for n in ("q", "k", "v", "do")}
    threads = min(16, len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    if dropout > 0.0:
        from oracle import dropout as od
        for l in sorted({l for l, _, _ in idx}):
            sl = [(b, h) for ll, b, h in idx if ll == l]
            x = host_layers[l]
            od.attention_backward_dropout(x["q"], x["k"], x["v"], x["do"], scale, dropout, 0x5EED,
                                          l, slices=sl)
        threads = int(os.environ.get("OMP_NUM_THREADS", threads))
    else:
        oracle.attention_backward(sel["q"], sel["k"], sel["v"], sel["do"], scale,
                                  nthreads=threads)
    dt = time.perf_counter() - t0
    ff, fb = flops(len(idx), 1, T, hs)
    nl = idx[-1][0] + 1
    single = None
    if dropout == 0.0:
        # one thread on a tenth of the sample
        n1 = max(1, len(idx) // 10)
        t1 = time.perf_counter()
        oracle.attention_backward(sel["q"][:n1], sel["k"][:n1], sel["v"][:n1], sel["do"][:n1],
                                  scale, nthreads=1)
        d1 = time.perf_counter() - t1
        f1f, f1b = flops(n1, 1, T, hs)
        single = {"value": round((f1f + f1b) / d1 / 1e12, 6), "cores": 1, "seconds": round(d1, 3),
                  "sample": f"the first {n1} of those slices"}
    return {"value": round((ff + fb) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3), "single_thread": single,
            "hardware_concurrency": oracle.hardware_threads(),
            "sample": f"{len(idx)} of the {B * H * len(host_layers)} (layer,b,h) slices "
                      f"(layers 0..{nl - 1}; T={T}, hs={hs}), forward+backward in float64"
                      f"{f' with dropout p={dropout}' if dropout > 0 else ''}, "
                      f"FLOP counted as on the GPU"}


class HipTimer:
    """Timing events of the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence (recording one does not write back and
    invalidate the caches)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = self.ct.c_void_p()
        st = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
        return e

    def record(self, e, stream_ptr: int):
        st = self.hip.hipEventRecord(e, stream_ptr)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        st = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value


def decode_main(args) -> int:
    """--mode decode: one decode step per layer at the GPT-2 shape (B=12, H=12,
    hs=64, 12 layers): the newest token against Tk = args.kv_len cached keys and
    values (gattn_fwd_decode), HBM-bound; value = bytes of q, k, v read and o
    written per second.  --mode generate: the pages' generate at the character-
    level shape (B=1, 6 heads, hs 64, 6 layers, block size 256): the whole
    forward recomputed at every prefix length T = 1..256 (gattn_fwd, no lse),
    against decoding the newest token with the earlier keys and values kept."""
    import numpy as np
    import torch

    import causal_self_attention_sdpa_amd as ga
    import synth_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    dcode = ga.BF16 if args.dtype == "bf16" else ga.F16
    lib = ga.load_library()
    sp = torch.cuda.current_stream().cuda_stream
    p = lambda x: x.data_ptr()
    timer = HipTimer()

    def inputs(B, H, T, hs, l, tag):
        x = si.attention_inputs(B, H, T, hs, args.dtype, seed=2024, workload=tag, layer=l)
        return {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in x.items()}

    if args.mode == "decode":
        B, H, hs, L, Tk = 12, 12, 64, 12, args.kv_len
        scale = 1.0 / math.sqrt(hs)
        layers = []
        for l in range(L):
            t = inputs(B, H, Tk, hs, l, "decode-gpt2")
            t["q1"] = t["q"][:, :, Tk - 1:].contiguous()
            t["o"] = torch.empty_like(t["q1"])
            nb = ga.gattn_fwd_decode_workspace_bytes(B, H, 1, Tk, hs, dcode)
            t["ws"] = torch.empty(nb, dtype=torch.uint8, device=dev)
            layers.append(t)
        calls = [(lib.gattn_fwd_decode, (p(t["q1"]), p(t["k"]), p(t["v"]), p(t["o"]), None, B, H,
                                         1, Tk, hs, scale, dcode, None, None, None, p(t["ws"]),
                                         t["ws"].numel(), sp)) for t in layers]
        ev = [(timer.event(), timer.event()) for _ in range(args.steps)]

        def step(rec):
            for l, (fn, a) in enumerate(calls):
                if rec is not None and l == rec % L:
                    timer.record(ev[rec][0], sp)
                if fn(*a) != 0:
                    raise RuntimeError("gattn_fwd_decode failed")
                if rec is not None and l == rec % L:
                    timer.record(ev[rec][1], sp)

        for _ in range(args.warmup):
            step(None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for st in range(args.steps):
            step(st)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        per_call = float(np.mean([timer.elapsed_ms(a, b) for a, b in ev])) * 1e3
        alg = (2 * Tk + 2) * B * H * hs * 2  # k, v read; q read, o written
        out = {"metric": f"decode attention HBM GB/s (one token, {Tk} cached keys) at B{B} H{H} hs{hs}",
               "value": round(alg * L / dt / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": args.dtype, "data": "synthetic",
               "config": {"workload": "GPT-2 124M attention, one decode step per layer",
                          "B": B, "H": H, "Tq": 1, "Tk": Tk, "hs": hs, "layers": L,
                          "parallelism": "single GPU"},
               "us_per_call": round(per_call, 2),
               "roofline": {"kernel": "one gattn_fwd_decode call (dec1_kernel for one new token, "
                                      "plus dec16_combine when the keys are split)",
                            "bound": "hbm", "achieved": round(alg / (per_call * 1e-6) / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(alg / (per_call * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": None, "algorithmic_bytes_per_launch": alg}}
        print(json.dumps(out), flush=True)
        return 0

    # generate: the pages' recompute-everything loop vs decoding with kept keys/values
    B, H, hs, L, Tmax = 1, 6, 64, 6, 256
    scale = 1.0 / math.sqrt(hs)
    layers = [inputs(B, H, Tmax, hs, l, "generate-char") for l in range(L)]
    for t in layers:
        t["o"] = torch.empty_like(t["q"])
        t["ws"] = torch.empty(max(1, ga.gattn_fwd_decode_workspace_bytes(B, H, 1, Tmax, hs, dcode)),
                              dtype=torch.uint8, device=dev)
        t["o1"] = torch.empty((B, H, 1, hs), dtype=tdt, device=dev)
    # prefix views (contiguous per prefix length T: rows 0..T-1 of each slice)
    pre = [[{n: t[n][:, :, :T].contiguous() for n in ("q", "k", "v")} for T in range(1, Tmax + 1)]
           for t in layers]
    kv_strides = (ctypes.c_int64 * 3)(H * Tmax * hs, Tmax * hs, hs)  # also row T-1 of q

    def recompute(stream=sp):
        for T in range(1, Tmax + 1):
            for l in range(L):
                x = pre[l][T - 1]
                if lib.gattn_fwd(p(x["q"]), p(x["k"]), p(x["v"]), p(layers[l]["o"]), None, B, H, T,
                                 hs, scale, dcode, stream) != 0:
                    raise RuntimeError("gattn_fwd failed")

    def cached(stream=sp):
        for T in range(1, Tmax + 1):
            for l in range(L):
                t = layers[l]
                q1 = t["q"][:, :, T - 1:T]
                if lib.gattn_fwd_decode(p(q1), p(t["k"]), p(t["v"]), p(t["o1"]), None, B, H, 1, T,
                                        hs, scale, dcode, kv_strides, kv_strides, None,
                                        p(t["ws"]), t["ws"].numel(), stream) != 0:
                    raise RuntimeError("gattn_fwd_decode failed")

    def graphed(fn):
        # the whole 256-token loop captured once as a HIP graph (the library only
        # enqueues kernels, so it can be captured); replaying it removes the
        # per-call host cost of this Python loop
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(torch.cuda.current_stream().cuda_stream)
        return g.replay

    res = {}
    for name, fn in (("recompute", recompute), ("cached", cached),
                     ("recompute_graph", graphed(recompute)), ("cached_graph", graphed(cached))):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = max(1, args.steps // 10)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / reps
    out = {"metric": "attention time to generate 256 tokens, char-level shape (B1 H6 hs64, 6 layers)",
           "value": round(res["recompute"] * 1e3, 3), "unit": "ms", "n_gpus": 1,
           "steps": max(1, args.steps // 10), "warmup": max(1, args.warmup),
           "ms_per_step": round(res["recompute"] * 1e3, 3), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
           "config": {"workload": "the pages' generate: whole forward at every prefix length",
                      "B": B, "H": H, "hs": hs, "layers": L, "block_size": Tmax,
                      "parallelism": "single GPU"},
           "cached_decode_ms": round(res["cached"] * 1e3, 3),
           "graph_ms": {"recompute": round(res["recompute_graph"] * 1e3, 3),
                        "cached": round(res["cached_graph"] * 1e3, 3)},
           "us_per_layer_call": {k: round(v / (Tmax * L) * 1e6, 2) for k, v in res.items()},
           "roofline": None}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--mode", choices=("train", "decode", "generate"), default="train",
                    help="train: forward + backward (the metric); decode: one new token per "
                         "layer against --kv-len kept keys; generate: the pages' generate loop")
    ap.add_argument("--kv-len", type=int, default=1024)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="gpt2-124m")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="override the workload's T (train mode; a scaling probe, not a workload "
                         "of the pages)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's B (train mode)")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default="bf16",
                    help="16-bit storage type of q, k, v, o and the gradients")
    ap.add_argument("--layout", choices=("contiguous", "fused", "copies"), default="contiguous",
                    help="contiguous: (B,H,T,hs) tensors (the metric); fused: q, k, v read in "
                         "place from a GPT block's (B,T,3C) projection output, y and dy (B,T,C), "
                         "dqkv (B,T,3C), through the strided entry points; copies: the "
                         "contiguous kernels plus the transposes a caller of the contiguous "
                         "entry points needs around them")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="attention dropout probability (train mode, contiguous layout); the "
                         "mask is drawn per layer and step from a seed and an offset")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-slices", type=int, default=400,
                    help="(layer,b,h) slices the CPU oracle baseline runs (0 to skip)")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the measured GEMM / copy peaks after the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the "
              "attention core shards over (b, h) with no exchange between GPUs).",
              file=sys.stderr)
        return 2

    if args.mode != "train":
        return decode_main(args)

    import numpy as np
    import torch

    import causal_self_attention_sdpa_amd as ga
    import synth_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = 1 << 28  # 256 MiB of float32 read and written once
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}))
        return 0

    tdt = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    dcode = ga.BF16 if args.dtype == "bf16" else ga.F16
    W = dict(WORKLOADS[args.workload])
    if args.seq_len or args.batch:
        W["T"] = args.seq_len or W["T"]
        W["B"] = args.batch or W["B"]
        W["label"] += f" (B, T overridden to {W['B']}, {W['T']})"
    B, H, T, hs, L = W["B"], W["H"], W["T"], W["hs"], W["layers"]
    tag = f"b{B}h{H}t{T}"
    metric = f"causal attention fwd+bwd TFLOP/s at B{B} H{H} T{T} hs{hs}; % of bf16 MFMA peak"
    scale = 1.0 / math.sqrt(hs)
    print(f"[bench] generating {L} layers of seeded inputs {B}x{H}x{T}x{hs}", file=sys.stderr,
          flush=True)
    layers = []
    host = []  # host copies of the layers the CPU baseline samples
    for l in range(L):
        x = si.attention_inputs(B, H, T, hs, args.dtype, seed=2024,
                                workload=f"{args.workload}-attn", layer=l,
                                qkv_scale=W["qkv_scale"])
        if l * B * H < args.cpu_slices:
            host.append(x)
        t = {n: torch.from_numpy(a).to(dev).to(tdt) for n, a in x.items()}
        t["o"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        for g in ("dq", "dk", "dv"):
            t[g] = torch.empty_like(t["q"])
        layers.append(t)
        if B * H * T * hs >= 1 << 26:  # long sequences: report progress while generating
            print(f"[bench] layer {l} generated", file=sys.stderr, flush=True)
    drop = args.dropout > 0.0
    ws = torch.empty(ga.gattn_bwd_workspace_bytes(B, H, T, hs, dcode), dtype=torch.uint8,
                     device=dev)
    if drop:
        # Each layer's forward stores its keep decisions (one bit per causal
        # pair, saved for the backward like lse); its backward reads them.
        for t in layers:
            t["keep"] = torch.empty(ga.gattn_dropout_keep_bytes(B, H, T), dtype=torch.uint8,
                                    device=dev)
    stream = torch.cuda.current_stream()
    timer = HipTimer()
    if drop and args.layout != "contiguous":
        print("--dropout is measured with the contiguous layout only", file=sys.stderr)
        return 2
    KT = DROP_KERNELS if drop else KERNELS
    ev = {k: [(timer.event(), timer.event()) for _ in range(args.steps)] for k in KT}
    seq = [(timer.event(), timer.event(), timer.event()) for _ in range(args.steps)]

    # C-ABI argument tuples, marshalled once: the timed loop is nothing but
    # library calls (and event records), so the host keeps ahead of the GPU.
    lib = ga.load_library()
    sp = stream.cuda_stream
    p = lambda x: x.data_ptr()
    wsb = ws.numel()
    call = []
    for l, t in enumerate(layers):
        if drop:
            # seed fixed, offset = layer: each layer draws its own mask
            pd, seed, off = args.dropout, 0x5EED, l
            call.append({
                "fwd_dropout": (lib.gattn_fwd_dropout,
                                (p(t["q"]), p(t["k"]), p(t["v"]), p(t["o"]), p(t["lse"]), B, H, T,
                                 hs, scale, dcode, pd, seed, off, p(t["keep"]), None, None, sp)),
                "bwd_dropout": (lib.gattn_bwd_dropout,
                                (p(t["q"]), p(t["k"]), p(t["v"]), p(t["o"]), p(t["do"]),
                                 p(t["lse"]), p(t["dq"]), p(t["dk"]), p(t["dv"]), B, H, T, hs,
                                 scale, dcode, pd, seed, off, p(t["keep"]), p(ws), wsb, None, None,
                                 None, sp)),
            })
            continue
        call.append({
            "fwd": (lib.gattn_fwd, (p(t["q"]), p(t["k"]), p(t["v"]), p(t["o"]), p(t["lse"]),
                                    B, H, T, hs, scale, dcode, sp)),
            "dq": (lib.gattn_bwd_dq, (p(t["q"]), p(t["k"]), p(t["v"]), p(t["o"]), p(t["do"]),
                                      p(t["lse"]), p(t["dq"]), B, H, T, hs, scale, dcode, p(ws),
                                      wsb, sp)),
            "dkdv": (lib.gattn_bwd_dkdv, (p(t["q"]), p(t["k"]), p(t["v"]), p(t["do"]),
                                          p(t["dk"]), p(t["dv"]), B, H, T, hs, scale, dcode,
                                          p(ws), wsb, sp)),
        })

    def run(l, name, idx):
        fn, a = call[l][name]
        if idx is not None and name in ev:
            timer.record(ev[name][idx][0], sp)
        st = fn(*a)
        if idx is not None and name in ev:
            timer.record(ev[name][idx][1], sp)
        if st != 0:
            raise RuntimeError(f"{name} failed with status {st}")

    if args.layout != "contiguous":
        C = H * hs
        st = lambda *v: (ctypes.c_int64 * 3)(*v)
        s_qkv, s_bc = st(T * 3 * C, hs, 3 * C), st(T * C, hs, C)
        to_btc = lambda a: a.transpose(1, 2).reshape(B, T, C)
        for t in layers:
            t["qkv"] = torch.cat([to_btc(t[n]) for n in ("q", "k", "v")], dim=2).contiguous()
            t["dy"] = to_btc(t["do"]).contiguous()
            t["y"] = torch.empty((B, T, C), dtype=tdt, device=dev)
            t["dqkv"] = torch.empty_like(t["qkv"])
            for n in ("q", "k", "v", "do", "o", "dq", "dk", "dv"):
                t[n] = None if args.layout == "fused" else t[n]
        eb = 2  # bytes per element

        def fwd_fused(t):
            a = t["qkv"].data_ptr()
            return lib.gattn_fwd_strided(a, a + C * eb, a + 2 * C * eb, p(t["y"]), p(t["lse"]),
                                         B, H, T, hs, scale, dcode, s_qkv, s_bc, sp)

        def bwd_fused(t):
            a, g = t["qkv"].data_ptr(), t["dqkv"].data_ptr()
            return lib.gattn_bwd_strided(a, a + C * eb, a + 2 * C * eb, p(t["y"]), p(t["dy"]),
                                         p(t["lse"]), g, g + C * eb, g + 2 * C * eb, B, H, T, hs,
                                         scale, dcode, p(ws), wsb, s_qkv, s_bc, s_qkv, sp)

        def fwd_copies(t):
            # what a caller of the contiguous entry points does around them
            qkv = t["qkv"].view(B, T, 3, H, hs).permute(2, 0, 3, 1, 4).contiguous()
            t["q"], t["k"], t["v"] = qkv[0], qkv[1], qkv[2]
            r = lib.gattn_fwd(p(t["q"]), p(t["k"]), p(t["v"]), p(t["o"]), p(t["lse"]), B, H, T,
                              hs, scale, dcode, sp)
            t["y"].copy_(to_btc(t["o"]))
            return r

        def bwd_copies(t):
            t["do"] = t["dy"].view(B, T, H, hs).transpose(1, 2).contiguous()
            r = lib.gattn_bwd(p(t["q"]), p(t["k"]), p(t["v"]), p(t["o"]), p(t["do"]),
                              p(t["lse"]), p(t["dq"]), p(t["dk"]), p(t["dv"]), B, H, T, hs,
                              scale, dcode, p(ws), wsb, sp)
            t["dqkv"].copy_(torch.stack((t["dq"], t["dk"], t["dv"]), dim=2)
                            .permute(0, 3, 2, 1, 4).reshape(B, T, 3 * C))
            return r

        fwd_l, bwd_l = (fwd_fused, bwd_fused) if args.layout == "fused" else (fwd_copies,
                                                                             bwd_copies)

    def step_layout(record: int | None):
        if record is not None:
            timer.record(seq[record][0], sp)
        for l in range(L):
            if fwd_l(layers[l]) != 0:
                raise RuntimeError("forward failed")
        if record is not None:
            timer.record(seq[record][1], sp)
        for l in reversed(range(L)):
            if bwd_l(layers[l]) != 0:
                raise RuntimeError("backward failed")
        if record is not None:
            timer.record(seq[record][2], sp)

    def step(record: int | None):
        if args.layout != "contiguous":
            return step_layout(record)
        # record = index of a timed step: its events bracket the kernels of layer record % L
        lt = None if record is None else record % L
        if record is not None:
            timer.record(seq[record][0], sp)
        for l in range(L):
            run(l, "fwd_dropout" if drop else "fwd", record if l == lt else None)
        if record is not None:
            timer.record(seq[record][1], sp)
        for l in reversed(range(L)):
            i = record if l == lt else None
            if drop:
                run(l, "bwd_dropout", i)
                continue
            run(l, "dq", i)
            run(l, "dkdv", i)
        if record is not None:
            timer.record(seq[record][2], sp)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    ff, fb = flops(B, H, T, hs)
    step_flops = L * (ff + fb)
    ms_per_step = dt / args.steps * 1e3
    value = step_flops * args.steps / dt / 1e12
    _, fb_fa = flops(B, H, T, hs, bwd_per_pair=10)
    value_fa = L * (ff + fb_fa) * args.steps / dt / 1e12
    fwd_ms = [timer.elapsed_ms(a, b) for a, b, _ in seq]
    bwd_ms = [timer.elapsed_ms(b, c) for _, b, c in seq]
    pairs = B * H * T * (T + 1) // 2
    if args.layout != "contiguous":
        out = {"metric": metric, "value": round(value, 3), "unit": "TFLOP/s",
               "pct_of_bf16_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 3), "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
               "data": "synthetic",
               "config": {"workload": W["label"], "layout": args.layout, "B": B, "H": H, "T": T,
                          "hs": hs, "layers": L, "qkv_scale": W["qkv_scale"],
                          "parallelism": "single GPU"},
               "fwd_ms": {"median": round(float(np.median(fwd_ms)), 4),
                          "min": round(min(fwd_ms), 4)},
               "bwd_ms": {"median": round(float(np.median(bwd_ms)), 4),
                          "min": round(min(bwd_ms), 4)},
               "roofline": None}
        print(json.dumps(out), flush=True)
        return 0
    mean_us = {k: float(np.mean([timer.elapsed_ms(a, b) for a, b in ev[k]])) * 1e3
               for k in KT}
    dom = max(mean_us, key=mean_us.get)
    sym = KT[dom][0].format(hs=hs, E="Bf16" if args.dtype == "bf16" else "F16")
    if W["bound"] == "mfma":
        alg = KT[dom][2] * hs * pairs
        achieved = alg / (mean_us[dom] * 1e-6) / 1e12
        roof = {"kernel": sym, "bound": "mfma", "achieved": round(achieved, 3),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": read_traffic(dom, tag), "algorithmic_flop_per_launch": alg}
    else:
        alg = KT[dom][3] * B * H * T * hs * 2 + KT[dom][4] * B * H * T * 4
        achieved = alg / (mean_us[dom] * 1e-6) / 1e9
        roof = {"kernel": sym, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(dom, tag), "algorithmic_bytes_per_launch": alg}

    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": W["label"] + (f", attention dropout p={args.dropout}" if drop else ""),
                   "B": B, "H": H, "T": T, "hs": hs, "layers": L, "qkv_scale": W["qkv_scale"],
                   "dropout": args.dropout,
                   **({"dropout_mask": "drawn by the forward, stored as 1 bit per query-key "
                                       "pair, read by the backward"} if drop else {}),
                   "flop_count": "causal pairs, fwd 4*hs, bwd 8*hs per pair",
                   "parallelism": "single GPU"},
        "value_flashattention_count": round(value_fa, 3),
        "fwd_ms": {"median": round(float(np.median(fwd_ms)), 4), "min": round(min(fwd_ms), 4)},
        "bwd_ms": {"median": round(float(np.median(bwd_ms)), 4), "min": round(min(bwd_ms), 4)},
        "kernels_us": {k: round(v, 2) for k, v in mean_us.items()},
        "roofline": roof,
    }
    if args.peaks:
        out["measured_peaks"] = measured_peaks(torch, dev)
    if args.cpu_slices > 0:
        print(f"[bench] timing the CPU oracle on {args.cpu_slices} slices", file=sys.stderr,
              flush=True)
        out["cpu_baseline"] = cpu_baseline(host, scale, args.cpu_slices, args.dropout)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
