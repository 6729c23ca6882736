"""Benchmark: KDA/CKDA chunk-forward tokens/s and roofline fraction on one MI355X.

Headline workload: KDA bf16 prefill, B=1 H=32 T=8192 d_k=d_v=128, chunk 64
(seeded synthetic inputs resident in HBM before timing).  One step = one
kda_chunk_forward call over the whole batch (the two-pass form: gate summary
and intra-chunk WY for every chunk, then state propagation and outputs).  The
streamed form (kda_chunk_forward_side with KDA_FLAG_STREAMED, the two running
at once on two streams) takes the same time at this shape and is reported
beside it (--streamed makes it the headline).  Every call is launched on a
non-default stream of ours.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-others] [--no-cpu]
                  [--backward] [--decode] [--gate-prep] [--copy-probe] [--mfma-probe]
                  [--streamed] [--settle SECONDS]

Timing: untimed calls for --settle seconds (default 0.25: a fresh process
sees the device below its sustained clocks for about its first 100 calls),
then W untimed calls, then K calls back to back, each bracketed by HIP
events on the launch stream; ms_per_step is the median call.  The roofline
object describes the whole call: its algorithmic bytes (read q, k, v, alpha,
beta, S0 once; write o and S_T once; intermediates excluded) over the median
call time, against MI355X's 8 TB/s.  "kernels" breaks the call down per
kernel (durations from events the library attaches to each launch with
KDA_FLAG_STAGE_EVENTS), with each kernel's share of the algorithmic bytes and
the HBM bytes rocprofv3 counted for it (profiles/hbm_traffic_kda_bf16_prefill.md,
used only while the kernel's sources are unchanged).  The cpu_baseline leg
times the CPU oracle (test infrastructure) on the host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_TFLOPS = 2500.0      # dense bf16, published


def algorithmic_bytes(w, io_bytes, with_s0: bool, with_st: bool):
    """Bytes the method must move for a chunked forward, split by kernel."""
    BTH = w.B * w.T * w.H
    read_in = BTH * (2 * w.Dk * io_bytes + w.Dv * io_bytes + 4 * w.Dk + 4)
    s0 = 4 * w.B * w.H * w.Dk * w.Dv if with_s0 else 0
    out = BTH * w.Dv * io_bytes
    st = 4 * w.B * w.H * w.Dk * w.Dv if with_st else 0
    # prep_fast (prep_stream in the streamed call) reads the inputs, chain
    # (chain_stream) writes the outputs and reads/writes the carried state;
    # prep_exact only re-does chunks the fast prep flagged, and the streamed
    # call's fallback chain only runs when the streamed chain gave up
    return {"prep_fast": read_in, "prep_stream": read_in, "prep_exact": 0,
            "chain": s0 + out + st, "chain_stream": s0 + out + st,
            "path": read_in + s0 + out + st}


KERNEL_SOURCES = {
    # files whose contents determine each kernel's code
    "prep_fast": ["prep_fast.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
    "chain": ["chain.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_dma.hpp", "kda_launch.hpp"],
    "prep_exact": ["prep_exact.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
    "prep_stream": ["prep_fast.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
    "chain_stream": ["chain_wide.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_kda_bf16_prefill.md")


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "gated_delta_rule_forward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) recorded in
    the rocprofv3 counter summary, or None when the summary is missing or the
    kernel's sources changed since the counters were taken."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^\| %s \| ([0-9a-f]{16}) \| ([0-9.]+) \| ([0-9.]+) \|" % re.escape(kernel), text, re.M)
    if not m or m.group(1) != kernel_source_hash(kernel):
        return None
    return float(m.group(2)) + float(m.group(3))


def chunk_flops(w):
    """Dense per-chunk contractions of the chunkwise form (per token-head:
    2*(3 Dk Dv + C (Dk + Dk + Dv) ...) ), counted as in the design notes."""
    C, Dk, Dv = w.chunk, w.Dk, w.Dv
    per_tok = 2 * (Dk * Dv * 3 + C * (2 * Dk + Dv) + C * C // 3)
    return w.B * w.T * w.H * per_tok


def settle(torch, call, seconds):
    """Run `call` back to back for about `seconds` of wall time before the
    warm-up calls: a freshly started process sees the device below its
    sustained clocks for its first ~100 headline calls (per-call medians
    310-348 us over calls 0-20, 297 over calls 50-100, 289 from call 100 on).
    Untimed; returns the number of calls made."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            call()
        n += 10
        torch.cuda.synchronize()
    return n


def time_forward(kda, torch, w, inp, steps, warmup, extra_flags=0, side=None, settle_s=0.0, info=None):
    # (on the current stream: main() makes it a non-default one)
    """Median and mean ms per kda_chunk_forward call (each call bracketed by
    events on the launch stream) and the mean duration of every kernel (a
    separate pass with the library's per-launch events).  With settle_s > 0
    the device is first brought to its sustained clocks (settle()); the
    number of those untimed calls goes to info["settle_calls"]."""
    stream = torch.cuda.current_stream()
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.dtype, device="cuda")
    st = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")

    def call(flags=0):
        kda.chunk_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                          chunk=w.chunk, mode=w.mode, out=out, final_state=st, workspace=ws,
                          stream=stream, flags=flags | extra_flags, side=side)

    if settle_s > 0:
        n = settle(torch, call, settle_s)
        if info is not None:
            info["settle_calls"] = n
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    calls = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    med, mean = statistics.median(calls), ev[0].elapsed_time(ev[steps]) / steps
    # per-kernel durations (separate pass; events recorded by the library)
    per = {}
    for _ in range(steps):
        call(kda.STAGE_EVENTS)
        tot = {}
        for name, t in kda.last_stage_times():      # a kernel may run once per part
            tot[name] = tot.get(name, 0.0) + t
        for name, t in tot.items():
            per.setdefault(name, []).append(t)
    torch.cuda.synchronize()
    per = {k: sum(v) / len(v) for k, v in per.items()}
    return med, mean, per, out, st


def time_train_step(kda, torch, w, inp, steps, warmup):
    """One training step split as kda_chunk_forward_save + kda_chunk_backward_saved
    on workload w: ms per step (the pair), and per call ms of each half."""
    import workloads
    stream = torch.cuda.current_stream()
    dO, dST = workloads.make_backward_seeds(w, device="cuda")
    saved = torch.empty(kda.backward_workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                        dtype=torch.uint8, device="cuda")
    out = torch.empty_like(inp["v"])
    st = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")
    grads = {"dq": torch.empty_like(inp["q"]), "dk": torch.empty_like(inp["k"]),
             "dv": torch.empty_like(inp["v"]), "d_alpha": torch.empty_like(inp["alpha"]),
             "d_beta": torch.empty_like(inp["beta"]),
             "d_initial_state": torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32,
                                            device="cuda")}

    def fwd():
        kda.chunk_forward_save(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                               chunk=w.chunk, mode=w.mode, out=out, final_state=st, saved=saved,
                               stream=stream)

    def bwd():
        kda.chunk_backward_saved(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO, saved,
                                 dST, chunk=w.chunk, mode=w.mode, grads=grads, stream=stream)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    for i in range(steps):
        ev[3 * i].record(stream)
        fwd()
        ev[3 * i + 1].record(stream)
        bwd()
        ev[3 * i + 2].record(stream)
    torch.cuda.synchronize()
    f = [ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps)]
    b = [ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps)]
    return (statistics.median([x + y for x, y in zip(f, b)]), statistics.median(f),
            statistics.median(b))


def time_backward(kda, torch, w, inp, steps, warmup):
    """kda_chunk_backward on workload w (loss gradients from workloads.make_backward_seeds):
    ms per call and per-kernel durations, plus the algorithmic bytes of the call
    (the inputs q, k, v, alpha, beta, dO, S0, dST read once; dq, dk, dv, dalpha,
    dbeta, dS0 written once)."""
    import workloads
    stream = torch.cuda.current_stream()
    dO, dST = workloads.make_backward_seeds(w, device="cuda")
    ws = torch.empty(kda.backward_workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    grads = {"dq": torch.empty_like(inp["q"]), "dk": torch.empty_like(inp["k"]),
             "dv": torch.empty_like(inp["v"]), "d_alpha": torch.empty_like(inp["alpha"]),
             "d_beta": torch.empty_like(inp["beta"]),
             "d_initial_state": torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32,
                                            device="cuda")}

    def call(flags=0):
        kda.chunk_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO, inp["S0"],
                           dST, chunk=w.chunk, mode=w.mode, grads=grads, workspace=ws,
                           stream=stream, flags=flags)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per = {}
    for _ in range(steps):
        call(kda.STAGE_EVENTS)
        for name, t in kda.last_stage_times():
            per.setdefault(name, []).append(t)
    torch.cuda.synchronize()
    per = {k: sum(v) / len(v) for k, v in per.items()}
    e = 2 if w.dtype == torch.bfloat16 else 4
    ntok = w.B * w.T * w.H
    state = w.B * w.H * w.Dk * w.Dv * 4
    nbytes = (ntok * (2 * (2 * w.Dk + 2 * w.Dv) * e + 2 * (4 * w.Dk + 4))
              + state * (3 if inp["S0"] is not None else 2))
    return ms, per, nbytes


def cpu_baseline(oracle, w, inp, max_heads=None, min_seconds=10.0):
    import numpy as np
    heads = list(range(w.H if max_heads is None else min(w.H, max_heads)))
    f = lambda t: t[:, :, heads].float().cpu().numpy()
    args = [f(inp[x]) for x in ("q", "k", "v", "alpha")]
    beta = inp["beta"][:, :, heads].float().cpu().numpy()
    s0 = None if inp["S0"] is None else inp["S0"][:, heads].float().cpu().numpy()
    nthreads = oracle.default_threads()
    nthreads = min(nthreads, 16)
    # repeat the same forward until about min_seconds of wall time have passed
    reps, dt = 0, 0.0
    while True:
        t0 = time.perf_counter()
        o, s = oracle.forward(*args, beta, s0, nthreads=nthreads)
        dt += time.perf_counter() - t0
        reps += 1
        if dt >= min_seconds or reps >= 200:
            break
    toks = reps * w.B * w.T * len(heads) / w.H        # tokens of the full batch equivalent
    return {"value": toks / dt, "unit": "tokens/s", "cores": min(nthreads, len(heads) * w.B),
            "kind": "oracle",
            "sample": f"{w.name}: B={w.B} T={w.T} heads {len(heads)}/{w.H}, fp64 sequential "
                      f"recurrence, {reps} passes in {dt:.1f} s wall; tokens/s scaled to all "
                      f"{w.H} heads"}, (o, s, heads)


def decode_bench(kda, torch, workloads, steps_cap=None):
    w = workloads.workload(4)
    n = w.steps if steps_cap is None else min(steps_cap, w.steps)
    inp = workloads.make_decode(w, steps=n, device="cuda")
    S = inp["S0"].clone()
    outs = torch.empty((n, w.B, w.H, w.D), dtype=w.dtype, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        for s in range(n):
            kda.decode_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["alpha"][s],
                            inp["beta"][s], S, out=outs[s], stream=stream)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_step = ms / n
    bytes_step = (2 * w.B * w.H * w.D * w.D * 4 + w.B * w.H * (4 * w.D * 2 + 4 * w.D + 4))
    return {"workload": w.name, "steps": n, "ms_total": ms, "us_per_step": 1e3 * per_step,
            "tokens_per_s": w.B * n / (ms / 1e3),
            "hbm_frac": bytes_step / (per_step / 1e3) / 1e9 / HBM_PEAK_GBS}


def gate_prep_bench(kda, torch, w, inp, steps):
    """kda_gate_prep (the standalone gate summary, row a1) on workload w: us per
    call and the HBM fraction of its algorithmic bytes (alpha read once; L,
    the meta byte and Gamma_C written once)."""
    alpha = inp["alpha"]
    stream = torch.cuda.current_stream()
    for _ in range(3):
        kda.gate_prep(alpha, w.chunk, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        kda.gate_prep(alpha, w.chunk, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / steps
    nc = (w.T + w.chunk - 1) // w.chunk
    # moved: alpha read once, the summary written once (L fp32 and the meta
    # byte per element, Gamma_C per chunk and channel); algorithmic: the
    # alpha read alone (the summary is an intermediate of the forward, which
    # recomputes it inside its prep kernel instead)
    read = w.B * w.T * w.H * w.Dk * 4
    moved = read + w.B * w.H * nc * w.chunk * w.Dk * (4 + 1) + w.B * w.H * nc * w.Dk * 4
    return {"workload": w.name, "us": us, "moved_bytes": moved, "algorithmic_bytes": read,
            "moved_GBps": moved / (us / 1e6) / 1e9,
            "moved_hbm_frac": moved / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_GBps": read / (us / 1e6) / 1e9,
            "algorithmic_hbm_frac": read / (us / 1e6) / 1e9 / HBM_PEAK_GBS}


def mfma_probe(kda):
    """Achieved dense MFMA rates of the probe library (libkda_probe.so): bf16
    16x16x32 and fp32 16x16x4, 8 independent chains per wavefront, 8 and 16
    wavefronts per compute unit."""
    import torch
    lib = ctypes.CDLL(os.path.join(os.path.dirname(kda.library_path()), "libkda_probe.so"))
    lib.kda_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double)]
    lib.kda_probe_mfma.restype = ctypes.c_int
    sink = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
    res = {}
    for kind, name, iters in ((0, "bf16_16x16x32", 20000), (1, "fp32_16x16x4", 5000)):
        for wpc in (8, 16):
            t = ctypes.c_double(0.0)
            rc = lib.kda_probe_mfma(kind, iters, wpc, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(t))
            if rc != 0:
                raise RuntimeError(f"kda_probe_mfma failed: {rc}")
            res[f"{name}_waves{wpc}_TFLOPs"] = t.value
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward on the headline workload even with --no-others")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode workload even with --no-others")
    ap.add_argument("--gate-prep", action="store_true",
                    help="time the standalone gate summary even with --no-others")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="also measure the dense MFMA peak rates (bf16 and fp32)")
    ap.add_argument("--settle", type=float, default=0.25,
                    help="seconds of untimed headline calls before the warm-up calls, so the "
                         "device runs at its sustained clocks (0: none)")
    ap.add_argument("--streamed", action="store_true",
                    help="time the streamed kda_chunk_forward_side call as the headline (not "
                         "under rocprofv3 counter passes, which run one dispatch at a time: the "
                         "streamed call's chain would wait out its bound for a prep grid that "
                         "cannot start)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_forward_amd as kda
    import workloads

    torch.cuda.init()
    w = workloads.workload(2)
    inp = workloads.make_prefill(w, device="cuda")
    torch.cuda.synchronize()
    # every call on a stream of ours (the null stream would wait for the side
    # stream's work: the overlapped forms need a non-default launch stream)
    torch.cuda.set_stream(torch.cuda.Stream())
    side = kda.SideStream()
    tinfo = {}
    if args.streamed:
        ms, mean_ms, per, out, st = time_forward(kda, torch, w, inp, args.steps, args.warmup,
                                                 extra_flags=kda.STREAMED, side=side,
                                                 settle_s=args.settle, info=tinfo)
    else:
        ms, mean_ms, per, out, st = time_forward(kda, torch, w, inp, args.steps, args.warmup,
                                                 settle_s=args.settle, info=tinfo)
    tokens = w.B * w.T
    io_bytes = 2
    ab = algorithmic_bytes(w, io_bytes, inp["S0"] is not None, True)
    kernels = {}
    traffic_total = 0.0
    for name, kms in per.items():
        kb = ab.get(name, 0)
        tr = measured_traffic(name) if name in KERNEL_SOURCES else None
        traffic_total = None if (tr is None or traffic_total is None) else traffic_total + tr
        kernels[name] = {"ms": kms, "algorithmic_bytes": kb,
                         "achieved_GBps": kb / (kms / 1e3) / 1e9 if kb else 0.0,
                         "hbm_frac": kb / (kms / 1e3) / 1e9 / HBM_PEAK_GBS if kb else 0.0,
                         "traffic_bytes": tr,
                         "traffic_ratio": (tr / kb) if (tr is not None and kb) else None}
    achieved = ab["path"] / (ms / 1e3) / 1e9
    line = {
        "metric": "KDA/CKDA chunk-forward tokens/s (H=32,d=128,T=8192) + % MFMA/HBM roofline",
        "value": tokens / (ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_bf16_prefill B=1 H=32 T=8192 d_k=d_v=128 chunk=64",
                   "B": w.B, "H": w.H, "T": w.T, "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk,
                   "mode": "KDA", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_total,
                     "scope": "whole call", "algorithmic_bytes": ab["path"],
                     "traffic_ratio": (traffic_total / ab["path"]) if traffic_total else None,
                     "mfma_bf16_frac": chunk_flops(w) / (ms / 1e3) / 1e12 / MFMA_BF16_TFLOPS},
        "timing": {"median_ms": ms, "mean_ms": mean_ms, "calls": args.steps,
                   "settle_s": args.settle, "settle_calls": tinfo.get("settle_calls", 0),
                   "call": "kda_chunk_forward_side, KDA_FLAG_STREAMED" if args.streamed
                           else "kda_chunk_forward (two-pass)"},
        "kernels": kernels,
        "kernels_ms": per,
    }
    if not args.no_others:
        others = {}
        # the same workload in the other form (streamed: the prep on a second
        # stream while the chain consumes each chunk; or two-pass)
        ms1, _, per1, _, _ = time_forward(kda, torch, w, inp, max(20, args.steps // 4), 3,
                                          extra_flags=0 if args.streamed else kda.STREAMED,
                                          side=None if args.streamed else side)
        tr1 = [measured_traffic(n) for n in per1 if n in KERNEL_SOURCES]
        tr1 = None if (not tr1 or None in tr1) else sum(tr1)
        others["kda_bf16_prefill_two_pass" if args.streamed else "kda_bf16_prefill_streamed"] = {
            "ms": ms1, "tokens_per_s": tokens / (ms1 / 1e3),
            "path_hbm_frac": ab["path"] / (ms1 / 1e3) / 1e9 / HBM_PEAK_GBS,
            "traffic_bytes": tr1, "traffic_ratio": tr1 / ab["path"] if tr1 else None,
            "kernels_ms": per1}
        for wid in (3, 1, 0):
            wo = workloads.workload(wid)
            io = workloads.make_prefill(wo, device="cuda")
            # the long-context workload is streamed on a second stream of ours
            mso, _, pero, _, _ = time_forward(kda, torch, wo, io, max(20, args.steps // 4), 3,
                                              extra_flags=kda.STREAMED if wid == 3 else 0,
                                              side=side if wid == 3 else None)
            abo = algorithmic_bytes(wo, 2 if wo.dtype == torch.bfloat16 else 4,
                                    io["S0"] is not None, True)
            others[wo.name] = {"ms": mso, "tokens_per_s": wo.B * wo.T / (mso / 1e3),
                               "path_hbm_frac": abo["path"] / (mso / 1e3) / 1e9 / HBM_PEAK_GBS,
                               "kernels_ms": pero}
            del io
        # the long-context workload in parts (the prep of part p + 1 beside the
        # chain of part p) instead of streamed
        wo = workloads.workload(3)
        io = workloads.make_prefill(wo, device="cuda")
        mso, _, pero, _, _ = time_forward(kda, torch, wo, io, max(20, args.steps // 4), 3, side=side)
        others["ckda_bf16_long_ctx_parts"] = {"ms": mso, "tokens_per_s": wo.B * wo.T / (mso / 1e3),
                                              "kernels_ms": pero}
        del io
        # few heads, long context: sequence segments against one chain per head
        wo = workloads.workload(3, H=2)
        io = workloads.make_prefill(wo, device="cuda")
        for tag, fl in (("segments", 0), ("no_segments", kda.NO_SEGMENTS)):
            mso, _, pero, _, _ = time_forward(kda, torch, wo, io, 20, 3, fl)
            others[f"ckda_bf16_long_ctx_H2_{tag}"] = {"ms": mso, "tokens_per_s": wo.B * wo.T / (mso / 1e3),
                                                     "kernels_ms": pero}
        del io
        line["others"] = others
    if not args.no_others or args.decode:
        line.setdefault("others", {})["ckda_bf16_decode"] = decode_bench(kda, torch, workloads)
    if not args.no_others or args.gate_prep:
        line.setdefault("others", {})["kda_gate_prep"] = gate_prep_bench(kda, torch, w, inp,
                                                                         max(10, args.steps // 4))
    if not args.no_others or args.backward:
        # the backward (kda_chunk_backward) on the headline workload
        msb, perb, nbb = time_backward(kda, torch, w, inp, max(3, args.steps // 4), 3)
        line.setdefault("others", {})["kda_bf16_prefill_backward"] = {
            "ms": msb, "tokens_per_s": tokens / (msb / 1e3), "algorithmic_bytes": nbb,
            "path_hbm_frac": nbb / (msb / 1e3) / 1e9 / HBM_PEAK_GBS, "kernels_ms": perb}
        # a training step without recomputation: the saving forward, then the
        # gradients from its workspace
        mst, msf, msbs = time_train_step(kda, torch, w, inp, max(3, args.steps // 4), 3)
        line["others"]["kda_bf16_prefill_train_step_saved"] = {
            "ms": mst, "forward_save_ms": msf, "backward_saved_ms": msbs,
            "tokens_per_s": tokens / (mst / 1e3)}
    if args.mfma_probe:
        line["mfma_probe"] = mfma_probe(kda)
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = 1 << 30
    if not args.no_cpu:
        import oracle
        import numpy as np
        cb, (o_ref, s_ref, heads) = cpu_baseline(oracle, w, inp)
        line["cpu_baseline"] = cb
        g = out[:, :, heads].float().cpu().numpy()
        gs = st[:, heads].cpu().numpy()

        def errs(x, r):
            # normwise max error, and the elementwise relative error with a
            # floor of 1e-3 max|r| (information only)
            ar = np.abs(r)
            den = ar.max()
            d = np.abs(x - r)
            return float(d.max() / den), float((d / np.maximum(ar, 1e-3 * den)).max())

        eo, eoe = errs(g, o_ref)
        es, ese = errs(gs, s_ref)
        line["parity_vs_oracle"] = {"out_normwise_max_err": eo, "state_normwise_max_err": es,
                                    "out_elementwise_max_rel_err": eoe,
                                    "state_elementwise_max_rel_err": ese}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
