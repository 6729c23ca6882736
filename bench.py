"""Benchmark: KDA/CKDA chunk-forward tokens/s and roofline fraction on one MI355X.

Headline workload: KDA bf16 prefill, B=1 H=32 T=8192 d_k=d_v=128, chunk 64
(seeded synthetic inputs resident in HBM before timing).  One step = one
kda_chunk_forward call over the whole batch (gate summary, intra-chunk WY,
state propagation and outputs).  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-others] [--no-cpu]
                  [--backward] [--decode] [--gate-prep] [--copy-probe]

The roofline object describes the kernel with the largest average duration,
timed live with HIP events recorded by the library on the launch stream
(KDA_FLAG_STAGE_EVENTS).  Its algorithmic bytes are the bytes that kernel must
move for the method (its share of: read q, k, v, alpha, beta, S0; write o,
S_T) — intermediates excluded.  The cpu_baseline leg times the CPU oracle
(test infrastructure) on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
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
    # prep_fast reads the inputs, chain writes the outputs and reads/writes the
    # carried state; prep_exact only re-does chunks that prep_fast flagged
    return {"prep_fast": read_in, "prep_exact": 0, "chain": s0 + out + st,
            "path": read_in + s0 + out + st}


KERNEL_SOURCES = {
    # files whose contents determine each kernel's code
    "prep_fast": ["prep_fast.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
    "chain": ["chain.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
    "prep_exact": ["prep_exact.hip", "kda_chunk.hpp", "kda_device.hpp", "kda_launch.hpp"],
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


def time_forward(kda, torch, w, inp, steps, warmup, extra_flags=0):
    stream = torch.cuda.current_stream()
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.dtype, device="cuda")
    st = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")

    def call(flags=0):
        kda.chunk_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["S0"],
                          chunk=w.chunk, mode=w.mode, out=out, final_state=st, workspace=ws,
                          stream=stream, flags=flags | extra_flags)

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
    return ms, per, out, st


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
    nbytes = (w.B * w.T * w.H * w.Dk * 4 + w.B * w.H * nc * w.chunk * w.Dk * (4 + 1)
              + w.B * w.H * nc * w.Dk * 4)
    return {"workload": w.name, "us": us, "algorithmic_bytes": nbytes,
            "achieved_GBps": nbytes / (us / 1e6) / 1e9,
            "hbm_frac": nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
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
    ms, per, out, st = time_forward(kda, torch, w, inp, args.steps, args.warmup)
    tokens = w.B * w.T
    io_bytes = 2
    ab = algorithmic_bytes(w, io_bytes, inp["S0"] is not None, True)
    dom = max((k for k in per if ab.get(k)), key=per.get)
    dom_ms = per[dom]
    achieved = ab[dom] / (dom_ms / 1e3) / 1e9
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(dom), "kernel": dom,
                     "kernel_ms": dom_ms, "algorithmic_bytes": ab[dom]},
        "path_roofline": {"bound": "hbm", "algorithmic_bytes": ab["path"],
                          "achieved": ab["path"] / (ms / 1e3) / 1e9,
                          "frac": ab["path"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "mfma_bf16_frac": chunk_flops(w) / (ms / 1e3) / 1e12 / MFMA_BF16_TFLOPS},
        "kernels_ms": per,
    }
    if not args.no_others:
        others = {}
        for wid in (3, 1, 0):
            wo = workloads.workload(wid)
            io = workloads.make_prefill(wo, device="cuda")
            mso, pero, _, _ = time_forward(kda, torch, wo, io, max(3, args.steps // 4), 2)
            abo = algorithmic_bytes(wo, 2 if wo.dtype == torch.bfloat16 else 4,
                                    io["S0"] is not None, True)
            others[wo.name] = {"ms": mso, "tokens_per_s": wo.B * wo.T / (mso / 1e3),
                               "path_hbm_frac": abo["path"] / (mso / 1e3) / 1e9 / HBM_PEAK_GBS,
                               "kernels_ms": pero}
            del io
        # few heads, long context: sequence segments against one chain per head
        wo = workloads.workload(3, H=2)
        io = workloads.make_prefill(wo, device="cuda")
        for tag, fl in (("segments", 0), ("no_segments", kda.NO_SEGMENTS)):
            mso, pero, _, _ = time_forward(kda, torch, wo, io, 20, 2, fl)
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
        line["parity_vs_oracle"] = {
            "out_normwise_max_err": float(np.abs(g - o_ref).max() / np.abs(o_ref).max()),
            "state_normwise_max_err": float(np.abs(st[:, heads].cpu().numpy() - s_ref).max()
                                            / np.abs(s_ref).max())}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
