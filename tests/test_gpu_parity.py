"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case prints its name before touching the GPU.  Inputs come from
workloads.py (seeded, synthetic); expected values come only from oracle/.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import oracle
import workloads
from parity import TOL, np32, oracle_threads, say, slice_err_out, slice_err_state, elem_note

pytestmark = pytest.mark.gpu

DEV = "cuda"


def to_dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def run_oracle(inp, heads=None):
    """Oracle forward on (a subset of) heads; inputs may live on the GPU."""
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    q, k, v, a = (np32(sel(inp[x])) for x in ("q", "k", "v", "alpha"))
    b = np32(sel(inp["beta"]))
    s0 = None
    if inp.get("S0") is not None:
        s0 = np32(inp["S0"] if heads is None else inp["S0"][:, heads])
    return oracle.forward(q, k, v, a, b, s0, nthreads=oracle_threads())


def run_gpu(inp, chunk, mode, **kw):
    if kw.get("stream") is not None:
        torch.cuda.synchronize()         # (inputs were made on the current stream)
    out, st = kda.chunk_forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                inp.get("S0"), chunk=chunk, mode=mode, **kw)
    torch.cuda.synchronize()
    return out, st


# (name, base workload, overrides)
SMALL = [
    ("kda_fp32_tiny_T64", 0, {}),
    ("ckda_fp32_B2_H4_T1024", 1, {}),
    ("f32_ckda_dk32_dv48_c32_T67_s0", 1, dict(B=1, H=3, T=67, D=32, chunk=32, s0_std=0.5)),
    ("f32_kda_d64_c64_T5", 0, dict(B=2, H=2, T=5, D=64, chunk=64)),
    ("f32_ckda_d16_c16_T1", 1, dict(B=1, H=1, T=1, D=16, chunk=16)),
    ("bf16_ckda_d128_c64_T67_s0", 3, dict(B=1, H=2, T=67, chunk=64)),
    ("bf16_kda_d64_c16_T200", 2, dict(B=2, H=3, T=200, D=64, chunk=16)),
    ("bf16_ckda_d32_c32_T96", 3, dict(B=1, H=2, T=96, D=32, chunk=32, s0_std=None)),
    ("bf16_kda_d128_c32_T1", 2, dict(B=1, H=1, T=1, chunk=32)),
    ("bf16_ckda_d16_c16_T333", 3, dict(B=3, H=1, T=333, D=16, chunk=16)),
    ("bf16_ckda_d128_c64_T1000", 3, dict(B=1, H=4, T=1000, chunk=64)),
]


@pytest.mark.parametrize("name,base,ov", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small(name, base, ov):
    w = workloads.workload(base, **ov)
    say(f"[forward] {name}: {w}")
    inp = workloads.make_prefill(w, device="cpu")
    o_ref, s_ref = run_oracle(inp)
    out, st = run_gpu(to_dev(inp), w.chunk, w.mode)
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_forward_dk_ne_dv_and_zero_state_pointer():
    """Dk != Dv (rows/columns of S must not be swapped) and an explicit zero
    initial state gives the same result as a NULL one."""
    w = workloads.workload(1, B=1, H=2, T=130, D=64, chunk=32)
    inp = workloads.make_prefill(w)
    inp["v"] = inp["v"][..., :32].contiguous()
    say("[forward] f32 Dk=64 Dv=32")
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    out, st = run_gpu(d, 32, workloads.CKDA)
    assert slice_err_out(np32(out), o_ref) <= 1e-4
    assert slice_err_state(np32(st), s_ref) <= 1e-4
    d["S0"] = torch.zeros(1, 2, 64, 32, device=DEV)
    out2, st2 = run_gpu(d, 32, workloads.CKDA)
    assert torch.equal(out, out2) and torch.equal(st, st2)


STATES = [
    ("f32_ckda_dk32_dv48_c32_T67_s0", 1, dict(B=1, H=3, T=67, D=32, chunk=32, s0_std=0.5)),
    ("bf16_kda_d64_c16_T200", 2, dict(B=2, H=3, T=200, D=64, chunk=16)),
    ("bf16_ckda_d128_c64_T1000_s0", 3, dict(B=1, H=4, T=1000, chunk=64)),
]


@pytest.mark.parametrize("name,base,ov", STATES, ids=[c[0] for c in STATES])
def test_forward_chunk_states(name, base, ov):
    """kda_chunk_forward_states: the state entering every chunk, in the io
    dtype, against the oracle's state before token n*chunk; outputs and final
    state identical to kda_chunk_forward's."""
    w = workloads.workload(base, **ov)
    say(f"[forward states] {name}: {w}")
    inp = workloads.make_prefill(w, device="cpu")
    q, k, v, a = (np32(inp[x]) for x in ("q", "k", "v", "alpha"))
    s0 = None if inp.get("S0") is None else np32(inp["S0"])
    o_ref, s_ref, cs_ref = oracle.forward(q, k, v, a, np32(inp["beta"]), s0,
                                          nthreads=oracle_threads(), chunk=w.chunk)
    d = to_dev(inp)
    nc = (w.T + w.chunk - 1) // w.chunk
    cs = torch.full((w.B, w.H, nc, w.D, w.D), float("nan"), dtype=w.dtype, device=DEV)
    out, st = run_gpu(d, w.chunk, w.mode, chunk_states=cs)
    out_plain, st_plain = run_gpu(d, w.chunk, w.mode)
    ec = slice_err_state(np32(cs).reshape(w.B, w.H * nc, w.D, w.D),
                         cs_ref.reshape(w.B, w.H * nc, w.D, w.D))
    say(f"  err chunk states {ec:.3e}")
    assert ec <= TOL[w.dtype]
    assert torch.equal(out, out_plain) and torch.equal(st, st_plain)


# (name, base workload, overrides, (alpha_min, alpha_max, beta_max, eps, normalize_q), forget)
PROLOGUE = [
    ("f32_kda_d32_c32_T67", 0, dict(B=1, H=3, T=67, D=32, chunk=32), (0.0, 1.0, 1.0, 1e-6, 1), 0.0),
    ("f32_ckda_d64_c64_T130_s0", 1, dict(B=2, H=1, T=130, D=64, chunk=64, s0_std=0.3),
     (-1.0, 1.0, 2.0, 1e-6, 1), 0.0),
    ("bf16_kda_d64_c16_T200_rawq", 2, dict(B=2, H=2, T=200, D=64, chunk=16),
     (0.2, 0.99, 1.0, 1e-5, 0), 0.0),
    ("bf16_ckda_d128_c64_T300_s0", 3, dict(B=1, H=2, T=300, chunk=64), (-1.0, 1.0, 2.0, 1e-6, 1), 0.0),
    # KDA gates of exactly 0 (logit -200): their chunks go through the exact kernel
    ("bf16_kda_d128_c64_T256_zero_gates", 2, dict(B=1, H=2, T=256, chunk=64),
     (0.0, 1.0, 1.0, 1e-6, 1), 0.002),
    # eps comparable to the raw norms (|k_raw| ~ sqrt(D): 11.3 at D = 128, 8 at
    # D = 64), so where eq. (18) puts eps changes the keys by tens of percent
    ("bf16_ckda_d128_c64_T200_eps4", 3, dict(B=1, H=2, T=200, chunk=64), (-1.0, 1.0, 2.0, 4.0, 1), 0.0),
    ("f32_ckda_d64_c32_T99_eps3", 1, dict(B=1, H=2, T=99, D=64, chunk=32, s0_std=0.3),
     (-1.0, 1.0, 2.0, 3.0, 1), 0.0),
    ("f32_kda_d32_c16_T50_eps2_rawq", 0, dict(B=2, H=1, T=50, D=32, chunk=16), (0.0, 1.0, 1.0, 2.0, 0), 0.0),
]


@pytest.mark.parametrize("name,base,ov,pro,forget", PROLOGUE, ids=[c[0] for c in PROLOGUE])
def test_forward_prologue(name, base, ov, pro, forget):
    """kda_chunk_forward_prologue (gate range, beta and key / query
    normalisation fused into the kernels) against the oracle's forward from
    the same raw inputs."""
    w = workloads.workload(base, **ov)
    say(f"[forward prologue] {name}: {w} {pro}")
    inp = workloads.make_prefill_raw(w, device="cpu", forget_frac=forget)
    amin, amax, bmax, eps, nq = pro
    o_ref, s_ref = oracle.forward_prologue(
        np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(inp["gate"]),
        np32(inp["beta_logit"]), None if inp["S0"] is None else np32(inp["S0"]),
        alpha_min=amin, alpha_max=amax, beta_max=bmax, eps=eps, normalize_q=bool(nq),
        nthreads=oracle_threads())
    d = to_dev(inp)
    out, st = kda.chunk_forward_prologue(d["q"], d["k"], d["v"], d["gate"], d["beta_logit"],
                                         d["S0"], alpha_min=amin, alpha_max=amax, beta_max=bmax,
                                         eps=eps, normalize_q=bool(nq), chunk=w.chunk, mode=w.mode)
    torch.cuda.synchronize()
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


# (name, base workload, overrides, sequence lengths)
VARLEN = [
    ("bf16_kda_d64_c32_mixed", 2, dict(H=2, D=64, chunk=32, s0_std=0.3), [0, 1, 64, 130, 37, 200]),
    ("f32_ckda_d32_c16_mixed", 1, dict(H=3, D=32, chunk=16, s0_std=0.5), [5, 0, 48, 17]),
    ("bf16_ckda_d128_c64_long", 3, dict(H=2, chunk=64), [300, 64, 1, 129]),
]


@pytest.mark.parametrize("name,base,ov,lengths", VARLEN, ids=[c[0] for c in VARLEN])
def test_forward_varlen(name, base, ov, lengths):
    """kda_chunk_forward_varlen: every sequence of the packed batch against the
    oracle run on that sequence alone with its own initial state."""
    w = workloads.workload(base, **ov)
    say(f"[forward varlen] {name}: {w} lengths {lengths}")
    inp = workloads.make_varlen(w, lengths)
    d = to_dev(inp)
    out, st = kda.chunk_forward_varlen(d["q"][0], d["k"][0], d["v"][0], d["alpha"][0],
                                       d["beta"][0], d["cu_seqlens"], d["S0"], chunk=w.chunk,
                                       mode=w.mode)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    worst_o = worst_s = 0.0
    for i, L in enumerate(lengths):
        sl = slice(cu[i], cu[i + 1])
        sub = {x: inp[x][:, sl] for x in ("q", "k", "v", "alpha", "beta")}
        sub["S0"] = None if inp["S0"] is None else inp["S0"][i:i + 1]
        o_ref, s_ref = run_oracle(sub)
        if L > 0:
            worst_o = max(worst_o, slice_err_out(np32(out[sl])[None], o_ref))
        worst_s = max(worst_s, slice_err_state(np32(st[i:i + 1]), s_ref))
    say(f"  err out {worst_o:.3e} state {worst_s:.3e}")
    assert worst_o <= TOL[w.dtype] and worst_s <= TOL[w.dtype]


def test_forward_varlen_uniform_equals_dense():
    """Equal lengths: the packed batch numbers its chunks exactly like the
    dense batch, so outputs and states are bit-identical to kda_chunk_forward."""
    w = workloads.workload(2, B=3, H=2, T=100, chunk=64, s0_std=0.2)
    say(f"[forward varlen] uniform vs dense {w}")
    d = to_dev(workloads.make_prefill(w))
    out, st = run_gpu(d, w.chunk, w.mode)
    cu = torch.arange(0, 301, 100, dtype=torch.int32, device=DEV)
    flat = lambda t: t.reshape((1, -1) + tuple(t.shape[2:]))[0]
    out2, st2 = kda.chunk_forward_varlen(flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["alpha"]),
                                         flat(d["beta"]), cu, d["S0"], chunk=w.chunk, mode=w.mode)
    torch.cuda.synchronize()
    assert torch.equal(out2.reshape(out.shape), out) and torch.equal(st2, st)


def test_forward_varlen_prologue():
    """Packed batch with the fused parameterisation, per sequence against the
    oracle's forward from raw inputs."""
    w = workloads.workload(3, H=2, chunk=64, s0_std=None)
    lengths = [70, 33, 0, 128]
    say(f"[forward varlen prologue] {w} lengths {lengths}")
    total = sum(lengths)
    inp = workloads.make_prefill_raw(workloads.workload(3, B=1, H=2, T=total, chunk=64, s0_std=None))
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    pro = dict(alpha_min=-1.0, alpha_max=1.0, beta_max=2.0, eps=1e-6, normalize_q=True)
    d = to_dev(inp)
    out, st = kda.chunk_forward_varlen(d["q"][0], d["k"][0], d["v"][0], d["gate"][0],
                                       d["beta_logit"][0], torch.tensor(cu, dtype=torch.int32, device=DEV),
                                       None, chunk=64, mode=workloads.CKDA, prologue=pro)
    torch.cuda.synchronize()
    worst = 0.0
    for i, L in enumerate(lengths):
        sl = slice(cu[i], cu[i + 1])
        o_ref, s_ref = oracle.forward_prologue(
            np32(inp["q"][:, sl]), np32(inp["k"][:, sl]), np32(inp["v"][:, sl]),
            np32(inp["gate"][:, sl]), np32(inp["beta_logit"][:, sl]), None,
            nthreads=oracle_threads(), **pro)
        if L > 0:
            worst = max(worst, slice_err_out(np32(out[sl])[None], o_ref))
        worst = max(worst, slice_err_state(np32(st[i:i + 1]), s_ref))
    say(f"  err {worst:.3e}")
    assert worst <= 2e-2


# (name, base workload, overrides, theta_max)
PHASE = [
    ("f32_kda_d32_c32_T67", 0, dict(B=1, H=3, T=67, D=32, chunk=32), 3.0),
    ("f32_ckda_d64_c16_T130_s0", 1, dict(B=2, H=1, T=130, D=64, chunk=16, s0_std=0.3), 1.0),
    ("bf16_kda_d128_c64_T300_s0", 2, dict(B=1, H=2, T=300, chunk=64, s0_std=0.1), 3.0),
    ("bf16_ckda_d128_c64_T200", 3, dict(B=1, H=2, T=200, chunk=64), 0.5),
    ("bf16_kda_d64_c32_T96", 2, dict(B=2, H=2, T=96, D=64, chunk=32), 0.1),
]


@pytest.mark.parametrize("name,base,ov,tmax", PHASE, ids=[c[0] for c in PHASE])
def test_forward_phase(name, base, ov, tmax):
    """kda_chunk_forward_phase against the oracle's phase-variant recurrence
    (gates and phases per channel pair; CKDA cases include exact 0 and -1
    gates, so zero-segment columns and the exact kernel are exercised)."""
    w = workloads.workload(base, **ov)
    say(f"[forward phase] {name}: {w} theta_max {tmax}")
    inp = workloads.make_prefill_phase(w, theta_max=tmax)
    o_ref, s_ref = oracle.forward_phase(
        np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(inp["alpha"]), np32(inp["theta"]),
        np32(inp["beta"]), None if inp["S0"] is None else np32(inp["S0"]), nthreads=oracle_threads())
    d = to_dev(inp)
    out, st = kda.chunk_forward_phase(d["q"], d["k"], d["v"], d["alpha"], d["theta"], d["beta"],
                                      d["S0"], chunk=w.chunk, mode=w.mode)
    torch.cuda.synchronize()
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_forward_phase_zero_is_kda_bitwise():
    """theta = 0 makes every rotation the identity (sin 0 = 0, cos 0 = 1
    exactly), so the phase path gives bit for bit the plain path with each
    pair's gate on both of its channels."""
    w = workloads.workload(2, B=1, H=2, T=150, chunk=64, s0_std=0.2)
    say(f"[forward phase] theta = 0 vs plain {w}")
    d = to_dev(workloads.make_prefill_phase(w))
    zero = torch.zeros_like(d["theta"])
    out1, st1 = kda.chunk_forward_phase(d["q"], d["k"], d["v"], d["alpha"], zero, d["beta"],
                                        d["S0"], chunk=64, mode=w.mode)
    out2, st2 = run_gpu(dict(d, alpha=d["alpha"].repeat_interleave(2, dim=-1).contiguous()), 64, w.mode)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(st1, st2)


@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.float32, 32, 48), (torch.bfloat16, 128, 128),
                                         (torch.bfloat16, 16, 80), (torch.bfloat16, 64, 96),
                                         (torch.float32, 64, 64)])
def test_decode_phase(dtype, Dk, Dv):
    """kda_decode_step_phase: three steps against the oracle's phase-variant
    recurrence on the same tokens."""
    say(f"[decode phase] {dtype} Dk={Dk} Dv={Dv}")
    g = torch.Generator().manual_seed(Dk + Dv)
    B, H, N = 3, 2, 3
    q = torch.randn(N, B, H, Dk, generator=g).to(dtype)
    k = (torch.randn(N, B, H, Dk, generator=g) * 0.3).to(dtype)
    v = torch.randn(N, B, H, Dv, generator=g).to(dtype)
    a = torch.rand(N, B, H, Dk // 2, generator=g) * 0.5 + 0.5
    th = (torch.rand(N, B, H, Dk // 2, generator=g) - 0.5) * 6.0
    b = torch.rand(N, B, H, generator=g)
    S0 = torch.randn(B, H, Dk, Dv, generator=g) * 0.2
    S = S0.to(DEV).contiguous()
    outs = []
    for t in range(N):
        outs.append(kda.decode_step_phase(q[t].to(DEV).contiguous(), k[t].to(DEV).contiguous(),
                                          v[t].to(DEV).contiguous(), a[t].to(DEV).contiguous(),
                                          th[t].to(DEV).contiguous(), b[t].to(DEV).contiguous(), S,
                                          mode=workloads.CKDA))
    torch.cuda.synchronize()
    perm = lambda x: np32(x.permute(1, 0, *range(2, x.dim())))        # [N,B,...] -> [B,N,...]
    o_ref, s_ref = oracle.forward_phase(perm(q), perm(k), perm(v), perm(a), perm(th), perm(b),
                                        np32(S0))
    o_gpu = np.stack([np32(o) for o in outs], axis=1)
    eo, es = slice_err_out(o_gpu, o_ref), slice_err_state(np32(S), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


# (name, base workload, overrides, expected segments) — few chains and many
# chunks, so the forward cuts every (b, h) into segments
SEGMENTED = [
    ("f32_kda_d32_c16_T2500", 0, dict(B=1, H=1, T=2500, D=32, chunk=16), 4),
    ("bf16_ckda_d128_c64_T9000_s0", 3, dict(B=1, H=2, T=9000, chunk=64, s0_std=0.2), 4),
]


def _stage_names():
    names = [n for n, _ in kda.last_stage_times()]
    return names


@pytest.mark.parametrize("name,base,ov,nseg", SEGMENTED, ids=[c[0] for c in SEGMENTED])
def test_forward_segmented(name, base, ov, nseg):
    """Sequence segments (segment maps, fp32 chaining of the segment start
    states, then all segments side by side) against the oracle's sequential
    recurrence; the stage list shows that the segmented path ran."""
    w = workloads.workload(base, **ov)
    say(f"[forward segmented] {name}: {w}")
    inp = workloads.make_prefill(w, device="cpu")
    o_ref, s_ref = run_oracle(inp)
    out, st = run_gpu(to_dev(inp), w.chunk, w.mode, flags=kda.STAGE_EVENTS)
    names = _stage_names()
    say(f"  stages {names}")
    assert "chain_summary" in names and "segment_combine" in names
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_forward_segmented_chunk_states_and_phase():
    """Segments together with the chunk-start states output and with the
    phase variant."""
    w = workloads.workload(2, B=1, H=1, T=5000, D=64, chunk=32, s0_std=0.3)
    say(f"[forward segmented] chunk states {w}")
    inp = workloads.make_prefill(w, device="cpu")
    q, k, v, a = (np32(inp[x]) for x in ("q", "k", "v", "alpha"))
    o_ref, s_ref, cs_ref = oracle.forward(q, k, v, a, np32(inp["beta"]), np32(inp["S0"]),
                                          nthreads=oracle_threads(), chunk=32)
    nc = (w.T + 31) // 32
    cs = torch.empty((1, 1, nc, 64, 64), dtype=w.dtype, device=DEV)
    out, st = run_gpu(to_dev(inp), 32, w.mode, chunk_states=cs, flags=kda.STAGE_EVENTS)
    assert "chain_summary" in _stage_names()
    ec = slice_err_state(np32(cs).reshape(1, nc, 64, 64), cs_ref.reshape(1, nc, 64, 64))
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e} chunk states {ec:.3e}")
    assert eo <= 2e-2 and es <= 2e-2 and ec <= 2e-2
    wp = workloads.workload(1, B=1, H=1, T=3000, D=64, chunk=16, s0_std=0.3)
    say(f"[forward segmented] phase {wp}")
    ip = workloads.make_prefill_phase(wp, theta_max=2.0)
    o_ref, s_ref = oracle.forward_phase(np32(ip["q"]), np32(ip["k"]), np32(ip["v"]),
                                        np32(ip["alpha"]), np32(ip["theta"]), np32(ip["beta"]),
                                        np32(ip["S0"]), nthreads=oracle_threads())
    d = to_dev(ip)
    out, st = kda.chunk_forward_phase(d["q"], d["k"], d["v"], d["alpha"], d["theta"], d["beta"],
                                      d["S0"], chunk=16, mode=wp.mode, flags=kda.STAGE_EVENTS)
    torch.cuda.synchronize()
    assert "chain_summary" in _stage_names()
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= 1e-4 and es <= 1e-4


def test_forward_kda_bf16_prefill_full():
    """KDA bf16 prefill, B=1 H=32 T=8192 d=128 chunk=64, every head, through
    the two-pass call the benchmark times for its headline."""
    w = workloads.workload(2)
    say(f"[forward] kda_bf16_prefill full {w}")
    inp = workloads.make_prefill(w, device=DEV)
    out, st = run_gpu(inp, w.chunk, w.mode)
    o_ref, s_ref = run_oracle(inp)
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= 2e-2 and es <= 2e-2


def test_forward_ckda_long_ctx_full():
    """CKDA bf16 long context, B=1 H=16 T=65536 d=128, S0 ~ N(0, 0.02^2), every
    head against the oracle, through the call the benchmark times (streamed,
    from a non-null stream); the parts form (the same side stream lent from
    the null stream) and the two-pass call are bitwise equal to it."""
    w = workloads.workload(3)
    say(f"[forward] ckda_bf16_long_ctx full, all heads {w}")
    inp = workloads.make_prefill(w, device=DEV)
    side = kda.SideStream()
    out, st = run_gpu(inp, w.chunk, w.mode, side=side, flags=kda.STREAMED | kda.STAGE_EVENTS,
                      stream=torch.cuda.Stream())
    assert "chain_stream" in [n for n, _ in kda.last_stage_times()]
    o_ref, s_ref = run_oracle(inp)
    eo = slice_err_out(np32(out), o_ref)
    es = slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= 2e-2 and es <= 2e-2
    out1, st1 = run_gpu(inp, w.chunk, w.mode, side=side, flags=kda.STAGE_EVENTS)
    assert [n for n, _ in kda.last_stage_times()].count("chain") == 8
    out2, st2 = run_gpu(inp, w.chunk, w.mode)
    assert torch.equal(out, out1) and torch.equal(st, st1)
    assert torch.equal(out, out2) and torch.equal(st, st2)


DECODE = [
    ("f32_d16_dv16", torch.float32, 2, 3, 16, 16, 7),
    ("f32_d64_dv48", torch.float32, 1, 2, 64, 48, 5),
    ("bf16_d128_dv128", torch.bfloat16, 4, 4, 128, 128, 9),
    ("bf16_d32_dv80", torch.bfloat16, 3, 2, 32, 80, 4),
    ("bf16_d64_dv96", torch.bfloat16, 3, 3, 64, 96, 6),
    ("bf16_d128_dv32", torch.bfloat16, 2, 5, 128, 32, 5),
    ("f32_d64_dv64", torch.float32, 1, 3, 64, 64, 6),
]


@pytest.mark.parametrize("name,dt,B,H,Dk,Dv,N", DECODE, ids=[c[0] for c in DECODE])
def test_decode_small(name, dt, B, H, Dk, Dv, N):
    say(f"[decode] {name}")
    w = workloads.workload(4, B=B, H=H, D=Dk, dtype=dt, steps=N)
    inp = workloads.make_decode(w)
    inp["v"] = torch.randn(N, B, H, Dv, generator=torch.Generator().manual_seed(9)).to(dt)
    inp["S0"] = inp["S0"][..., :1].expand(B, H, Dk, Dv).contiguous() * torch.linspace(1, 2, Dv)
    o_ref, s_ref = oracle.decode(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
                                 np32(inp["alpha"]), np32(inp["beta"]), np32(inp["S0"]))
    d = to_dev(inp)
    S = d["S0"].clone()
    outs = torch.empty(N, B, H, Dv, dtype=dt, device=DEV)
    for s in range(N):
        kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["alpha"][s], d["beta"][s], S,
                        out=outs[s])
    torch.cuda.synchronize()
    eo = slice_err_out(np.swapaxes(np32(outs), 0, 1), np.swapaxes(o_ref, 0, 1))
    es = slice_err_state(np32(S), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[dt] and es <= TOL[dt]


def test_decode_ckda_bf16_decode_sampled():
    """CKDA decode, B=256 H=32 d=128, state [256,32,128,128] resident and updated
    in place for 1000 steps; the oracle follows every head of 16 batch rows
    (512 pairs: every workgroup-to-XCD residue and both column slices)."""
    w = workloads.workload(4)
    say(f"[decode] ckda_bf16_decode full, 1000 steps, 512 pairs")
    inp = workloads.make_decode(w, device=DEV)
    S = inp["S0"].clone()
    N = w.steps
    outs = torch.empty(N, w.B, w.H, w.D, dtype=w.dtype, device=DEV)
    for s in range(N):
        kda.decode_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["alpha"][s], inp["beta"][s],
                        S, out=outs[s])
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(0, 256, 17) for h in range(w.H)]
    assert len({(b * w.H + h) % 8 for b, h in pairs}) == 8
    bi = torch.tensor([p[0] for p in pairs], device=DEV)
    hi = torch.tensor([p[1] for p in pairs], device=DEV)
    pick = lambda t: t[:, bi, hi].unsqueeze(2)      # [N, P, 1, ...]
    o_ref, s_ref = oracle.decode(np32(pick(inp["q"])), np32(pick(inp["k"])), np32(pick(inp["v"])),
                                 np32(pick(inp["alpha"])), np32(pick(inp["beta"])),
                                 np32(inp["S0"][bi, hi].unsqueeze(1)), nthreads=oracle_threads())
    eo = slice_err_out(np.swapaxes(np32(pick(outs)), 0, 1), np.swapaxes(o_ref, 0, 1))
    es = slice_err_state(np32(S[bi, hi].unsqueeze(1)), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_decode_equals_forward(dt):
    """T decode steps and one chunked forward over the same T tokens agree."""
    say(f"[decode==forward] {dt}")
    w = workloads.workload(1, B=2, H=2, T=40, D=32, chunk=16, dtype=dt, s0_std=0.3)
    inp = to_dev(workloads.make_prefill(w))
    out_f, st_f = run_gpu(inp, 16, workloads.CKDA)
    S = inp["S0"].clone()
    outs = []
    for t in range(w.T):
        sl = lambda x: x[:, t].contiguous()
        outs.append(kda.decode_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]),
                                    sl(inp["beta"]), S))
    out_d = torch.stack(outs, dim=1)
    torch.cuda.synchronize()
    tol = TOL[dt]
    assert slice_err_out(np32(out_d), np32(out_f).astype(np.float64)) <= 2 * tol
    assert slice_err_state(np32(S), np32(st_f).astype(np.float64)) <= 2 * tol


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_resume_and_in_place_state(dt):
    """forward(x1 || x2) = forward(x2; S0 = S_T(x1)), with final_state written
    over initial_state in place."""
    say(f"[resume] {dt}")
    w = workloads.workload(1, B=1, H=3, T=150, D=64, chunk=32, dtype=dt, s0_std=0.1)
    inp = to_dev(workloads.make_prefill(w))
    out_all, st_all = run_gpu(inp, 32, workloads.CKDA)
    cut = 77
    p1 = {k: (v[:, :cut].contiguous() if k not in ("S0",) else v) for k, v in inp.items()}
    p2 = {k: (v[:, cut:].contiguous() if k not in ("S0",) else v) for k, v in inp.items()}
    o1, s1 = run_gpu(p1, 32, workloads.CKDA)
    state = s1.clone()
    o2, s2 = kda.chunk_forward(p2["q"], p2["k"], p2["v"], p2["alpha"], p2["beta"], state,
                               chunk=32, final_state=state)
    torch.cuda.synchronize()
    assert s2.data_ptr() == state.data_ptr()
    tol = TOL[dt]
    both = torch.cat([o1, o2], dim=1)
    assert slice_err_out(np32(both), np32(out_all).astype(np.float64)) <= tol
    assert slice_err_state(np32(state), np32(st_all).astype(np.float64)) <= tol


def test_mode_flag_does_not_change_numbers():
    """KDA-range inputs give bit-identical results in KDA and CKDA mode."""
    say("[mode]")
    w = workloads.workload(2, B=1, H=2, T=300)
    inp = to_dev(workloads.make_prefill(w))
    a = run_gpu(inp, 64, workloads.KDA)
    b = run_gpu(inp, 64, workloads.CKDA)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_deterministic_and_nan_isolated():
    """Two runs are bitwise equal (no LDS race), and a NaN in one head's keys
    leaves every other head bit-identical."""
    say("[determinism / NaN isolation]")
    w = workloads.workload(3, B=1, H=4, T=257)
    inp = to_dev(workloads.make_prefill(w))
    a = run_gpu(inp, 64, workloads.CKDA)
    b = run_gpu(inp, 64, workloads.CKDA)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    bad = dict(inp)
    bad["k"] = inp["k"].clone()
    bad["k"][0, 100, 2, 5] = float("nan")
    c = run_gpu(bad, 64, workloads.CKDA)
    others = [0, 1, 3]
    assert torch.equal(a[0][:, :, others], c[0][:, :, others])
    assert torch.equal(a[1][:, others], c[1][:, others])
    assert torch.isnan(c[0][:, 100:, 2]).any()


def test_empty_sequence_copies_state():
    say("[T=0]")
    s0 = torch.randn(2, 3, 16, 32, device=DEV)
    x = torch.empty(2, 0, 3, 16, device=DEV)
    v = torch.empty(2, 0, 3, 32, device=DEV)
    out, st = kda.chunk_forward(x, x, v, x, torch.empty(2, 0, 3, device=DEV), s0, chunk=16)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 3, 32) and torch.equal(st, s0)


def test_gate_prep_matches_oracle():
    """Gate summary: parity and last-zero index exact; L within the fp32
    accumulation bound; chunk decay within fp32 product rounding."""
    say("[gate_prep]")
    w = workloads.workload(1, B=2, H=3, T=203, D=64, chunk=64)
    inp = workloads.make_prefill(w)
    ref = oracle.gate_prep(np32(inp["alpha"]), 64)
    L, meta, gend = kda.gate_prep(inp["alpha"].to(DEV), 64)
    torch.cuda.synchronize()
    meta = meta.cpu().numpy()
    T, C = w.T, w.chunk
    valid = np.zeros(ref["L"].shape, dtype=bool)
    for n in range(ref["L"].shape[2]):
        valid[:, :, n, :max(0, min(C, T - n * C))] = True
    assert np.array_equal((meta & 1)[valid], ref["parity"][valid])
    assert np.array_equal((meta >> 1)[valid], ref["zpos"][valid])
    assert np.all(meta[~valid] == 0)
    # per step: log2 rounding (<= 2^-22 |log2 a|) + one fp32 add (<= 2^-24 |L|)
    Lg = L.cpu().numpy().astype(np.float64)
    r_idx = np.arange(C)[None, None, None, :, None] + 1
    bound = r_idx * (2.0 ** -22 * 40 + 2.0 ** -24 * np.abs(ref["L"]).max()) + 1e-7
    assert np.all(np.abs(Lg - ref["L"])[valid] <= np.broadcast_to(bound, Lg.shape)[valid])
    g = gend.cpu().numpy().astype(np.float64)
    assert np.allclose(g, ref["gend"], rtol=64 * 2.0 ** -23, atol=1e-37)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_exact_fallback_chunks(dt):
    """Chunks the fast prep kernel cannot factor go to the exact kernel:
    zero gates in KDA mode (no extra zero-segment columns) and gates so small
    that a chunk's log2 decay spans more than the midpoint factorisation allows.
    Flagged and unflagged chunks are mixed in one call; results must still
    match the oracle."""
    say(f"[fallback] {dt}")
    D = 64 if dt == torch.float32 else 128
    w = workloads.workload(1, B=1, H=3, T=200, D=D, chunk=64, dtype=dt)
    inp = workloads.make_prefill(w)
    a = inp["alpha"]
    a[0, 70:80, 1, :5] = 1e-12          # head 1, chunk 1: ~40 bits per token
    a[0, 150:190, 2, 3] = 2.0 ** -30    # head 2, chunk 2: span >> 192 bits
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    for mode in (workloads.KDA, workloads.CKDA):
        out, st = run_gpu(d, 64, mode)
        eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
        say(f"  mode {mode}: err out {eo:.3e} state {es:.3e}")
        assert eo <= TOL[dt] and es <= TOL[dt]


def _unit_flags(ws, w):
    """The per-unit fallback flags of a single-pass forward, read from its
    workspace (white-box: the regions W, U, Ktil, Q*Gamma, P, Gamma_C, FL in
    that order, each starting on a 256-byte boundary; FL is one byte per
    (b, h, chunk) unit)."""
    nc = (w.T + w.chunk - 1) // w.chunk
    nu = w.B * w.H * nc
    e = 4 if w.dtype == torch.float32 else 2
    C, D = w.chunk, w.D
    sizes = [nu * C * D * e, nu * C * D * e, nu * D * C * e, nu * C * D * e, nu * C * C * e, nu * D * 4]
    off = sum((x + 255) // 256 * 256 for x in sizes)
    assert off + (nu + 255) // 256 * 256 == ws.numel()
    return ws[off:off + nu].cpu()


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("ckda", [False, True])
def test_half_span_band_stays_fast(dt, ckda):
    """Chunks whose log2 decay over 64 tokens spans 128 to 192 bits in some
    channels (half spans 64 < |M| <= 96 of the midpoint factorisation): the
    factors reach 2^96 and the masked upper-triangle products overflow, yet
    the chunks stay on the fast kernel (no unit flagged) and match the oracle.
    KDA-range gates run in both modes; CKDA gates (signs, exact -1 and 0)
    in CKDA mode."""
    D = 64 if dt == torch.float32 else 128
    w = workloads.workload(1 if ckda else 0, B=1, H=4, T=256 + 19, D=D, chunk=64, dtype=dt,
                           s0_std=0.3)
    say(f"[half-span band] {dt} ckda={ckda} {w}")
    inp = workloads.make_prefill(w)
    a = inp["alpha"]
    sgn = lambda x: torch.where(x < 0, -1.0, 1.0)
    # head 0, chunk 1, channels 0-7: 2.2 bits per token -> half span 70.4
    a[0, 64:128, 0, :8] = sgn(a[0, 64:128, 0, :8]) * 2.0 ** -2.2
    # head 1, chunk 2, channels 10-20: 2.8 bits per token -> half span 89.6
    a[0, 128:192, 1, 10:21] = sgn(a[0, 128:192, 1, 10:21]) * 2.0 ** -2.8
    # head 2, chunk 0, every channel: 2.95 bits per token -> half span 94.4
    a[0, 0:64, 2, :] = sgn(a[0, 0:64, 2, :]) * 2.0 ** -2.95
    # head 3, chunk 3, channels 30-33: half span 81 on channels with mixed gates
    a[0, 192:256:2, 3, 30:34] = sgn(a[0, 192:256:2, 3, 30:34]) * 2.0 ** -4.0
    a[0, 193:256:2, 3, 30:34] = sgn(a[0, 193:256:2, 3, 30:34]) * 2.0 ** -1.0625
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, D, D, 64, dt), dtype=torch.uint8, device=DEV)
    for mode in ((workloads.CKDA,) if ckda else (workloads.KDA, workloads.CKDA)):
        out, st = run_gpu(d, 64, mode, workspace=ws)
        fl = _unit_flags(ws, w)
        eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
        say(f"  mode {mode}: flagged units {int(fl.sum())}, err out {eo:.3e} state {es:.3e}")
        assert int(fl.sum()) == 0
        assert eo <= TOL[dt] and es <= TOL[dt]


# zero-gate rate per head: about 1, 2, 3 and 4 extra contraction passes of the
# fast prep kernel (Dk zero-segment columns each), then more zeros than the
# CKDA column budget (4 Dk per chunk) so that chunk goes to the exact kernel
DENSE_ZERO_RATES = (0.012, 0.024, 0.04, 0.056, 0.09)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_forward_dense_zero_gates(dt):
    """CKDA gates with many exact zeros: every later zero segment of a channel
    is its own contraction column, contracted Dk columns per pass.  Heads with
    rising zero rates take one to four extra passes or the exact kernel; one
    more head puts a zero on every other token of channels 0 and Dk - 1
    (32 segments in one channel) and at the first and last token of every
    chunk.  Results must match the oracle."""
    D = 64 if dt == torch.float32 else 128
    H = len(DENSE_ZERO_RATES) + 1
    w = workloads.workload(1, B=1, H=H, T=256 + 37, D=D, chunk=64, dtype=dt, s0_std=0.3)
    say(f"[dense zeros] {dt} {w}")
    inp = workloads.make_prefill(w)
    a = inp["alpha"]
    g = torch.Generator().manual_seed(77)
    for h, rate in enumerate(DENSE_ZERO_RATES):
        mask = torch.rand(a[:, :, h].shape, generator=g) < rate
        a[:, :, h][mask] = 0.0
    hz = H - 1
    a[0, 1::2, hz, 0] = 0.0
    a[0, ::2, hz, D - 1] = 0.0
    a[0, ::64, hz, :] = 0.0
    a[0, 63::64, hz, 5:9] = 0.0
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    out, st = run_gpu(d, 64, workloads.CKDA)
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[dt] and es <= TOL[dt]


# (name, base workload, overrides, flags) — at most 128 (b, h, 16-column)
# chains and at least 256 chunks, so with a side stream the forward runs in
# parts: chunk factors of part p + 1 on the caller's second stream while the
# chain runs part p
PARTS = [
    ("bf16_ckda_d128_c16_H9_T4133_s0", 3, dict(B=1, H=9, T=4133, chunk=16, s0_std=0.2), 0),
    ("f32_kda_d32_c16_B2_T4100_nosegments", 0, dict(B=2, H=1, T=4100, D=32, chunk=16),
     kda.NO_SEGMENTS),
]


@pytest.mark.parametrize("name,base,ov,flags", PARTS, ids=[c[0] for c in PARTS])
def test_forward_parts(name, base, ov, flags):
    """Prep / chain overlap in parts on a caller-owned side stream
    (kda_chunk_forward_side): the oracle's sequential recurrence, and bitwise
    the single-stream path for the outputs and the final state; the stage list
    shows one chain launch per part.  Without a side stream, or with
    KDA_FLAG_SINGLE_STREAM, the call keeps to one stream (one chain launch)."""
    w = workloads.workload(base, **ov)
    say(f"[forward parts] {name}: {w}")
    inp = workloads.make_prefill(w, device="cpu")
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    side = kda.SideStream()
    out, st = run_gpu(d, w.chunk, w.mode, flags=flags | kda.STAGE_EVENTS, side=side)
    names = _stage_names()
    say(f"  stages {names}")
    assert names.count("chain") == 8 and names.count("prep_fast") == 8
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
    for kw in (dict(flags=flags | kda.STAGE_EVENTS),
               dict(flags=flags | kda.SINGLE_STREAM | kda.STAGE_EVENTS, side=side)):
        out1, st1 = run_gpu(d, w.chunk, w.mode, **kw)
        assert _stage_names().count("chain") == 1
        assert torch.equal(out, out1) and torch.equal(st, st1)
    # an explicit (non-default) caller stream with the side stream
    cs_ = torch.cuda.Stream()
    cs_.wait_stream(torch.cuda.current_stream())
    out2, st2 = run_gpu(d, w.chunk, w.mode, flags=flags | kda.STAGE_EVENTS, stream=cs_, side=side)
    assert _stage_names().count("chain") == 8
    assert torch.equal(out, out2) and torch.equal(st, st2)
    # the same side stream lent to two calls enqueued back to back
    outs = [run_gpu(d, w.chunk, w.mode, flags=flags, side=side) for _ in range(2)]
    for o3, s3 in outs:
        assert torch.equal(o3, out) and torch.equal(s3, st)


def test_forward_phase_long_single_stream():
    """The phase variant at a shape the plain forward would run in parts with a
    side stream: one stream, one chain launch, against the oracle's phase
    recurrence."""
    w = workloads.workload(3, B=1, H=9, T=4133, chunk=16, s0_std=0.2)
    say(f"[forward phase long] {w}")
    inp = workloads.make_prefill_phase(w, theta_max=2.0)
    o_ref, s_ref = oracle.forward_phase(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
                                        np32(inp["alpha"]), np32(inp["theta"]), np32(inp["beta"]),
                                        np32(inp["S0"]), nthreads=oracle_threads())
    d = to_dev(inp)
    out, st = kda.chunk_forward_phase(d["q"], d["k"], d["v"], d["alpha"], d["theta"], d["beta"],
                                      d["S0"], chunk=w.chunk, mode=w.mode, flags=kda.STAGE_EVENTS)
    torch.cuda.synchronize()
    names = [n for n, _ in kda.last_stage_times()]
    assert names.count("chain") == 1
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("dt,Dk,Dv,mode,pro", [
    (torch.bfloat16, 128, 128, workloads.CKDA, (-1.0, 1.0, 2.0, 1e-6, True)),
    (torch.float32, 64, 48, workloads.KDA, (0.0, 1.0, 1.0, 1e-6, False)),
    (torch.bfloat16, 32, 80, workloads.CKDA, (-1.0, 1.0, 2.0, 0.0, True)),
    # eps of the order of the raw norms (|k_raw| ~ 11 at Dk = 128, 8 at 64)
    (torch.bfloat16, 128, 128, workloads.CKDA, (-1.0, 1.0, 2.0, 4.0, True)),
    (torch.float32, 64, 64, workloads.KDA, (0.0, 1.0, 1.0, 3.0, True)),
])
def test_decode_prologue(dt, Dk, Dv, mode, pro):
    """kda_decode_step_prologue: six steps from raw inputs (gate and beta
    logits, unnormalised q, k; some gates at -200, i.e. alpha = alpha_min)
    against the oracle's prologue recurrence over the same tokens."""
    amin, amax, bmax, eps, normq = pro
    say(f"[decode prologue] {dt} Dk={Dk} Dv={Dv} mode={mode} pro={pro}")
    g = torch.Generator().manual_seed(Dk * 7 + Dv)
    B, H, N = 3, 2, 6
    q = torch.randn(N, B, H, Dk, generator=g).to(dt)
    k = torch.randn(N, B, H, Dk, generator=g).to(dt)
    v = torch.randn(N, B, H, Dv, generator=g).to(dt)
    gate = 2.0 * torch.randn(N, B, H, Dk, generator=g)
    gate[torch.rand(N, B, H, Dk, generator=g) < 0.05] = -200.0
    blog = torch.randn(N, B, H, generator=g)
    S0 = 0.3 * torch.randn(B, H, Dk, Dv, generator=g)
    S = S0.to(DEV).contiguous()
    outs = []
    for t in range(N):
        outs.append(kda.decode_step_prologue(q[t].to(DEV), k[t].to(DEV), v[t].to(DEV),
                                             gate[t].to(DEV), blog[t].to(DEV).contiguous(), S,
                                             alpha_min=amin, alpha_max=amax, beta_max=bmax,
                                             eps=eps, normalize_q=normq, mode=mode))
    torch.cuda.synchronize()
    perm = lambda x: np32(x.permute(1, 0, *range(2, x.dim())))
    o_ref, s_ref = oracle.forward_prologue(perm(q), perm(k), perm(v), perm(gate), perm(blog),
                                           np32(S0), alpha_min=amin, alpha_max=amax,
                                           beta_max=bmax, eps=eps, normalize_q=normq)
    o_gpu = np.stack([np32(o) for o in outs], axis=1)
    eo, es = slice_err_out(o_gpu, o_ref), slice_err_state(np32(S), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[dt] and es <= TOL[dt]


# fp32 with Dk or Dv = 128: cfg1-style CKDA inputs (signs, exact -1 and 0 gates,
# beta up to exactly 2) at d = 128
F32_128 = [
    ("f32_ckda_d128_c64_B2_H4_T1024", 1, dict(B=2, H=4, T=1024, D=128, chunk=64), None),
    ("f32_kda_d128_c64_T201_s0", 0, dict(B=1, H=3, T=201, D=128, chunk=64, s0_std=0.3), None),
    ("f32_ckda_dk64_dv128_c32_T130", 1, dict(B=1, H=2, T=130, D=64, chunk=32), 128),
    ("f32_ckda_dk64_dv128_c16_T77_s0", 1, dict(B=2, H=1, T=77, D=64, chunk=16, s0_std=0.2), 128),
]


@pytest.mark.parametrize("name,base,ov,dv", F32_128, ids=[c[0] for c in F32_128])
def test_forward_f32_d128(name, base, ov, dv):
    """The fp32 chunked forward at Dk = 128 (chunk 64) and at Dv = 128 (Dk = 64,
    any chunk) against the oracle at the fp32 tolerance."""
    w = workloads.workload(base, **ov)
    say(f"[forward fp32 128] {name}: {w} Dv={dv or w.D}")
    inp = workloads.make_prefill(w, device="cpu")
    if dv is not None:
        g = torch.Generator().manual_seed(77)
        inp["v"] = torch.randn((w.B, w.T, w.H, dv), generator=g).contiguous()
        if inp.get("S0") is not None:
            inp["S0"] = (0.2 * torch.randn((w.B, w.H, w.D, dv), generator=g)).contiguous()
    if base == 1:
        a = inp["alpha"]
        assert bool((a == -1.0).any()) and bool((a == 0.0).any())
        assert bool((inp["beta"] == 2.0).any())
    o_ref, s_ref = run_oracle(inp)
    out, st = run_gpu(to_dev(inp), w.chunk, w.mode)
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= 1e-4 and es <= 1e-4


def test_forward_f32_d128_exact_fallback_and_states():
    """fp32 Dk = 128: chunks flagged for the exact kernel (a KDA-mode zero gate;
    a span beyond the fast factorisation) through the half-channel factor
    passes, the chunk-start states, and a packed batch."""
    w = workloads.workload(1, B=1, H=3, T=200, D=128, chunk=64, dtype=torch.float32)
    say(f"[fp32 d128 fallback] {w}")
    inp = workloads.make_prefill(w)
    a = inp["alpha"]
    a.abs_()                                  # KDA-range gates ...
    a[0, 70, 1, 5] = 0.0                      # ... with one exact zero (KDA mode: exact kernel)
    a[0, 150:190, 2, 3] = 2.0 ** -30          # a span far beyond the midpoint factorisation
    inp["beta"].clamp_(max=1.0)
    q, k, v = (np32(inp[x]) for x in ("q", "k", "v"))
    o_ref, s_ref, cs_ref = oracle.forward(q, k, v, np32(a), np32(inp["beta"]), None,
                                          nthreads=oracle_threads(), chunk=64)
    d = to_dev(inp)
    nc = (w.T + 63) // 64
    cs = torch.full((w.B, w.H, nc, w.D, w.D), float("nan"), dtype=torch.float32, device=DEV)
    for mode in (workloads.KDA, workloads.CKDA):
        out, st = run_gpu(d, 64, mode, chunk_states=cs)
        eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
        ec = slice_err_state(np32(cs).reshape(w.B, w.H * nc, w.D, w.D),
                             cs_ref.reshape(w.B, w.H * nc, w.D, w.D))
        say(f"  mode {mode}: err out {eo:.3e} state {es:.3e} chunk states {ec:.3e}")
        assert eo <= 1e-4 and es <= 1e-4 and ec <= 1e-4
    # packed batch of the same tokens as sequences of 70 and 130
    cu = torch.tensor([0, 70, 200], dtype=torch.int32, device=DEV)
    outv, stv = kda.chunk_forward_varlen(d["q"][0], d["k"][0], d["v"][0], d["alpha"][0],
                                         d["beta"][0], cu, None, chunk=64, mode=workloads.CKDA)
    torch.cuda.synchronize()
    for i, (lo, hi) in enumerate(((0, 70), (70, 200))):
        sub = {x: inp[x][:, lo:hi] for x in ("q", "k", "v", "alpha", "beta")}
        sub["S0"] = None
        o_r, s_r = run_oracle(sub)
        assert slice_err_out(np32(outv[lo:hi])[None], o_r) <= 1e-4
        assert slice_err_state(np32(stv[i:i + 1]), s_r) <= 1e-4
