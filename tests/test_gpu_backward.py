"""GPU parity of the chunkwise backward (kda_chunk_backward) against the
oracle's token-by-token gradients.

Each case prints its name before touching the GPU.  Inputs come from
workloads.py; expected values only from oracle/.  Error measure as for the
forward (tests/parity.py): per (b, h) slice, max |gpu - oracle| / max |oracle|,
for every gradient separately; fp32 within 1e-4, bf16 within 2e-2.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import oracle
import workloads
from parity import TOL, np32, oracle_threads, say, slice_err_out, slice_err_state

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (name, base workload, overrides, with S0, with dST)
CASES = [
    ("f32_kda_d64_c64_T200", 0, dict(B=1, H=2, T=200, D=64, chunk=64), True, True),
    ("f32_ckda_d64_c64_T130", 1, dict(B=2, H=2, T=130, D=64, chunk=64), False, True),
    ("f32_ckda_d32_c32_T77", 1, dict(B=1, H=3, T=77, D=32, chunk=32), True, False),
    ("f32_kda_d64_c32_T1", 0, dict(B=2, H=1, T=1, D=64, chunk=32), True, True),
    ("bf16_kda_d128_c64_T300", 2, dict(B=1, H=2, T=300, chunk=64), True, True),
    ("bf16_ckda_d128_c64_T257", 3, dict(B=1, H=2, T=257, chunk=64), True, False),
    ("bf16_ckda_d64_c64_T192", 3, dict(B=2, H=1, T=192, D=64, chunk=64), False, True),
    ("bf16_ckda_d128_c32_T100", 3, dict(B=1, H=2, T=100, chunk=32), True, True),
    ("bf16_kda_d32_c32_T65", 2, dict(B=1, H=2, T=65, D=32, chunk=32), False, False),
]

GRADS = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("d_alpha", "dalpha"), ("d_beta", "dbeta")]


def _inputs(base, ov, s0, dst):
    w = workloads.workload(base, **ov)
    if s0 and w.s0_std is None:
        w = workloads.workload(base, **ov, s0_std=0.5)
    if not s0:
        w = workloads.workload(base, **{**ov, "s0_std": None})
    inp = workloads.make_prefill(w)
    dO, dST = workloads.make_backward_seeds(w, dst=dst)
    return w, inp, dO, dST


def _oracle(inp, dO, dST):
    s0 = None if inp["S0"] is None else np32(inp["S0"])
    return oracle.backward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(inp["alpha"]),
                           np32(inp["beta"]), np32(dO), s0, None if dST is None else np32(dST),
                           nthreads=oracle_threads())


def _gpu(w, inp, dO, dST, **kw):
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    g = kda.chunk_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(DEV), d["S0"],
                           None if dST is None else dST.to(DEV), chunk=w.chunk, mode=w.mode, **kw)
    torch.cuda.synchronize()
    return g


def _errors(g, ref):
    errs = {}
    for gn, rn in GRADS:
        a, b = np32(g[gn]), ref[rn]
        if a.ndim == 3:
            a, b = a[..., None], b[..., None]
        errs[gn] = slice_err_out(a, b)
    errs["d_initial_state"] = slice_err_state(np32(g["d_initial_state"]), ref["dS0"])
    return errs


@pytest.mark.parametrize("name,base,ov,s0,dst", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, base, ov, s0, dst):
    w, inp, dO, dST = _inputs(base, ov, s0, dst)
    say(f"[backward] {name}: {w} S0={s0} dST={dst}")
    ref = _oracle(inp, dO, dST)
    g = _gpu(w, inp, dO, dST)
    errs = _errors(g, ref)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (k, v)


def test_backward_empty_sequence_passes_dst_through():
    """T = 0: the loss is <S0, dST>, so dS0 = dST and nothing else is written."""
    say("[backward] T=0")
    B, H, D = 1, 2, 64
    z = torch.empty((B, 0, H, D), device=DEV)
    dST = torch.randn((B, H, D, D), device=DEV)
    g = kda.chunk_backward(z, z, z, z, torch.empty((B, 0, H), device=DEV), z, None, dST,
                           chunk=64, mode=workloads.CKDA)
    torch.cuda.synchronize()
    assert torch.equal(g["d_initial_state"], dST)


def test_backward_small_gates_take_the_direct_form():
    """Gates at exactly 0 and just below 2^-6 in magnitude (the quotient form's
    limit) in every chunk: d_alpha there comes from the direct per-channel
    form and must still match the oracle."""
    w = workloads.workload(1, B=1, H=2, T=150, D=64, chunk=64, s0_std=0.5)
    inp = workloads.make_prefill(w)
    a = inp["alpha"]
    gen = torch.Generator().manual_seed(5)
    m = torch.rand(a.shape, generator=gen)
    a[m < 0.02] = 0.0
    a[(m >= 0.02) & (m < 0.04)] = 0.0151
    a[(m >= 0.04) & (m < 0.06)] = -0.003
    dO, dST = workloads.make_backward_seeds(w)
    say("[backward] small gates f32 d64 T150")
    ref = _oracle(inp, dO, dST)
    g = _gpu(w, inp, dO, dST)
    errs = _errors(g, ref)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (k, v)


def test_backward_without_initial_state_gradient():
    """d_initial_state = NULL is allowed and changes nothing else."""
    w, inp, dO, dST = _inputs(1, dict(B=1, H=2, T=100, D=32, chunk=32), True, True)
    say("[backward] no d_initial_state")
    g1 = _gpu(w, inp, dO, dST)
    g2 = _gpu(w, inp, dO, dST, want_d_initial_state=False)
    assert g2["d_initial_state"] is None
    for gn, _ in GRADS:
        assert torch.equal(g1[gn], g2[gn]), gn


def test_backward_full_headline_shape_sampled_heads():
    """The headline shape (B=1, H=32, T=8192, d=128, bf16 KDA, chunk 64) in the
    launch configuration the benchmark times: every head on the GPU, the
    oracle's gradients for three sampled heads."""
    w = workloads.workload(2)
    inp = workloads.make_prefill(w)
    dO, dST = workloads.make_backward_seeds(w)
    say(f"[backward] full {w.name}")
    g = _gpu(w, inp, dO, dST)
    heads = [0, 13, 31]
    sel = lambda t: None if t is None else t[:, :, heads].contiguous()
    sub = {k: sel(v) for k, v in inp.items() if k != "S0"}
    sub["S0"] = None if inp["S0"] is None else inp["S0"][:, heads].contiguous()
    ref = _oracle(sub, sel(dO), dST[:, heads].contiguous())
    gs = {k: (None if v is None else (v[:, :, heads] if k != "d_initial_state" else v[:, heads]))
          for k, v in g.items()}
    errs = _errors(gs, ref)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (k, v)


@pytest.mark.parametrize("name,base,ov,dv", [
    ("f32_ckda_dk64_dv32_c64_T150", 1, dict(B=1, H=2, T=150, D=64, chunk=64), 32),
    ("bf16_ckda_dk128_dv64_c64_T200", 3, dict(B=1, H=2, T=200, chunk=64), 64),
    ("bf16_kda_dk64_dv112_c32_T90", 2, dict(B=1, H=1, T=90, D=64, chunk=32), None),
])
def test_backward_dk_ne_dv(name, base, ov, dv):
    """Dk != Dv: rows and columns of the state and its gradient must not be
    swapped anywhere (v, dO and dS_T keep their first Dv columns; for Dv >
    Dk the inputs are drawn at width Dv and q, k, alpha cut to Dk)."""
    w, inp, dO, dST = _inputs(base, ov, True, True)
    if dv is None:
        # Dv = 112 > Dk = 64: draw at D = 112 and cut the key side
        w = workloads.workload(base, **{**ov, "D": 112, "s0_std": 0.5})
        inp = workloads.make_prefill(w)
        dO, dST = workloads.make_backward_seeds(w)
        for k_ in ("q", "k", "alpha"):
            inp[k_] = inp[k_][..., :64].contiguous()
        # keys back to unit length after the cut (the recipe's normalisation)
        inp["k"] = (inp["k"].float() / inp["k"].float().norm(dim=-1, keepdim=True)).to(w.dtype).contiguous()
        inp["S0"] = inp["S0"][:, :, :64, :].contiguous()
        dST = dST[:, :, :64, :].contiguous()
    else:
        inp["v"] = inp["v"][..., :dv].contiguous()
        dO = dO[..., :dv].contiguous()
        if inp["S0"] is not None:
            inp["S0"] = inp["S0"][..., :dv].contiguous()
        dST = dST[..., :dv].contiguous()
    say(f"[backward] {name}: q {tuple(inp['q'].shape)} v {tuple(inp['v'].shape)}")
    ref = _oracle(inp, dO, dST)
    g = _gpu(w, inp, dO, dST)
    errs = _errors(g, ref)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (k, v)


# ---- backward from raw inputs (kda_chunk_backward_prologue) ---------------------
PRO_CASES = [
    ("f32_ckda_d64_c64_T150", 1, dict(B=1, H=2, T=150, D=64, chunk=64, s0_std=0.5),
     dict(alpha_min=-1.0, alpha_max=1.0, beta_max=2.0, eps=1e-6, normalize_q=True)),
    ("f32_kda_d32_c32_T70_noqnorm", 0, dict(B=2, H=1, T=70, D=32, chunk=32),
     dict(alpha_min=0.0, alpha_max=1.0, beta_max=1.0, eps=0.25, normalize_q=False)),
    ("bf16_ckda_d128_c64_T200", 3, dict(B=1, H=2, T=200, chunk=64),
     dict(alpha_min=-1.0, alpha_max=1.0, beta_max=2.0, eps=1e-6, normalize_q=True)),
    ("bf16_kda_d64_c64_T129", 2, dict(B=1, H=2, T=129, D=64, chunk=64, s0_std=0.3),
     dict(alpha_min=0.2, alpha_max=0.99, beta_max=1.0, eps=0.0, normalize_q=True)),
]


@pytest.mark.parametrize("name,base,ov,pro", PRO_CASES, ids=[c[0] for c in PRO_CASES])
def test_backward_prologue_matches_oracle(name, base, ov, pro):
    w = workloads.workload(base, **ov)
    raw = workloads.make_prefill_raw(w)
    dO, dST = workloads.make_backward_seeds(w)
    say(f"[backward prologue] {name}: {pro}")
    s0 = None if raw["S0"] is None else np32(raw["S0"])
    ref = oracle.backward_prologue(np32(raw["q"]), np32(raw["k"]), np32(raw["v"]), np32(raw["gate"]),
                                   np32(raw["beta_logit"]), np32(dO), s0, np32(dST),
                                   nthreads=oracle_threads(), **pro)
    d = {k: (None if v is None else v.to(DEV)) for k, v in raw.items()}
    g = kda.chunk_backward_prologue(d["q"], d["k"], d["v"], d["gate"], d["beta_logit"], dO.to(DEV),
                                    d["S0"], dST.to(DEV), chunk=w.chunk, mode=w.mode, **pro)
    torch.cuda.synchronize()
    pairs = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("d_gate", "dgate"),
             ("d_beta_logit", "dbeta_logit"))
    errs = {}
    for gn, rn in pairs:
        a_, b_ = np32(g[gn]), ref[rn]
        if a_.ndim == 3:
            a_, b_ = a_[..., None], b_[..., None]
        errs[gn] = slice_err_out(a_, b_)
    errs["d_initial_state"] = slice_err_state(np32(g["d_initial_state"]), ref["dS0"])
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[w.dtype], (k, v)


# ---- packed batches (kda_chunk_backward_varlen) ---------------------------------
VL_CASES = [
    ("f32_ckda_d64_c64", 1, dict(H=2, D=64, chunk=64, s0_std=0.5), [70, 0, 1, 130, 64]),
    ("bf16_ckda_d128_c64", 3, dict(H=2, chunk=64), [200, 33, 0, 64]),
    ("bf16_kda_d64_c32", 2, dict(H=1, D=64, chunk=32, s0_std=0.3), [5, 97, 32]),
]


@pytest.mark.parametrize("name,base,ov,lengths", VL_CASES, ids=[c[0] for c in VL_CASES])
def test_backward_varlen_matches_oracle(name, base, ov, lengths):
    """Every sequence of the packed batch against the oracle's gradients of
    that sequence alone (its own initial state and final-state gradient)."""
    w = workloads.workload(base, **ov)
    inp = workloads.make_varlen(w, lengths)
    N, total = len(lengths), sum(lengths)
    gen = torch.Generator().manual_seed(77)
    dO = torch.randn((1, total, w.H, w.D), generator=gen).to(w.dtype)
    dST = torch.randn((N, w.H, w.D, w.D), generator=gen)
    say(f"[backward varlen] {name}: lengths {lengths}")
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    g = kda.chunk_backward_varlen(d["q"][0], d["k"][0], d["v"][0], d["alpha"][0], d["beta"][0],
                                  d["cu_seqlens"], dO[0].to(DEV), d["S0"], dST.to(DEV),
                                  chunk=w.chunk, mode=w.mode)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    worst = {}
    for i, L in enumerate(lengths):
        sl = slice(cu[i], cu[i + 1])
        sub = {x: inp[x][:, sl] for x in ("q", "k", "v", "alpha", "beta")}
        sub["S0"] = None if inp["S0"] is None else inp["S0"][i:i + 1]
        ref = _oracle(sub, dO[:, sl], dST[i:i + 1])
        e = {"d_initial_state": slice_err_state(np32(g["d_initial_state"][i:i + 1]), ref["dS0"])}
        if L > 0:
            for gn, rn in GRADS:
                a_, b_ = np32(g[gn][sl])[None], ref[rn]
                if a_.ndim == 3:
                    a_, b_ = a_[..., None], b_[..., None]
                e[gn] = slice_err_out(a_, b_)
        for k_, v_ in e.items():
            worst[k_] = max(worst.get(k_, 0.0), v_)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    for k_, v_ in worst.items():
        assert v_ <= TOL[w.dtype], (k_, v_)


def test_backward_varlen_uniform_equals_dense():
    """Equal lengths: the packed batch numbers its chunks like the dense batch,
    so every gradient is bit-identical to kda_chunk_backward's."""
    w = workloads.workload(2, B=3, H=2, T=100, chunk=64, s0_std=0.2)
    say(f"[backward varlen] uniform vs dense {w}")
    inp = workloads.make_prefill(w)
    dO, dST = workloads.make_backward_seeds(w)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    gd = kda.chunk_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(DEV), d["S0"],
                            dST.to(DEV), chunk=64, mode=w.mode)
    flat = lambda t: t.reshape(w.B * w.T, *t.shape[2:]).contiguous()
    cu = torch.arange(0, (w.B + 1) * w.T, w.T, dtype=torch.int32, device=DEV)
    gv = kda.chunk_backward_varlen(flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["alpha"]),
                                   flat(d["beta"]), cu, flat(dO.to(DEV)), d["S0"], dST.to(DEV),
                                   chunk=64, mode=w.mode)
    torch.cuda.synchronize()
    for gn in ("dq", "dk", "dv", "d_alpha", "d_beta"):
        assert torch.equal(flat(gd[gn]), gv[gn]), gn
    assert torch.equal(gd["d_initial_state"], gv["d_initial_state"])


# ---- packed batches from raw inputs (kda_chunk_backward_varlen_prologue) ---------
VLP_CASES = [
    ("f32_ckda_d64_c64", 1, dict(H=2, D=64, chunk=64), [70, 0, 1, 130],
     dict(alpha_min=-1.0, alpha_max=1.0, beta_max=2.0, eps=1e-6, normalize_q=True)),
    ("bf16_kda_d128_c32", 2, dict(H=1, chunk=32), [97, 33, 64],
     dict(alpha_min=0.0, alpha_max=1.0, beta_max=1.0, eps=1e-6, normalize_q=False)),
]


@pytest.mark.parametrize("name,base,ov,lengths,pro", VLP_CASES, ids=[c[0] for c in VLP_CASES])
def test_backward_varlen_prologue_matches_oracle(name, base, ov, lengths, pro):
    """Every sequence of a packed batch from raw inputs against the oracle's
    raw-input gradients of that sequence alone."""
    N, total = len(lengths), sum(lengths)
    w = workloads.workload(base, B=1, T=total, s0_std=None, **ov)
    raw = workloads.make_prefill_raw(w, forget_frac=0.01)
    gen = torch.Generator().manual_seed(91)
    S0 = 0.3 * torch.randn((N, w.H, w.D, w.D), generator=gen)
    dO = torch.randn((1, total, w.H, w.D), generator=gen).to(w.dtype)
    dST = torch.randn((N, w.H, w.D, w.D), generator=gen)
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    say(f"[backward varlen prologue] {name}: lengths {lengths} {pro}")
    d = {k: (None if v is None else v.to(DEV)) for k, v in raw.items()}
    g = kda.chunk_backward_varlen_prologue(d["q"][0], d["k"][0], d["v"][0], d["gate"][0],
                                           d["beta_logit"][0], cu.to(DEV), dO[0].to(DEV),
                                           S0.to(DEV), dST.to(DEV), chunk=w.chunk, mode=w.mode,
                                           **pro)
    torch.cuda.synchronize()
    c = cu.tolist()
    worst = {}
    pairs = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("d_gate", "dgate"),
             ("d_beta_logit", "dbeta_logit"))
    for i, L in enumerate(lengths):
        sl = slice(c[i], c[i + 1])
        ref = oracle.backward_prologue(np32(raw["q"][:, sl]), np32(raw["k"][:, sl]),
                                       np32(raw["v"][:, sl]), np32(raw["gate"][:, sl]),
                                       np32(raw["beta_logit"][:, sl]), np32(dO[:, sl]),
                                       np32(S0[i:i + 1]), np32(dST[i:i + 1]),
                                       nthreads=oracle_threads(), **pro)
        e = {"d_initial_state": slice_err_state(np32(g["d_initial_state"][i:i + 1]), ref["dS0"])}
        if L > 0:
            for gn, rn in pairs:
                a_, b_ = np32(g[gn][sl])[None], ref[rn]
                if a_.ndim == 3:
                    a_, b_ = a_[..., None], b_[..., None]
                e[gn] = slice_err_out(a_, b_)
        for k_, v_ in e.items():
            worst[k_] = max(worst.get(k_, 0.0), v_)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    for k_, v_ in worst.items():
        assert v_ <= TOL[w.dtype], (k_, v_)


def test_backward_varlen_prologue_uniform_equals_dense():
    """Equal lengths: bit-identical to kda_chunk_backward_prologue."""
    w = workloads.workload(3, B=3, H=2, T=100, chunk=64, s0_std=0.2)
    say(f"[backward varlen prologue] uniform vs dense {w}")
    raw = workloads.make_prefill_raw(w, forget_frac=0.01)
    dO, dST = workloads.make_backward_seeds(w)
    pro = dict(alpha_min=-1.0, alpha_max=1.0, beta_max=2.0, eps=1e-6, normalize_q=True)
    d = {k: (None if v is None else v.to(DEV)) for k, v in raw.items()}
    gd = kda.chunk_backward_prologue(d["q"], d["k"], d["v"], d["gate"], d["beta_logit"],
                                     dO.to(DEV), d["S0"], dST.to(DEV), chunk=64, mode=w.mode, **pro)
    flat = lambda t: t.reshape(w.B * w.T, *t.shape[2:]).contiguous()
    cu = torch.arange(0, (w.B + 1) * w.T, w.T, dtype=torch.int32, device=DEV)
    gv = kda.chunk_backward_varlen_prologue(flat(d["q"]), flat(d["k"]), flat(d["v"]),
                                            flat(d["gate"]), flat(d["beta_logit"]), cu,
                                            flat(dO.to(DEV)), d["S0"], dST.to(DEV), chunk=64,
                                            mode=w.mode, **pro)
    torch.cuda.synchronize()
    for gn in ("dq", "dk", "dv", "d_gate", "d_beta_logit"):
        assert torch.equal(flat(gd[gn]), gv[gn]), gn
    assert torch.equal(gd["d_initial_state"], gv["d_initial_state"])
