"""Seeded random sweep over the supported shapes: the chunked forward and the
backward through the C ABI against the oracle (per-slice normwise errors
within the dtype's tolerance).  Shapes (batch, heads, ragged lengths, Dk and
Dv apart, chunk, dtype, mode, with or without S0) are drawn from a fixed seed
and kept small enough for the oracle to finish in seconds.  Inputs follow the
workload recipe of workloads.py."""
import random

import numpy as np
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import oracle
import workloads
from parity import TOL, np32, oracle_threads, say, slice_err_out, slice_err_state, elem_note

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _draw(n, seed, backward):
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        dt = rng.choice(["f32", "bf16"])
        dks = ([32, 64] if dt == "f32" else [32, 64, 128]) if backward else \
              ([16, 32, 64] if dt == "f32" else [16, 32, 64, 128])
        Dk = rng.choice(dks)
        Dv = rng.choice([16, 32, 48, 64] if dt == "f32" else [16, 32, 48, 64, 80, 96, 112, 128])
        chunk = rng.choice([32, 64] if backward else [16, 32, 64])
        T = rng.randint(1, 300)
        B, H = rng.randint(1, 2), rng.randint(1, 3)
        mode = rng.choice([workloads.KDA, workloads.CKDA])
        s0 = rng.random() < 0.5
        name = f"{'bwd' if backward else 'fwd'}{i}_{dt}_{'ckda' if mode else 'kda'}_B{B}H{H}T{T}_dk{Dk}dv{Dv}_c{chunk}{'_s0' if s0 else ''}"
        cases.append((name, dt, B, H, T, Dk, Dv, chunk, mode, s0, 1000 + i))
    return cases


FWD = _draw(16, 20261203, backward=False)
BWD = _draw(8, 20261204, backward=True)


def _inputs(dt, B, H, T, Dk, Dv, mode, s0, seed):
    g = torch.Generator().manual_seed(seed)
    dtype = DT[dt]
    q = workloads._unit_rows((B, T, H, Dk), g, "cpu", dtype)
    k = workloads._unit_rows((B, T, H, Dk), g, "cpu", dtype)
    v = torch.randn((B, T, H, Dv), generator=g).to(dtype)
    alpha = workloads._gates((B, T, H, Dk), mode, g, "cpu")
    beta = workloads._betas((B, T, H), mode, g, "cpu")
    S0 = (0.3 * torch.randn((B, H, Dk, Dv), generator=g)).contiguous() if s0 else None
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(), "alpha": alpha,
            "beta": beta, "S0": S0}


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


@pytest.mark.parametrize("name,dt,B,H,T,Dk,Dv,chunk,mode,s0,seed", FWD, ids=[c[0] for c in FWD])
def test_forward_random_shape(name, dt, B, H, T, Dk, Dv, chunk, mode, s0, seed):
    say(f"[random forward] {name}")
    inp = _inputs(dt, B, H, T, Dk, Dv, mode, s0, seed)
    o_ref, s_ref = oracle.forward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
                                  np32(inp["alpha"]), np32(inp["beta"]),
                                  None if inp["S0"] is None else np32(inp["S0"]),
                                  nthreads=oracle_threads())
    d = _dev(inp)
    out, st = kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                chunk=chunk, mode=mode)
    torch.cuda.synchronize()
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[DT[dt]] and es <= TOL[DT[dt]]


@pytest.mark.parametrize("name,dt,B,H,T,Dk,Dv,chunk,mode,s0,seed", BWD, ids=[c[0] for c in BWD])
def test_backward_random_shape(name, dt, B, H, T, Dk, Dv, chunk, mode, s0, seed):
    say(f"[random backward] {name}")
    inp = _inputs(dt, B, H, T, Dk, Dv, mode, s0, seed)
    g = torch.Generator().manual_seed(seed + 7)
    dO = torch.randn((B, T, H, Dv), generator=g).to(DT[dt])
    dST = torch.randn((B, H, Dk, Dv), generator=g)
    ref = oracle.backward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]), np32(inp["alpha"]),
                          np32(inp["beta"]), np32(dO),
                          None if inp["S0"] is None else np32(inp["S0"]), np32(dST),
                          nthreads=oracle_threads())
    d = _dev(inp)
    gr = kda.chunk_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(DEV), d["S0"],
                            dST.to(DEV), chunk=chunk, mode=mode)
    torch.cuda.synchronize()
    errs = {}
    for gn, rn in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("d_alpha", "dalpha"),
                   ("d_beta", "dbeta")):
        a, b = np32(gr[gn]), ref[rn]
        if a.ndim == 3:
            a, b = a[..., None], b[..., None]
        errs[gn] = slice_err_out(a, b)
    errs["d_initial_state"] = slice_err_state(np32(gr["d_initial_state"]), ref["dS0"])
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[DT[dt]], (k_, v_)
