"""KDA_FLAG_VALIDATE_RANGES through the C ABI: in-range inputs give results
bitwise equal to an unchecked call; one element outside the mode's ranges
(KDA: alpha in [0,1], beta in [0,1]; CKDA: alpha in [-1,1], beta in [0,2];
NaN anywhere; the phase variant's theta finite) gives status KDA_ERR_RANGE
with the outputs untouched; under graph capture the flag is refused before
anything is enqueued."""
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import workloads
from parity import say

pytestmark = pytest.mark.gpu
RANGE, UNSUP = 8, 3
NAN = float("nan")

# (name, mode, tensor, index, value, rejected)
CASES = [
    ("kda_alpha_zero", kda.KDA, "alpha", (0, 5, 1, 3), 0.0, False),
    ("kda_alpha_below_zero", kda.KDA, "alpha", (0, 5, 1, 3), -1e-30, True),
    ("kda_alpha_one", kda.KDA, "alpha", (0, 6, 0, 3), 1.0, False),
    ("kda_alpha_above_one", kda.KDA, "alpha", (0, 6, 0, 3), 1.0000001, True),
    ("kda_alpha_negative", kda.KDA, "alpha", (0, 77, 0, 0), -0.5, True),
    ("ckda_alpha_negative", kda.CKDA, "alpha", (0, 77, 0, 0), -0.5, False),
    ("ckda_alpha_minus_one", kda.CKDA, "alpha", (0, 1, 1, 9), -1.0, False),
    ("ckda_alpha_above_one", kda.CKDA, "alpha", (0, 199, 1, 127), 1.0001, True),
    ("kda_beta_above_one", kda.KDA, "beta", (0, 150, 1), 1.5, True),
    ("ckda_beta_above_one", kda.CKDA, "beta", (0, 150, 1), 1.5, False),
    ("ckda_beta_two", kda.CKDA, "beta", (0, 3, 0), 2.0, False),
    ("ckda_beta_above_two", kda.CKDA, "beta", (0, 3, 0), 2.01, True),
    ("ckda_beta_negative", kda.CKDA, "beta", (0, 0, 0), -1e-7, True),
    ("ckda_alpha_nan", kda.CKDA, "alpha", (0, 10, 0, 64), NAN, True),
    ("kda_beta_nan", kda.KDA, "beta", (0, 199, 1), NAN, True),
]


def _inputs(mode):
    w = workloads.workload(2, B=1, H=2, T=200, mode=mode)
    d = {k: (None if v is None else v.to("cuda")) for k, v in workloads.make_prefill(w).items()}
    return w, d


def _forward(w, d, flags):
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((w.B, w.T, w.H, w.Dv), 7.0, dtype=w.dtype, device="cuda")
    st = torch.full((w.B, w.H, w.Dk, w.Dv), 7.0, dtype=torch.float32, device="cuda")
    kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk=w.chunk,
                      mode=w.mode, out=out, final_state=st, workspace=ws, flags=flags)
    return out, st


@pytest.mark.parametrize("mode", [kda.KDA, kda.CKDA], ids=["kda", "ckda"])
def test_in_range_matches_unchecked(mode):
    w, d = _inputs(mode)
    say(f"[ranges] in range: {w}")
    o0, s0 = _forward(w, d, 0)
    o1, s1 = _forward(w, d, kda.VALIDATE_RANGES)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(s0, s1)


@pytest.mark.parametrize("name,mode,key,idx,val,bad", CASES, ids=[c[0] for c in CASES])
def test_forward_and_decode(name, mode, key, idx, val, bad):
    w, d = _inputs(mode)
    say(f"[ranges] {name}: {w}")
    d[key][idx] = val
    if bad:
        ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                         dtype=torch.uint8, device="cuda")
        out = torch.full((w.B, w.T, w.H, w.Dv), 7.0, dtype=w.dtype, device="cuda")
        with pytest.raises(kda.KdaError) as e:
            kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                              chunk=w.chunk, mode=mode, out=out, workspace=ws,
                              flags=kda.VALIDATE_RANGES)
        assert e.value.status == RANGE
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())                      # nothing was enqueued
        # packed-batch form: the same token range as two sequences
        cu = torch.tensor([0, 90, w.T], dtype=torch.int32, device="cuda")
        with pytest.raises(kda.KdaError) as e:
            kda.chunk_forward_varlen(d["q"][0], d["k"][0], d["v"][0], d["alpha"][0],
                                     d["beta"][0], cu, None, chunk=w.chunk, mode=mode,
                                     flags=kda.VALIDATE_RANGES)
        assert e.value.status == RANGE
    else:
        o0, s0 = _forward(w, d, 0)
        o1, s1 = _forward(w, d, kda.VALIDATE_RANGES)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(s0, s1)
    # decode on the token that holds the value
    t = idx[1]
    sl = lambda x: x[:, t].contiguous()
    S = torch.zeros((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")
    if bad:
        with pytest.raises(kda.KdaError) as e:
            kda.decode_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["alpha"]), sl(d["beta"]),
                            S, mode=mode, flags=kda.VALIDATE_RANGES)
        assert e.value.status == RANGE
        torch.cuda.synchronize()
        assert bool((S == 0).all())
    else:
        kda.decode_step(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["alpha"]), sl(d["beta"]), S,
                        mode=mode, flags=kda.VALIDATE_RANGES)
        torch.cuda.synchronize()


def test_refused_under_capture():
    w, d = _inputs(kda.CKDA)
    say(f"[ranges] capture: {w}")
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.dtype, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g):
        try:
            kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                              chunk=w.chunk, mode=w.mode, out=out, workspace=ws,
                              flags=kda.VALIDATE_RANGES)
        except kda.KdaError as e:
            status = e.status
    torch.cuda.synchronize()
    assert status == UNSUP


INF = float("inf")


@pytest.mark.parametrize("name,val,bad", [("theta_nan", NAN, True), ("theta_inf", INF, True),
                                          ("theta_minus_inf", -INF, True),
                                          ("theta_large_finite", 1.0e4, False)],
                         ids=["theta_nan", "theta_inf", "theta_minus_inf", "theta_large_finite"])
def test_phase_theta(name, val, bad):
    """The phase variant (chunked forward and decode step) checks every theta
    for finiteness: NaN or +-inf gives KDA_ERR_RANGE with nothing written; a
    large finite phase is in range."""
    w = workloads.workload(3, B=1, H=2, T=130, chunk=64, s0_std=0.1)
    say(f"[ranges] phase {name}: {w}")
    d = {k: (None if v is None else v.to("cuda"))
         for k, v in workloads.make_prefill_phase(w, theta_max=2.0).items()}
    d["theta"][0, 70, 1, 5] = val
    out = torch.full((w.B, w.T, w.H, w.Dv), 7.0, dtype=w.dtype, device="cuda")
    t = 70
    sl = lambda x: x[:, t].contiguous()
    S = torch.zeros((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")
    args = (sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["alpha"]), sl(d["theta"]), sl(d["beta"]), S)
    if bad:
        with pytest.raises(kda.KdaError) as e:
            kda.chunk_forward_phase(d["q"], d["k"], d["v"], d["alpha"], d["theta"], d["beta"],
                                    d["S0"], chunk=w.chunk, mode=w.mode, out=out,
                                    flags=kda.VALIDATE_RANGES)
        assert e.value.status == RANGE
        with pytest.raises(kda.KdaError) as e:
            kda.decode_step_phase(*args, mode=w.mode, flags=kda.VALIDATE_RANGES)
        assert e.value.status == RANGE
        torch.cuda.synchronize()
        assert bool((out == 7.0).all()) and bool((S == 0).all())
    else:
        kda.chunk_forward_phase(d["q"], d["k"], d["v"], d["alpha"], d["theta"], d["beta"],
                                d["S0"], chunk=w.chunk, mode=w.mode, out=out,
                                flags=kda.VALIDATE_RANGES)
        kda.decode_step_phase(*args, mode=w.mode, flags=kda.VALIDATE_RANGES)
        torch.cuda.synchronize()
