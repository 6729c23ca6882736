"""The training-step split of the backward: kda_chunk_forward_save (the
forward that keeps what the gradient pass needs) and kda_chunk_backward_saved
(the gradients from that workspace), through the C ABI.

Checks: the saved forward's outputs against the oracle's recurrence at the
dtype tolerance; the gradients bit for bit equal to kda_chunk_backward's (the
same kernels on the same data), which the backward tests hold against the
oracle's gradients; T = 0; and the headline shape (B=1, H=32, T=8192, d=128)
on the same terms.  Each case prints its name before touching the GPU."""
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import workloads
from parity import TOL, np32, say, slice_err_out, slice_err_state
from test_gpu_parity import run_oracle, to_dev

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (name, base workload, overrides, with S0, with dST)
CASES = [
    ("f32_kda_d64_c64_T200", 0, dict(B=1, H=2, T=200, D=64, chunk=64), True, True),
    ("f32_ckda_d32_c32_T77", 1, dict(B=1, H=3, T=77, D=32, chunk=32), True, False),
    ("bf16_kda_d128_c64_T300", 2, dict(B=1, H=2, T=300, chunk=64), True, True),
    ("bf16_ckda_d128_c64_T257", 3, dict(B=2, H=3, T=257, chunk=64), False, True),
    ("bf16_ckda_d64_c32_T100", 3, dict(B=1, H=2, T=100, D=64, chunk=32), True, False),
]


def _inputs(base, ov, s0, dst):
    w = workloads.workload(base, **ov)
    if s0 and w.s0_std is None:
        w = workloads.workload(base, **ov, s0_std=0.5)
    if not s0:
        w = workloads.workload(base, **{**ov, "s0_std": None})
    inp = workloads.make_prefill(w)
    dO, dST = workloads.make_backward_seeds(w, dst=dst)
    return w, inp, dO, dST


def _run(w, d, dO, dST):
    out, st, saved = kda.chunk_forward_save(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                            chunk=w.chunk, mode=w.mode)
    g = kda.chunk_backward_saved(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO, saved, dST,
                                 chunk=w.chunk, mode=w.mode)
    ref = kda.chunk_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO, d["S0"], dST,
                             chunk=w.chunk, mode=w.mode)
    torch.cuda.synchronize()
    return out, st, g, ref


def _same(g, ref):
    for name in ("dq", "dk", "dv", "d_alpha", "d_beta", "d_initial_state"):
        assert torch.equal(g[name], ref[name]), name


@pytest.mark.parametrize("name,base,ov,s0,dst", CASES, ids=[c[0] for c in CASES])
def test_saved_backward(name, base, ov, s0, dst):
    w, inp, dO, dST = _inputs(base, ov, s0, dst)
    say(f"[saved] {name}: {w} S0={s0} dST={dst}")
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    out, st, g, ref = _run(w, d, dO.to(DEV), None if dST is None else dST.to(DEV))
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  forward err out {eo:.3e} state {es:.3e}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
    _same(g, ref)


def test_saved_empty():
    """T = 0: the final state is the initial one; dS0 = dST."""
    say("[saved] T=0")
    w = workloads.workload(2, B=2, H=3, T=0, s0_std=0.5)
    inp = to_dev(workloads.make_prefill(w))
    dST = torch.randn((w.B, w.H, w.D, w.D), device=DEV)
    dO = torch.empty((w.B, 0, w.H, w.D), dtype=w.dtype, device=DEV)
    out, st, saved = kda.chunk_forward_save(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                            inp["S0"], chunk=64, mode=w.mode)
    g = kda.chunk_backward_saved(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], dO, saved,
                                 dST, chunk=64, mode=w.mode)
    torch.cuda.synchronize()
    assert torch.equal(st, inp["S0"]) and torch.equal(g["d_initial_state"], dST)


def test_saved_kda_bf16_prefill():
    """The headline shape: the saved forward's output and state against the
    oracle on every head, the gradients bitwise those of kda_chunk_backward."""
    w = workloads.workload(2)
    say(f"[saved] kda_bf16_prefill {w}")
    inp = workloads.make_prefill(w, device=DEV)
    dO, dST = workloads.make_backward_seeds(w, device=DEV)
    out, st, g, ref = _run(w, inp, dO, dST)
    _same(g, ref)
    del g, ref
    o_ref, s_ref = run_oracle(inp)
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  forward err out {eo:.3e} state {es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2
