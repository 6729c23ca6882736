"""kda_chunk_forward_noalloc (the built-in scratch in place of a workspace)
against kda_chunk_forward on the same inputs, through the C ABI: two calls in
a row on one stream, the second smaller, each bit-identical to the entry point
it stands in for (same kernels, same order of operations) and within the
oracle's tolerance."""
import numpy as np
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import oracle
import workloads
from parity import TOL, np32, oracle_threads, say, slice_err_out, slice_err_state

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    # name, base workload, overrides  (bf16 d=128: 9.3 MB of workspace; then a
    # smaller fp32 call with a ragged tail and a non-zero initial state)
    ("bf16_ckda_d128_c64_B2_H4_T1000", 3, dict(B=2, H=4, T=1000, chunk=64)),
    ("f32_ckda_dk32_c32_T67_s0", 1, dict(B=1, H=3, T=67, D=32, chunk=32, s0_std=0.5)),
]


def _one(name, base, ov):
    w = workloads.workload(base, **ov)
    say(f"[noalloc] {name}: {w}")
    inp = workloads.make_prefill(w)
    d = {x: (None if t is None else t.to(DEV)) for x, t in inp.items()}
    n = kda.workspace_size(w.B, w.T, w.H, w.D, w.D, w.chunk, w.dtype)
    assert n <= kda.NOALLOC_SCRATCH_BYTES
    out_ref, st_ref = kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                                        chunk=w.chunk, mode=w.mode)
    out = torch.full_like(out_ref, float("nan"))
    st = torch.full_like(st_ref, float("nan"))
    kda.chunk_forward_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], out, st,
                              chunk=w.chunk, mode=w.mode)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(st, st_ref)
    o_ref, s_ref = oracle.forward(np32(inp["q"]), np32(inp["k"]), np32(inp["v"]),
                                  np32(inp["alpha"]), np32(inp["beta"]),
                                  None if inp["S0"] is None else np32(inp["S0"]),
                                  nthreads=oracle_threads())
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  bitwise equal to kda_chunk_forward; err out {eo:.3e} state {es:.3e}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


def test_noalloc_two_calls_then_smaller():
    for name, base, ov in CASES:
        _one(name, base, ov)


def test_noalloc_refuses_above_scratch():
    """A shape whose workspace exceeds the scratch is refused before any work."""
    w = workloads.workload(2, T=4096)
    say(f"[noalloc] refusal {w}")
    assert kda.workspace_size(w.B, w.T, w.H, w.D, w.D, w.chunk, w.dtype) > kda.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(1, dtype=w.dtype, device=DEV)
    q = torch.zeros((w.B, w.T, w.H, w.D), dtype=w.dtype, device=DEV)
    a = torch.zeros((w.B, w.T, w.H, w.D), dtype=torch.float32, device=DEV)
    b = torch.zeros((w.B, w.T, w.H), dtype=torch.float32, device=DEV)
    out = torch.zeros_like(q)
    with pytest.raises(kda.KdaError) as ei:
        kda.chunk_forward_noalloc(q, q, q, a, b, None, out, None, chunk=w.chunk, mode=w.mode)
    assert ei.value.status == 9
    del x
