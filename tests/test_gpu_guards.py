"""Guard regions: every output (and the workspace, at exactly its queried size)
is a view into the middle of a larger buffer whose bytes outside the view are
a sentinel; after each call through the C ABI every sentinel byte must be
unchanged.  Covers the chunked forward with both workspace store variants
(ordinary stores below 128 (b, h, 16-column) chains, non-temporal ones from
128), the chunk-start states, packed batches (rows past cu[N] untouched), the
parts path on a side stream, the allocation-free forward, decode and the
backward, and the streamed path.  The results themselves are checked elsewhere; here they are only
required to be finite where written."""
import math

import pytest
import torch

import gated_delta_rule_forward_amd as kda
import workloads
from parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENT = 0xA5
MARGIN = 4096          # bytes of sentinel on each side


class Guarded:
    """A tensor view of `shape` inside a sentinel-filled buffer."""

    def __init__(self, shape, dtype, init=None):
        self.esz = torch.empty((), dtype=dtype).element_size()
        self.n = math.prod(shape)
        self.m = MARGIN // self.esz
        self.buf = torch.empty(self.n + 2 * self.m, dtype=dtype, device=DEV)
        self.buf.view(torch.uint8).fill_(SENT)
        self.t = self.buf[self.m:self.m + self.n].view(shape)
        if init is not None:
            self.t.copy_(init)

    def intact(self):
        b = self.buf.view(torch.uint8)
        head, tail = b[:self.m * self.esz], b[(self.m + self.n) * self.esz:]
        return bool((head == SENT).all()) and bool((tail == SENT).all())


def _check(name, guards):
    torch.cuda.synchronize()
    bad = [k for k, g in guards.items() if not g.intact()]
    say(f"  {name}: guards {'intact' if not bad else 'BROKEN: ' + ', '.join(bad)}")
    assert not bad


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


# (name, base workload, overrides): 16 chains (ordinary workspace stores) and
# 128 chains (non-temporal whole-fragment stores), ragged tails, both dtypes
FORWARD = [
    ("bf16_ckda_H2_T199_c64", 3, dict(B=1, H=2, T=199, chunk=64)),
    ("bf16_kda_H16_T130_c64_nt", 2, dict(B=1, H=16, T=130, chunk=64)),
    ("f32_ckda_d64_B2_T77_c32", 1, dict(B=2, H=2, T=77, D=64, chunk=32)),
    ("bf16_ckda_d32_H4_T50_c16", 3, dict(B=1, H=4, T=50, D=32, chunk=16)),
]


@pytest.mark.parametrize("name,base,ov", FORWARD, ids=[c[0] for c in FORWARD])
def test_forward_guards(name, base, ov):
    w = workloads.workload(base, **ov)
    say(f"[guards forward] {name}: {w}")
    d = _dev(workloads.make_prefill(w))
    nws = kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype)
    g = {"out": Guarded((w.B, w.T, w.H, w.Dv), w.dtype),
         "final_state": Guarded((w.B, w.H, w.Dk, w.Dv), torch.float32),
         "workspace": Guarded((nws,), torch.uint8)}
    kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk=w.chunk,
                      mode=w.mode, out=g["out"].t, final_state=g["final_state"].t,
                      workspace=g["workspace"].t)
    _check("chunk_forward", g)
    assert bool(torch.isfinite(g["out"].t.float()).all())
    # with the chunk-start states
    nc = (w.T + w.chunk - 1) // w.chunk
    g["chunk_states"] = Guarded((w.B, w.H, nc, w.Dk, w.Dv), w.dtype)
    kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk=w.chunk,
                      mode=w.mode, out=g["out"].t, final_state=g["final_state"].t,
                      workspace=g["workspace"].t, chunk_states=g["chunk_states"].t)
    _check("chunk_forward_states", g)


def test_forward_parts_and_noalloc_guards():
    """The parts path (side stream; the state between parts lives at the end of
    the workspace) and the allocation-free entry point."""
    w = workloads.workload(3, B=1, H=2, T=4133, chunk=16, s0_std=0.2)
    say(f"[guards parts] {w}")
    d = _dev(workloads.make_prefill(w))
    nws = kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype)
    g = {"out": Guarded((w.B, w.T, w.H, w.Dv), w.dtype),
         "final_state": Guarded((w.B, w.H, w.Dk, w.Dv), torch.float32),
         "workspace": Guarded((nws,), torch.uint8)}
    kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk=w.chunk,
                      mode=w.mode, out=g["out"].t, final_state=g["final_state"].t,
                      workspace=g["workspace"].t, side=kda.SideStream(),
                      flags=kda.STAGE_EVENTS | kda.NO_SEGMENTS)
    torch.cuda.synchronize()
    assert [n for n, _ in kda.last_stage_times()].count("chain") == 8
    _check("chunk_forward_side (parts)", g)
    # the streamed path: ready words and control words at the workspace's end
    w3 = workloads.workload(2, B=1, H=9, T=333)
    d3 = _dev(workloads.make_prefill(w3))
    nws3 = kda.workspace_size(w3.B, w3.T, w3.H, w3.Dk, w3.Dv, w3.chunk, w3.dtype)
    g3 = {"out": Guarded((w3.B, w3.T, w3.H, w3.Dv), w3.dtype),
          "final_state": Guarded((w3.B, w3.H, w3.Dk, w3.Dv), torch.float32),
          "workspace": Guarded((nws3,), torch.uint8)}
    torch.cuda.synchronize()
    kda.chunk_forward(d3["q"], d3["k"], d3["v"], d3["alpha"], d3["beta"], d3["S0"],
                      chunk=w3.chunk, mode=w3.mode, out=g3["out"].t,
                      final_state=g3["final_state"].t, workspace=g3["workspace"].t,
                      side=kda.SideStream(), flags=kda.STAGE_EVENTS | kda.STREAMED,
                      stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert "chain_stream" in [n for n, _ in kda.last_stage_times()]
    _check("chunk_forward_side (streamed)", g3)
    w2 = workloads.workload(3, B=1, H=4, T=300, chunk=64)
    d2 = _dev(workloads.make_prefill(w2))
    g2 = {"out": Guarded((w2.B, w2.T, w2.H, w2.Dv), w2.dtype),
          "final_state": Guarded((w2.B, w2.H, w2.Dk, w2.Dv), torch.float32)}
    kda.chunk_forward_noalloc(d2["q"], d2["k"], d2["v"], d2["alpha"], d2["beta"], d2["S0"],
                              g2["out"].t, g2["final_state"].t, chunk=w2.chunk, mode=w2.mode)
    _check("chunk_forward_noalloc", g2)


def test_varlen_guards():
    """Packed batch whose inputs hold more rows than cu[N]: rows past cu[N] of
    the output keep their sentinel, like the bytes around every buffer."""
    w = workloads.workload(3, H=2, chunk=64, s0_std=0.3)
    lengths = [70, 0, 129, 1]
    used = sum(lengths)
    rows = used + 37
    inp = workloads.make_varlen(w, lengths + [37])        # 37 extra rows past cu[N]
    d = _dev(inp)
    cu = d["cu_seqlens"][:len(lengths) + 1].contiguous()
    N = len(lengths)
    S0 = d["S0"][:N].contiguous()
    g = {"out": Guarded((rows, w.H, w.Dv), w.dtype),
         "final_state": Guarded((N, w.H, w.Dk, w.Dv), torch.float32)}
    say(f"[guards varlen] lengths {lengths} (+37 rows past cu[N])")
    kda.chunk_forward_varlen(d["q"][0], d["k"][0], d["v"][0], d["alpha"][0], d["beta"][0], cu,
                             S0, chunk=w.chunk, mode=w.mode, out=g["out"].t,
                             final_state=g["final_state"].t)
    _check("chunk_forward_varlen", g)
    tail = g["out"].t[used:].contiguous().view(torch.uint8)
    assert bool((tail == SENT).all()), "rows past cu[N] were written"


@pytest.mark.parametrize("dt,Dk,Dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 48)])
def test_decode_guards(dt, Dk, Dv):
    w = workloads.workload(4, B=3, H=2, D=Dk, dtype=dt, steps=3)
    inp = workloads.make_decode(w)
    say(f"[guards decode] {dt} Dk={Dk} Dv={Dv}")
    S = Guarded((w.B, w.H, Dk, Dv), torch.float32, init=inp["S0"][..., :Dv].to(DEV))
    out = Guarded((w.B, w.H, Dv), dt)
    for s in range(w.steps):
        v = inp["v"][s][..., :Dv].contiguous().to(DEV)
        kda.decode_step(inp["q"][s].to(DEV), inp["k"][s].to(DEV), v, inp["alpha"][s].to(DEV),
                        inp["beta"][s].to(DEV), S.t, out=out.t)
    _check("decode_step", {"state": S, "out": out})


@pytest.mark.parametrize("name,base,ov", [
    ("bf16_ckda_d128_c64_T150", 3, dict(B=1, H=2, T=150, chunk=64)),
    ("f32_kda_d32_c32_B2_T70", 0, dict(B=2, H=3, T=70, D=32, chunk=32, s0_std=0.3)),
], ids=["bf16_ckda_d128_c64_T150", "f32_kda_d32_c32_B2_T70"])
def test_backward_guards(name, base, ov):
    w = workloads.workload(base, **ov)
    say(f"[guards backward] {name}: {w}")
    d = _dev(workloads.make_prefill(w))
    dO, dST = workloads.make_backward_seeds(w)
    nws = kda.backward_workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype)
    g = {"dq": Guarded((w.B, w.T, w.H, w.Dk), w.dtype),
         "dk": Guarded((w.B, w.T, w.H, w.Dk), w.dtype),
         "dv": Guarded((w.B, w.T, w.H, w.Dv), w.dtype),
         "d_alpha": Guarded((w.B, w.T, w.H, w.Dk), torch.float32),
         "d_beta": Guarded((w.B, w.T, w.H), torch.float32),
         "d_initial_state": Guarded((w.B, w.H, w.Dk, w.Dv), torch.float32),
         "workspace": Guarded((nws,), torch.uint8)}
    kda.chunk_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], dO.to(DEV), d["S0"],
                       dST.to(DEV), chunk=w.chunk, mode=w.mode,
                       grads={k: g[k].t for k in ("dq", "dk", "dv", "d_alpha", "d_beta",
                                                  "d_initial_state")},
                       workspace=g["workspace"].t)
    _check("chunk_backward", g)
