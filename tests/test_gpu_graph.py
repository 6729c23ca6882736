"""HIP graph capture of the chunked forward (through the C ABI): a call
captured once from torch's capture stream and replayed several times, with
the program's own eager work and synchronisations between the replays; every
replay must equal the eager call bitwise.  Covers the single-pass launch
sequence, the parts path and the streamed path (prep grid and chain at the
same time), whose second stream (the caller's, lent to kda_chunk_forward_side)
the capture takes in through its events."""
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import workloads
from parity import say

pytestmark = pytest.mark.gpu

# (name, base workload, overrides, path: "single", "parts" or "streamed")
GRAPH_CASES = [
    ("bf16_kda_d128_c64_H4_T700", 2, dict(B=1, H=4, T=700), "single"),
    ("bf16_ckda_d128_c16_H9_T4133_parts", 3, dict(B=1, H=9, T=4133, chunk=16, s0_std=0.2),
     "parts"),
    ("bf16_ckda_d128_c64_H8_T1500_streamed", 3, dict(B=1, H=8, T=1500, s0_std=0.2), "streamed"),
]


@pytest.mark.parametrize("name,base,ov,path", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_forward_graph_replay(name, base, ov, path):
    w = workloads.workload(base, **ov)
    say(f"[graph] {name}: {w}")
    d = {k: (None if v is None else v.to("cuda")) for k, v in workloads.make_prefill(w).items()}
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, w.chunk, w.dtype),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.T, w.H, w.Dv), dtype=w.dtype, device="cuda")
    st = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")

    side = None if path == "single" else kda.SideStream()
    # (every call from a non-null stream, so that the streamed form is taken)
    main = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda.set_stream(main)

    sf = kda.STREAMED if path == "streamed" else 0

    def call(o, s, flags=0):
        kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], chunk=w.chunk,
                          mode=w.mode, out=o, final_state=s, workspace=ws, flags=flags | sf,
                          side=side)

    # eager reference
    call(out, st, kda.STAGE_EVENTS)
    torch.cuda.synchronize()
    names = [n for n, _ in kda.last_stage_times()]
    say(f"  stages {names}")
    assert names.count("chain") == (8 if path == "parts" else 1)
    assert names.count("chain_stream") == (1 if path == "streamed" else 0)
    ref_out, ref_st = out.clone(), st.clone()

    other = torch.cuda.Stream()
    other.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(other):
        call(out, st)
    torch.cuda.current_stream().wait_stream(other)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, st)
    torch.cuda.synchronize()

    o2 = torch.empty_like(out)
    s2 = torch.empty_like(st)
    for rep in range(3):
        out.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = torch.equal(out, ref_out) and torch.equal(st, ref_st)
        say(f"  replay {rep}: bitwise {ok}")
        assert ok
        call(o2, s2)                         # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_out) and torch.equal(s2, ref_st)
    torch.cuda.set_stream(torch.cuda.default_stream())
