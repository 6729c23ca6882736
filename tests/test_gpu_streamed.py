"""Streamed forward: kda_chunk_forward_side with KDA_FLAG_STREAMED at bf16,
chunk 64, Dk 128 or 64 and at least 8 (b, h) sequences, from a non-null
stream.  The prep grid on the
second stream (from kda_side_stream_create: a hardware queue of its own)
forms each chunk's factors and raises that chunk's ready word; the chain,
running on the caller's stream at the same time, waits for each word before
it loads the chunk.  A chunk that needs the exact kernel (ready word 2),
or a wait that runs past its bound, makes the chain give up; the call then
runs the exact kernel and a fallback chain after the prep grid has finished.

White-box: the last 384 bytes of the workspace are the control words of the
streamed call, as 32-bit words: prep counters [0:8], chain counters [32:40],
chains done [40], chains expected [41], column tiles per chain workgroup
[42], give-up word [64]; the tests read them to see which way the call went.
Before them lie the units' ready words, padded to 256 bytes (3 once a chain
workgroup took the unit: the prep grid keeps a bounded lead over that mark).

Checks: the oracle's recurrence across column-tile widths (Dv 128, 96, 48 at
Dk 128; 64, 48 at Dk 64), ragged tails, initial states, both modes and
batches; no give-up and every chain done on ordinary inputs; bitwise equality
with the single-stream call where both run the same chain arithmetic (at most
64 (b, h, 16-column) chains: the 16-column-tile chain); chunks flagged for the
exact kernel (the give-up path) still match the oracle; repeated calls lent
the same side stream; a call from the null stream (which takes the two-pass
form: a side stream from kda_side_stream_create is a blocking one)."""
import pytest
import torch

import gated_delta_rule_forward_amd as kda
import workloads
from parity import TOL, np32, say, slice_err_out, slice_err_state, elem_note
from test_gpu_parity import run_oracle, run_gpu, to_dev, _stage_names

pytestmark = pytest.mark.gpu

DEV = "cuda"
SF = kda.STREAMED


def _ctl(ws):
    """(gave up, chains done, chains expected) from the control words."""
    w = ws[-384:].cpu().view(torch.int32)
    return int(w[64]), int(w[40]), int(w[41])


def _tiles(ws):
    """Column tiles per chain workgroup the call chose."""
    return int(ws[-384:].cpu().view(torch.int32)[42])


def _ready(ws, nu):
    """The units' ready words (a 256-byte padded block just before the control
    words): 1 formed, 2 for the exact kernel, 3 formed and taken by a chain
    workgroup."""
    start = ws.numel() - 384 - ((4 * nu + 255) // 256) * 256
    return ws[start:start + 4 * nu].cpu().view(torch.int32)


def _prefill(base, dv, **ov):
    w = workloads.workload(base, **ov)
    inp = workloads.make_prefill(w)
    if dv != w.D:
        inp["v"] = inp["v"][..., :dv].contiguous()
        if inp["S0"] is not None:
            inp["S0"] = inp["S0"][..., :dv].contiguous()
    return w, inp


# (name, base workload, Dv, overrides, column tiles per chain workgroup)
STREAMED = [
    ("kda_d128_dv128_B1_H8_T1000", 2, 128, dict(B=1, H=8, T=1000), 1),
    ("ckda_d128_dv128_B2_H4_T777_s0", 3, 128, dict(B=2, H=4, T=777, s0_std=0.3), 1),
    ("ckda_d128_dv96_B1_H9_T300_s0", 3, 96, dict(B=1, H=9, T=300, s0_std=0.2), 1),
    ("kda_d128_dv48_B3_H3_T129", 2, 48, dict(B=3, H=3, T=129), 1),
    ("ckda_d64_dv64_B1_H12_T513_s0", 3, 64, dict(B=1, H=12, T=513, D=64, s0_std=0.3), 1),
    ("kda_d64_dv48_B2_H5_T64", 2, 48, dict(B=2, H=5, T=64, D=64), 1),
    ("kda_d128_dv128_B1_H24_T200", 2, 128, dict(B=1, H=24, T=200), 2),
    # 160 chains at Dk 64: more than 128 workgroups at one tile
    ("ckda_d64_dv64_B1_H40_T130_s0", 3, 64, dict(B=1, H=40, T=130, D=64, s0_std=0.3), 2),
    # 288 chains at Dk 128: more than 128 workgroups at two tiles
    ("kda_d128_dv128_B3_H12_T100", 2, 128, dict(B=3, H=12, T=100), 4),
]


@pytest.mark.parametrize("name,base,dv,ov,tiles", STREAMED, ids=[c[0] for c in STREAMED])
def test_streamed_forward(name, base, dv, ov, tiles):
    w, inp = _prefill(base, dv, **ov)
    say(f"[streamed] {name}: {w} Dv={dv}")
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.D, dv, 64, w.dtype), dtype=torch.uint8,
                     device=DEV)
    side = kda.SideStream()
    cs_ = torch.cuda.Stream()
    out, st = run_gpu(d, 64, w.mode, workspace=ws, side=side, flags=SF | kda.STAGE_EVENTS,
                      stream=cs_)
    names = _stage_names()
    gave_up, done, expect = _ctl(ws)
    say(f"  stages {names}; gave up {gave_up}, chains {done}/{expect}, tiles {_tiles(ws)}")
    assert names == ["stream_clear", "chain_stream", "prep_stream", "prep_exact", "chain"]
    assert gave_up == 0 and done == expect > 0
    assert _tiles(ws) == tiles
    # every unit was taken by the chain (the mark the prep's lead limit reads)
    assert bool((_ready(ws, w.B * w.H * -(-w.T // 64)) == 3).all())
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
    # the single-stream call (the 16-column chain here, or the wide one at most
    # 64 chains: the same products in the same order)
    out1, st1 = run_gpu(d, 64, w.mode, flags=kda.STAGE_EVENTS, stream=cs_)
    assert "chain_stream" not in _stage_names()
    if w.B * w.H * (dv // 16) <= 64:
        assert torch.equal(out, out1) and torch.equal(st, st1)
    # repeated calls lent the same side stream, back to back
    outs = [run_gpu(d, 64, w.mode, workspace=ws, side=side, stream=cs_, flags=SF) for _ in range(2)]
    for o2, s2 in outs:
        assert torch.equal(o2, out) and torch.equal(s2, st)
    assert _ctl(ws)[0] == 0
    # from the null stream: the two-pass form, same results as the call on one stream
    o3, s3 = run_gpu(d, 64, w.mode, workspace=ws, side=side, flags=SF | kda.STAGE_EVENTS)
    assert "chain_stream" not in _stage_names()
    assert torch.equal(o3, out1) and torch.equal(s3, st1)


def test_streamed_flagged_chunks_give_up():
    """Chunks the fast prep cannot factor (ready word 2): the chain gives up,
    the exact kernel forms those chunks and the fallback chain recomputes every
    sequence; the result matches the oracle."""
    w = workloads.workload(3, B=1, H=8, T=300, s0_std=0.2)
    inp = workloads.make_prefill(w)
    a = inp["alpha"]
    a[0, 70:80, 5, :5] = 1e-12          # head 5, chunk 1: ~40 bits per token
    a[0, 150:190, 6, 3] = 2.0 ** -30    # head 6, chunk 2
    say(f"[streamed give-up] {w}")
    o_ref, s_ref = run_oracle(inp)
    d = to_dev(inp)
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.D, w.D, 64, w.dtype), dtype=torch.uint8,
                     device=DEV)
    out, st = run_gpu(d, 64, w.mode, workspace=ws, side=kda.SideStream(),
                      stream=torch.cuda.Stream(), flags=SF)
    gave_up, done, expect = _ctl(ws)
    say(f"  gave up {gave_up}, chains {done}/{expect}")
    assert gave_up == 1
    assert int((_ready(ws, w.B * w.H * -(-w.T // 64)) == 2).sum()) == 2   # the two flagged units
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
    out1, st1 = run_gpu(d, 64, w.mode)
    assert torch.equal(out, out1) and torch.equal(st, st1)


def test_streamed_give_up_past_the_lead_limit():
    """A give-up early in a sequence longer than the prep's lead limit
    (H=32, T=2048: 32 chunks, a limit of 28): the prep units past the limit
    stop waiting for marks that no longer come, and the result is bitwise the
    single-stream call's."""
    w = workloads.workload(2, B=1, H=32, T=2048)
    inp = workloads.make_prefill(w)
    inp["alpha"][0, 150:160, 3, :4] = 1e-30      # head 3, chunk 2: flagged for the exact kernel
    say(f"[streamed give-up, long] {w}")
    d = to_dev(inp)
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.D, w.D, 64, w.dtype), dtype=torch.uint8,
                     device=DEV)
    out, st = run_gpu(d, 64, w.mode, workspace=ws, side=kda.SideStream(),
                      stream=torch.cuda.Stream(), flags=SF)
    gave_up, done, expect = _ctl(ws)
    say(f"  gave up {gave_up}, chains {done}/{expect}")
    assert gave_up == 1
    out1, st1 = run_gpu(d, 64, w.mode)
    assert torch.equal(out, out1) and torch.equal(st, st1)


def test_streamed_not_taken():
    """Forms outside the streamed path keep their launch sequence with a side
    stream: fewer than 8 sequences, too many chains, the final state written
    over the initial one, KDA_FLAG_SINGLE_STREAM, no KDA_FLAG_STREAMED (all
    from a non-null stream; chunk-start states have no side-stream entry
    point)."""
    w = workloads.workload(2, B=1, H=8, T=200)
    d = to_dev(workloads.make_prefill(w))
    side = kda.SideStream()
    main = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda.set_stream(main)
    run_gpu(d, 64, w.mode, side=side, flags=SF | kda.STAGE_EVENTS | kda.SINGLE_STREAM)
    assert "chain_stream" not in _stage_names()
    run_gpu(d, 64, w.mode, side=side, flags=kda.STAGE_EVENTS)          # (without the flag)
    assert "chain_stream" not in _stage_names()
    w7 = workloads.workload(2, B=1, H=7, T=200)
    d7 = to_dev(workloads.make_prefill(w7))
    run_gpu(d7, 64, w7.mode, side=side, flags=SF | kda.STAGE_EVENTS)
    assert "chain_stream" not in _stage_names()
    # 1024 (b, h, 16-column) chains: even 4 column tiles per workgroup would
    # take every compute unit
    wb = workloads.workload(2, B=4, H=32, T=64)
    db = to_dev(workloads.make_prefill(wb))
    run_gpu(db, 64, wb.mode, side=side, flags=SF | kda.STAGE_EVENTS)
    assert "chain_stream" not in _stage_names()
    S = torch.zeros((w.B, w.H, w.D, w.D), device=DEV)
    kda.chunk_forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, chunk=64, mode=w.mode,
                      final_state=S, side=side, flags=SF | kda.STAGE_EVENTS)
    torch.cuda.synchronize()
    assert "chain_stream" not in _stage_names()
    # (and the streamed form is what this stream takes for the plain call)
    run_gpu(d, 64, w.mode, side=side, flags=SF | kda.STAGE_EVENTS)
    assert "chain_stream" in _stage_names()
    torch.cuda.set_stream(torch.cuda.default_stream())


def test_streamed_kda_bf16_prefill_full():
    """KDA bf16 prefill, B=1 H=32 T=8192 d=128 chunk=64 through the streamed
    call (the form the benchmark reports beside the two-pass headline), every
    head against the oracle."""
    w = workloads.workload(2)
    say(f"[streamed] kda_bf16_prefill full {w}")
    inp = workloads.make_prefill(w, device=DEV)
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.D, w.D, 64, w.dtype), dtype=torch.uint8,
                     device=DEV)
    out, st = run_gpu(inp, w.chunk, w.mode, workspace=ws, side=kda.SideStream(),
                      stream=torch.cuda.Stream(), flags=SF)
    gave_up, done, expect = _ctl(ws)
    say(f"  gave up {gave_up}, chains {done}/{expect}")
    assert gave_up == 0 and done == expect
    o_ref, s_ref = run_oracle(inp)
    eo, es = slice_err_out(np32(out), o_ref), slice_err_state(np32(st), s_ref)
    say(f"  err out {eo:.3e} state {es:.3e}{elem_note()}")
    assert eo <= 2e-2 and es <= 2e-2
