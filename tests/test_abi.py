"""C-ABI contract tests that need no GPU.

The library must load, export every entry point include/kda.h declares, and
reject bad arguments with the documented status code *before* any HIP call
(so these calls use fake, never-dereferenced device addresses).
"""
import ctypes
import os
import re

import pytest

import gated_delta_rule_forward_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULLP, SHAPE, UNSUP, MISAL, WS, ALIAS = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert {"kda_chunk_forward", "kda_chunk_forward_states", "kda_chunk_forward_prologue",
            "kda_chunk_forward_phase", "kda_decode_step_phase", "kda_chunk_forward_varlen", "kda_decode_step",
            "kda_decode_step_prologue", "kda_chunk_forward_workspace_size",
            "kda_chunk_backward", "kda_chunk_backward_workspace_size",
            "kda_chunk_backward_prologue", "kda_chunk_backward_prologue_workspace_size",
            "kda_chunk_backward_varlen", "kda_chunk_backward_varlen_workspace_size",
            "kda_chunk_backward_varlen_prologue", "kda_chunk_backward_varlen_prologue_workspace_size",
            "kda_gate_prep", "kda_status_string", "kda_abi_version",
            "kda_chunk_forward_noalloc", "kda_chunk_forward_side", "kda_side_stream_create",
            "kda_side_stream_destroy"} <= set(syms)
    for s in syms:
        assert hasattr(lib, s), s


def test_side_stream_helpers_refuse_null(lib):
    null = ctypes.POINTER(kda._Side)()
    assert lib.kda_side_stream_create(null) == NULLP
    assert lib.kda_side_stream_destroy(null) == NULLP


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 18
    for s in range(10):
        assert lib.kda_status_string(s) != b"unknown status"
    assert lib.kda_status_string(99) == b"unknown status"


def ws_size(lib, B, T, H, Dk, Dv, C, dt):
    n = ctypes.c_size_t(123)
    st = lib.kda_chunk_forward_workspace_size(B, T, H, Dk, Dv, C, dt, ctypes.byref(n))
    return st, n.value


def test_workspace_size(lib):
    st, n = ws_size(lib, 1, 8192, 32, 128, 128, 64, BF16)
    assert st == OK
    nu = 32 * 128
    # W, Kt, QG, U, P bf16 + chunk decay fp32 + one flag byte, per chunk; then
    # (streamed forward) one ready word per chunk and a 384-byte control block
    assert n == nu * (3 * 64 * 128 * 2 + 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4 + 1) \
        + nu * 4 + 384
    # below 8 (b, h) there is no streamed form: the per-chunk regions only
    st, n = ws_size(lib, 1, 4096, 4, 128, 128, 64, BF16)
    assert n == 4 * 64 * (3 * 64 * 128 * 2 + 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4 + 1)
    assert ws_size(lib, 1, 0, 1, 16, 16, 16, F32) == (OK, 0)
    assert ws_size(lib, 1, 10, 1, 24, 16, 16, F32)[0] == UNSUP          # Dk not supported
    assert ws_size(lib, 1, 10, 1, 16, 24, 16, F32)[0] == UNSUP          # Dv not a multiple of 16
    assert ws_size(lib, 1, 10, 1, 16, 16, 48, F32)[0] == UNSUP          # chunk
    assert ws_size(lib, 1, 10, 1, 128, 16, 16, F32)[0] == UNSUP         # fp32 Dk 128: chunk 64 only
    assert ws_size(lib, 1, 10, 1, 128, 16, 32, F32)[0] == UNSUP
    assert ws_size(lib, 1, 10, 1, 128, 128, 64, F32)[0] == OK
    assert ws_size(lib, 1, 10, 1, 64, 128, 16, F32)[0] == OK           # fp32 Dv 128, any chunk
    assert ws_size(lib, 0, 10, 1, 16, 16, 16, F32)[0] == SHAPE
    assert ws_size(lib, 1, -1, 1, 16, 16, 16, F32)[0] == SHAPE
    assert ws_size(lib, 1, 10, 1, 16, 16, 16, 7)[0] == UNSUP
    assert lib.kda_chunk_forward_workspace_size(1, 1, 1, 16, 16, 16, F32, None) == NULLP


class Fake:
    """Distinct, 16-byte aligned, never-dereferenced addresses."""
    def __init__(self):
        self.next = 0x7f0000000000

    def __call__(self, nbytes=1 << 20):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return ctypes.c_void_p(p)


def fwd(lib, **kw):
    f = Fake()
    B, T, H, Dk, Dv, C = kw.get("B", 1), kw.get("T", 64), kw.get("H", 2), kw.get("Dk", 16), \
        kw.get("Dv", 16), kw.get("C", 16)
    dt = kw.get("dt", F32)
    st, need = ws_size(lib, max(B, 1), max(T, 0), max(H, 1), Dk, Dv, C, dt)
    args = dict(q=f(), k=f(), v=f(), alpha=f(), beta=f(), s0=None, out=f(), st=None,
                ws=f(max(need, 1) + 4096), wsb=need)
    args.update({k_: v_ for k_, v_ in kw.items() if k_ in args})
    return lib.kda_chunk_forward(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                                 args["s0"], args["out"], args["st"], B, T, H, Dk, Dv, C, dt,
                                 kw.get("mode", 1), kw.get("flags", 0), args["ws"], args["wsb"],
                                 None)


def test_workspace_includes_segments(lib):
    """Few chains and many chunks: the workspace also holds the segment maps
    and start states (here 4 segments of Dk x (Dk + Dv) and Dk x Dv fp32)."""
    st, n = ws_size(lib, 1, 2500, 1, 32, 32, 16, F32)
    assert st == OK
    nu = 157
    per_unit = 3 * 16 * 32 * 4 + 16 * 32 * 4 + 16 * 16 * 4 + 32 * 4 + 1
    seg = 4 * 32 * 64 * 4 + 4 * 32 * 32 * 4
    assert n >= nu * per_unit + seg
    st2, n2 = ws_size(lib, 1, 2500, 64, 32, 32, 16, F32)          # 128 chains: no segments
    assert n2 < 64 * nu * per_unit + 7 * 256 + 1


def test_forward_validation(lib):
    assert fwd(lib, q=None) == NULLP
    assert fwd(lib, out=None) == NULLP
    assert fwd(lib, ws=None) == NULLP
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, T=-3) == SHAPE
    assert fwd(lib, Dk=20) == UNSUP
    assert fwd(lib, Dv=8) == UNSUP
    assert fwd(lib, C=128) == UNSUP
    assert fwd(lib, mode=2) == UNSUP
    assert fwd(lib, flags=1 << 5) == UNSUP
    # the range-check flag is known; argument errors still come first, before
    # the device check makes any HIP call
    assert fwd(lib, flags=1, q=None) == NULLP
    assert fwd(lib, flags=1, Dk=20) == UNSUP
    assert fwd(lib, flags=1, wsb=0) == WS
    assert fwd(lib, dt=5) == UNSUP
    assert fwd(lib, q=ctypes.c_void_p(0x7f0000000008)) == MISAL
    assert fwd(lib, beta=ctypes.c_void_p(0x7f0000000002)) == MISAL
    assert fwd(lib, wsb=0) == WS


def test_forward_alias_rules(lib):
    f = Fake()
    base = f(1 << 24)
    # out overlapping q
    assert fwd(lib, q=base, out=ctypes.c_void_p(base.value + 256)) == ALIAS
    # final_state overlapping out
    assert fwd(lib, out=base, st=ctypes.c_void_p(base.value)) == ALIAS
    # workspace overlapping alpha
    assert fwd(lib, alpha=base, ws=ctypes.c_void_p(base.value + 1024)) == ALIAS
    # final_state == initial_state is allowed (validation passes -> would launch; so only
    # check that a *partial* overlap is rejected)
    s0 = f(1 << 20)
    assert fwd(lib, s0=s0, st=ctypes.c_void_p(s0.value + 16)) == ALIAS


def fwd_states(lib, cs, **kw):
    f = Fake()
    B, T, H, Dk, Dv, C = 1, kw.get("T", 64), 2, 16, 16, 16
    st, need = ws_size(lib, B, max(T, 0), H, Dk, Dv, C, F32)
    a = dict(q=f(), k=f(), v=f(), alpha=f(), beta=f(), out=f(), ws=f(max(need, 1) + 4096))
    a.update({k_: v_ for k_, v_ in kw.items() if k_ in a})
    return lib.kda_chunk_forward_states(a["q"], a["k"], a["v"], a["alpha"], a["beta"], None,
                                        a["out"], None, cs, B, T, H, Dk, Dv, C, F32, 1, 0,
                                        a["ws"], need, None)


def test_forward_states_validation(lib):
    f = Fake()
    assert fwd_states(lib, None) == NULLP                       # states required when T > 0
    assert fwd_states(lib, ctypes.c_void_p(0x7f0000000002)) == MISAL
    base = f(1 << 24)
    # the states region (1 x 2 x 4 x 16 x 16 fp32 = 8 KiB) overlapping q, out or workspace
    assert fwd_states(lib, ctypes.c_void_p(base.value + 4096), q=base) == ALIAS
    assert fwd_states(lib, ctypes.c_void_p(base.value), out=ctypes.c_void_p(base.value + 8188)) == ALIAS
    assert fwd_states(lib, ctypes.c_void_p(base.value + 64), ws=base) == ALIAS
    assert fwd_states(lib, f(), T=-1) == SHAPE


def fwd_prologue(lib, pro, mode=1, **kw):
    f = Fake()
    B, T, H, Dk, Dv, C = 1, 64, 2, 16, 16, 16
    st, need = ws_size(lib, B, T, H, Dk, Dv, C, F32)
    p = None if pro is None else ctypes.byref(kda.Prologue(*pro))
    return lib.kda_chunk_forward_prologue(f(), f(), f(), f(), f(), p, None, f(), None,
                                          B, T, H, Dk, Dv, C, F32, mode, 0,
                                          f(max(need, 1) + 4096), need, None)


def test_forward_prologue_validation(lib):
    assert fwd_prologue(lib, None) == NULLP
    assert fwd_prologue(lib, (-1.5, 1.0, 1.0, 1e-6, 1)) == UNSUP       # gate below -1
    assert fwd_prologue(lib, (0.5, 0.25, 1.0, 1e-6, 1)) == UNSUP       # alpha_min > alpha_max
    assert fwd_prologue(lib, (0.0, 1.0, 2.5, 1e-6, 1)) == UNSUP        # beta above 2
    assert fwd_prologue(lib, (0.0, 1.0, 1.0, -1.0, 1)) == UNSUP        # eps < 0
    assert fwd_prologue(lib, (0.0, 1.0, 1.0, float("nan"), 1)) == UNSUP
    assert fwd_prologue(lib, (0.0, 1.0, 1.0, 1e-6, 2)) == UNSUP        # normalize_q not 0/1
    assert fwd_prologue(lib, (-1.0, 1.0, 1.0, 1e-6, 1), mode=0) == UNSUP   # KDA: gates >= 0
    assert fwd_prologue(lib, (0.0, 1.0, 2.0, 1e-6, 1), mode=0) == UNSUP    # KDA: beta <= 1


def test_varlen_workspace_and_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_forward_varlen_workspace_size(3, 300, 2, 64, 64, 32, BF16, ctypes.byref(n)) == OK
    # per-unit regions for ceil(300 / 32) + 3 = 13 chunks x 2 heads, then the two tables
    per_unit = 3 * 32 * 64 * 2 + 32 * 64 * 2 + 32 * 32 * 2 + 64 * 4 + 1
    assert n.value >= 26 * per_unit and n.value < 26 * per_unit + 26 * 7 * 256 + 512
    assert lib.kda_chunk_forward_varlen_workspace_size(0, 10, 1, 16, 16, 16, F32, ctypes.byref(n)) == SHAPE
    f = Fake()

    def vl(cu=True, N=2, total=40, ws=True, q=True):
        need = ctypes.c_size_t(0)
        lib.kda_chunk_forward_varlen_workspace_size(max(N, 1), total, 2, 16, 16, 16, F32, ctypes.byref(need))
        return lib.kda_chunk_forward_varlen(f() if q else None, f(), f(), f(), f(), None,
                                            f() if cu else None, N, None, f(), None, total, 2, 16,
                                            16, 16, F32, 1, 0, f(need.value + 4096) if ws else None,
                                            need.value, None)
    assert vl(cu=False) == NULLP
    assert vl(ws=False) == NULLP
    assert vl(q=False) == NULLP
    assert vl(N=0) == SHAPE
    assert vl(total=-1) == SHAPE


def test_phase_validation(lib):
    f = Fake()
    st, need = ws_size(lib, 1, 64, 2, 16, 16, 16, F32)
    call = lambda theta, out=None: lib.kda_chunk_forward_phase(
        f(), f(), f(), f(), theta, f(), None, out or f(), None, 1, 64, 2, 16, 16, 16, F32, 1, 0,
        f(need + 4096), need, None)
    assert call(None) == NULLP
    assert call(ctypes.c_void_p(0x7f0000000004)) == MISAL            # pairs of floats: 8-byte rule
    base = f(1 << 20)
    assert call(ctypes.c_void_p(base.value + 16), out=base) == ALIAS     # out overlapping theta
    assert lib.kda_decode_step_phase(f(), f(), f(), f(), None, f(), f(), f(), 1, 1, 16, 16, F32,
                                     1, 0, None) == NULLP


def test_decode_validation(lib):
    f = Fake()
    a = [f() for _ in range(7)]

    def dec(ptrs=a, B=2, H=2, Dk=16, Dv=16, dt=BF16, mode=1, flags=0):
        return lib.kda_decode_step(*ptrs, B, H, Dk, Dv, dt, mode, flags, None)

    assert dec(ptrs=[None] + a[1:]) == NULLP
    assert dec(B=0) == SHAPE
    assert dec(Dk=48) == UNSUP
    assert dec(Dv=200) == UNSUP
    assert dec(mode=-1) == UNSUP
    assert dec(ptrs=a[:5] + [ctypes.c_void_p(a[5].value + 4)] + a[6:]) == MISAL   # state
    assert dec(ptrs=a[:4] + [ctypes.c_void_p(a[4].value + 2)] + a[5:]) == MISAL   # beta
    assert dec(ptrs=a[:6] + [a[5]]) == ALIAS          # out == state


def test_decode_prologue_validation(lib):
    f = Fake()
    a = [f() for _ in range(7)]      # q_raw, k_raw, v, gate, beta_logit, state, out

    def dec(ptrs=a, pro=kda.Prologue(-1.0, 1.0, 2.0, 1e-6, 1), mode=1, Dk=16):
        p = None if pro is None else ctypes.byref(pro)
        return lib.kda_decode_step_prologue(*ptrs[:5], p, *ptrs[5:], 2, 2, Dk, 16, BF16, mode, 0,
                                            None)

    assert dec(pro=None) == NULLP
    assert dec(ptrs=[None] + a[1:]) == NULLP
    assert dec(Dk=48) == UNSUP
    assert dec(mode=0) == UNSUP                                             # CKDA range in KDA mode
    assert dec(pro=kda.Prologue(0.5, 0.2, 1.0, 0.0, 1), mode=1) == UNSUP    # alpha_min > alpha_max
    assert dec(pro=kda.Prologue(-1.0, 1.0, 2.0, -1.0, 1)) == UNSUP         # eps < 0
    assert dec(ptrs=a[:5] + [ctypes.c_void_p(a[5].value + 4)] + a[6:]) == MISAL   # state
    assert dec(ptrs=a[:6] + [a[5]]) == ALIAS                                # out == state


def test_gate_prep_validation(lib):
    f = Fake()
    a = [f() for _ in range(4)]
    assert lib.kda_gate_prep(None, *a[1:], 1, 10, 1, 16, 16, None) == NULLP
    assert lib.kda_gate_prep(*a, 1, 10, 1, 16, 20, None) == UNSUP
    assert lib.kda_gate_prep(*a, 1, -1, 1, 16, 16, None) == SHAPE
    assert lib.kda_gate_prep(*a, 1, 0, 1, 16, 16, None) == OK       # nothing to do
    off = lambda i, d: a[:i] + [ctypes.c_void_p(a[i].value + d)] + a[i + 1:]
    assert lib.kda_gate_prep(*off(0, 4), 1, 10, 1, 16, 16, None) == MISAL   # alpha: 16 B
    assert lib.kda_gate_prep(*off(1, 8), 1, 10, 1, 16, 16, None) == MISAL   # L: 16 B
    assert lib.kda_gate_prep(*off(2, 2), 1, 10, 1, 16, 16, None) == MISAL   # meta: 4 B
    assert lib.kda_gate_prep(*off(3, 4), 1, 10, 1, 16, 16, None) == MISAL   # gend: 16 B


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.chunk_forward(x, x, x, x, torch.zeros(1, 4, 1), chunk=16, workspace=torch.zeros(1))


def test_backward_workspace_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_workspace_size(1, 8192, 32, 128, 128, 64, BF16, ctypes.byref(n)) == OK
    nu = 32 * 128
    fwd = nu * (3 * 64 * 128 * 2 + 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4 + 1)
    # plus Tinv, chunk states, Delta, state gradients, X (fp32) and one flag byte per unit
    extra = nu * (64 * 64 * 4 + 128 * 128 * 4 + 64 * 128 * 4 + 128 * 128 * 4 + 64 * 128 * 4) + nu
    assert n.value == fwd + extra
    assert lib.kda_chunk_backward_workspace_size(1, 100, 2, 16, 16, 64, BF16, ctypes.byref(n)) == UNSUP
    assert lib.kda_chunk_backward_workspace_size(1, 100, 2, 64, 64, 16, BF16, ctypes.byref(n)) == UNSUP
    assert lib.kda_chunk_backward_workspace_size(1, 100, 2, 128, 64, 64, F32, ctypes.byref(n)) == UNSUP
    assert lib.kda_chunk_backward_workspace_size(1, 0, 2, 64, 64, 64, F32, ctypes.byref(n)) == OK
    assert n.value == 0
    assert lib.kda_chunk_backward_workspace_size(1, 10, 2, 64, 64, 64, F32, None) == NULLP


def test_backward_validation(lib):
    f = Fake()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_workspace_size(1, 64, 2, 64, 64, 64, F32, ctypes.byref(n)) == OK
    need = n.value

    def bw(ptrs=None, T=64, Dk=64, chunk=64, dt=F32, mode=1, flags=0, ws=True, wsb=None):
        p = ptrs if ptrs is not None else [f() for _ in range(14)]
        return lib.kda_chunk_backward(*p, 1, T, 2, Dk, 64, chunk, dt, mode, flags,
                                      f(need + 4096) if ws else None,
                                      need if wsb is None else wsb, None)

    base = [f() for _ in range(14)]
    assert bw(ptrs=[None] + base[1:]) == NULLP                    # q
    assert bw(ptrs=base[:6] + [None] + base[7:]) == NULLP         # d_out
    assert bw(ws=False) == NULLP
    assert bw(wsb=need - 1) == WS
    assert bw(chunk=16) == UNSUP
    assert bw(Dk=16) == UNSUP
    assert bw(mode=5) == UNSUP
    assert bw(flags=4) == UNSUP                                    # segments are forward-only
    assert bw(flags=1) == UNSUP                                    # range check: forward only
    mis = list(base)
    mis[6] = ctypes.c_void_p(base[6].value + 4)                   # d_out: 16-byte rule
    assert bw(ptrs=mis) == MISAL
    al = list(base)
    al[8] = base[0]                                               # dq == q
    assert bw(ptrs=al) == ALIAS
    al = list(base)
    al[9] = base[8]                                               # dk == dq
    assert bw(ptrs=al) == ALIAS
    opt = list(base)
    opt[5] = opt[7] = opt[13] = None                              # S0, dST, dS0 optional
    assert bw(ptrs=opt, T=0) == OK                                # nothing to do, no HIP call


def test_save_and_saved_validation(lib):
    """kda_chunk_forward_save / kda_chunk_backward_saved: the backward's
    supported set and argument rules (checked before any HIP call)."""
    f = Fake()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_workspace_size(1, 64, 2, 64, 64, 64, F32, ctypes.byref(n)) == OK
    need = n.value

    def fs(ptrs=None, T=64, Dk=64, chunk=64, dt=F32, mode=1, flags=0, ws=True, wsb=None):
        p = ptrs if ptrs is not None else [f() for _ in range(8)]
        return lib.kda_chunk_forward_save(*p, 1, T, 2, Dk, 64, chunk, dt, mode, flags,
                                          f(need + 4096) if ws else None,
                                          need if wsb is None else wsb, None)

    base = [f() for _ in range(8)]                  # q k v alpha beta S0 out ST
    assert fs(ptrs=[None] + base[1:]) == NULLP
    assert fs(ptrs=base[:6] + [None] + base[7:]) == NULLP         # out
    assert fs(ws=False) == NULLP
    assert fs(wsb=need - 1) == WS
    assert fs(chunk=16) == UNSUP
    assert fs(Dk=16) == UNSUP
    assert fs(flags=4) == UNSUP
    al = list(base)
    al[6] = base[2]                                               # out == v
    assert fs(ptrs=al) == ALIAS
    al = list(base)
    al[7] = base[5]                                               # final state == S0
    assert fs(ptrs=al) == ALIAS
    opt = list(base)
    opt[5] = opt[7] = None
    assert fs(ptrs=opt, T=0) == OK                                # nothing to do, no HIP call

    def bs(ptrs=None, T=64, chunk=64, flags=0, ws=True, wsb=None):
        p = ptrs if ptrs is not None else [f() for _ in range(13)]
        return lib.kda_chunk_backward_saved(*p, 1, T, 2, 64, 64, chunk, F32, 1, flags,
                                            f(need + 4096) if ws else None,
                                            need if wsb is None else wsb, None)

    base = [f() for _ in range(13)]      # q k v alpha beta dO dST dq dk dv dalpha dbeta dS0
    assert bs(ptrs=base[:5] + [None] + base[6:]) == NULLP         # d_out
    assert bs(ptrs=base[:7] + [None] + base[8:]) == NULLP         # dq
    assert bs(ws=False) == NULLP
    assert bs(wsb=need - 1) == WS
    assert bs(chunk=16) == UNSUP
    al = list(base)
    al[7] = base[0]                                               # dq == q
    assert bs(ptrs=al) == ALIAS
    opt = list(base)
    opt[6] = opt[12] = None
    assert bs(ptrs=opt, T=0) == OK


def test_backward_prologue_validation(lib):
    f = Fake()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_prologue_workspace_size(1, 64, 2, 64, 64, 64, F32, ctypes.byref(n)) == OK
    need = n.value
    m = ctypes.c_size_t(0)
    lib.kda_chunk_backward_workspace_size(1, 64, 2, 64, 64, 64, F32, ctypes.byref(m))
    assert need > m.value                       # the transformed inputs and their gradients

    def bw(ptrs=None, pro=kda.Prologue(-1.0, 1.0, 2.0, 1e-6, 1), mode=1, T=64):
        p = ptrs if ptrs is not None else [f() for _ in range(14)]
        return lib.kda_chunk_backward_prologue(*p[:8], ctypes.byref(pro) if pro else None, *p[8:],
                                               1, T, 2, 64, 64, 64, F32, mode, 0, f(need + 4096),
                                               need, None)

    base = [f() for _ in range(14)]
    assert bw(pro=None) == NULLP
    assert bw(pro=kda.Prologue(-1.0, 1.0, 2.0, 1e-6, 1), mode=0) == UNSUP   # CKDA range in KDA mode
    assert bw(pro=kda.Prologue(0.5, 0.2, 1.0, 0.0, 1), mode=1) == UNSUP      # alpha_min > alpha_max
    assert bw(ptrs=[None] + base[1:]) == NULLP
    mis = list(base)
    mis[3] = ctypes.c_void_p(base[3].value + 4)                               # gate: 16-byte rule
    assert bw(ptrs=mis) == MISAL
    al = list(base)
    al[11] = base[3]                                                          # d_gate == gate
    assert bw(ptrs=al) == ALIAS


def test_backward_varlen_prologue_validation(lib):
    f = Fake()
    n, m = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_varlen_prologue_workspace_size(3, 200, 2, 64, 64, 64, F32,
                                                                  ctypes.byref(n)) == OK
    lib.kda_chunk_backward_varlen_workspace_size(3, 200, 2, 64, 64, 64, F32, ctypes.byref(m))
    assert n.value > m.value                     # plus the transformed inputs and their gradients
    assert lib.kda_chunk_backward_varlen_prologue_workspace_size(0, 200, 2, 64, 64, 64, F32,
                                                                  ctypes.byref(n)) == SHAPE
    need = n.value if n.value else 1 << 20
    lib.kda_chunk_backward_varlen_prologue_workspace_size(3, 200, 2, 64, 64, 64, F32, ctypes.byref(n))
    need = n.value

    def bw(ptrs=None, pro=kda.Prologue(-1.0, 1.0, 2.0, 1e-6, 1), mode=1):
        p = ptrs if ptrs is not None else [f() for _ in range(15)]
        pp = None if pro is None else ctypes.byref(pro)
        return lib.kda_chunk_backward_varlen_prologue(*p[:6], 3, *p[6:9], pp, *p[9:], 200, 2, 64,
                                                      64, 64, F32, mode, 0, f(need + 4096), need,
                                                      None)

    base = [f() for _ in range(15)]
    assert bw(ptrs=base[:5] + [None] + base[6:]) == NULLP             # cu_seqlens
    assert bw(ptrs=base, pro=None) == NULLP                            # prologue
    assert bw(ptrs=base, mode=0) == UNSUP                              # CKDA range in KDA mode
    mis = list(base)
    mis[5] = ctypes.c_void_p(base[5].value + 2)                        # cu_seqlens: 4-byte rule
    assert bw(ptrs=mis) == MISAL
    al = list(base)
    al[9] = base[5]                                                    # dq_raw == cu_seqlens
    assert bw(ptrs=al) == ALIAS


def test_backward_varlen_validation(lib):
    f = Fake()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 200, 2, 64, 64, 64, F32, ctypes.byref(n)) == OK
    need = n.value
    m = ctypes.c_size_t(0)
    lib.kda_chunk_backward_workspace_size(1, 200, 2, 64, 64, 64, F32, ctypes.byref(m))
    assert need > m.value                       # one more chunk per sequence, plus the tables
    assert lib.kda_chunk_backward_varlen_workspace_size(0, 200, 2, 64, 64, 64, F32, ctypes.byref(n)) == SHAPE
    assert lib.kda_chunk_backward_varlen_workspace_size(3, 200, 2, 64, 64, 16, F32, ctypes.byref(n)) == UNSUP

    def bw(ptrs=None, N=3, total=200):
        p = ptrs if ptrs is not None else [f() for _ in range(15)]
        return lib.kda_chunk_backward_varlen(*p[:6], N, *p[6:], total, 2, 64, 64, 64, F32, 1, 0,
                                             f(need + 4096), need, None)

    base = [f() for _ in range(15)]
    assert bw(ptrs=base[:5] + [None] + base[6:]) == NULLP             # cu_seqlens
    assert bw(ptrs=[None] + base[1:]) == NULLP                         # q
    mis = list(base)
    mis[5] = ctypes.c_void_p(base[5].value + 2)                        # cu_seqlens: 4-byte rule
    assert bw(ptrs=mis) == MISAL
    al = list(base)
    al[9] = base[5]                                                    # dq == cu_seqlens
    assert bw(ptrs=al) == ALIAS


def test_forward_workspace_reserves_the_parts_state(lib):
    """At most 128 (b, h, 16-column) chains (and more than 64, so no
    segments) with at least 256 chunks select the parts path, whose state
    between parts ([B H][Dk][Dv] fp32) lives in the workspace; 255 chunks do
    not.  The query must differ by the per-chunk regions plus that buffer."""
    def ws(T, H=9, D=128, chunk=64):
        n = ctypes.c_size_t(0)
        assert lib.kda_chunk_forward_workspace_size(1, T, H, D, D, chunk, BF16,
                                                    ctypes.byref(n)) == OK
        return n.value
    per_chunk = ws(64 * 2) - ws(64 * 1)            # the per-unit regions of one more chunk per head
    with_parts, without = ws(64 * 256), ws(64 * 255)
    state = (9 * 128 * 128 * 4 + 255) // 256 * 256
    assert with_parts - without == per_chunk + state
    # 256 chains (H = 32): no parts, so no state buffer
    big = lambda T: ws(T, H=32)
    assert big(64 * 256) - big(64 * 255) == big(64 * 2) - big(64 * 1)


def test_noalloc_refusals_before_any_hip_call(lib):
    """kda_chunk_forward_noalloc checks shape, flags and its scratch limit
    before it touches the GPU: a shape whose workspace exceeds the built-in
    scratch (KDA_NOALLOC_SCRATCH_BYTES, 32 MiB) is KDA_ERR_SCRATCH_LIMIT, the
    event and range-check flags are refused, and a bad shape keeps its own
    status."""
    SCRATCH_LIMIT = 9
    f = Fake()
    q, k, v, a, b, s0, o, st = (f() for _ in range(8))
    lib.kda_chunk_forward_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 8 + \
        [ctypes.c_uint, ctypes.c_void_p]
    call = lambda B, T, H, D, C, dt, fl: lib.kda_chunk_forward_noalloc(
        q, k, v, a, b, s0, o, st, B, T, H, D, D, C, dt, 1, fl, None)
    # the headline prefill needs ~297 MB of workspace
    assert call(1, 8192, 32, 128, 64, BF16, 0) == SCRATCH_LIMIT
    n_big = ws_size(lib, 1, 8192, 32, 128, 128, 64, BF16)[1]
    assert n_big > 32 << 20
    # the longest single-head bf16 d = 128 sequence that fits, found by
    # bisection on the workspace query; one token more is refused
    lo, hi = 1, 1 << 20
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if ws_size(lib, 1, mid, 1, 128, 128, 64, BF16)[1] <= 32 << 20:
            lo = mid
        else:
            hi = mid
    assert ws_size(lib, 1, hi, 1, 128, 128, 64, BF16)[1] > 32 << 20
    assert call(1, hi, 1, 128, 64, BF16, 0) == SCRATCH_LIMIT
    assert call(1, 64, 1, 128, 64, BF16, 2) == UNSUP          # KDA_FLAG_STAGE_EVENTS
    assert call(1, 64, 1, 128, 64, BF16, 1) == UNSUP          # KDA_FLAG_VALIDATE_RANGES
    assert call(1, 64, 1, 128, 64, BF16, 64) == UNSUP         # unknown flag
    assert call(0, 64, 1, 128, 64, BF16, 0) == SHAPE
    assert call(1, 64, 1, 24, 64, BF16, 0) == UNSUP
    assert lib.kda_status_string(SCRATCH_LIMIT) != b"unknown status"


def test_side_stream_refusals_before_any_hip_call(lib):
    """kda_chunk_forward_side: a side argument with a NULL stream or a NULL
    event is KDA_ERR_NULL_POINTER, found before any HIP call; shape errors keep
    their own status."""
    f = Fake()
    q, k, v, a, b, o, st, ws = (f() for _ in range(8))
    side = kda._Side(None, (ctypes.c_void_p * kda.SIDE_EVENTS)(*[f() for _ in range(kda.SIDE_EVENTS)]))
    lib.kda_chunk_forward_side.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 8 + \
        [ctypes.c_uint, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(kda._Side)]
    nws = ws_size(lib, 1, 4096, 1, 64, 64, 16, F32)[1]
    call = lambda sd, D=64: lib.kda_chunk_forward_side(q, k, v, a, b, None, o, st, 1, 4096, 1, D, D,
                                                       16, F32, 1, 0, ws, nws, None, ctypes.byref(sd))
    assert call(side) == NULLP                     # no stream
    side.stream = f()
    side.events[3] = None
    assert call(side) == NULLP                     # an event missing
    side.events[3] = f()
    assert call(side, D=24) == UNSUP               # the shape check still comes first


def test_backward_phase_validation(lib):
    """kda_chunk_backward_phase: the backward's supported set, theta and
    d_theta required, the pair-sized gate arrays in the alias checks."""
    f = Fake()
    n = ctypes.c_size_t(0)
    assert lib.kda_chunk_backward_phase_workspace_size(1, 64, 2, 64, 64, 64, F32, ctypes.byref(n)) == OK
    need = n.value
    m = ctypes.c_size_t(0)
    lib.kda_chunk_backward_workspace_size(1, 64, 2, 64, 64, 64, F32, ctypes.byref(m))
    assert need > m.value                       # the rotated inputs, their gradients, the tables
    z = ctypes.c_size_t(1)
    assert lib.kda_chunk_backward_phase_workspace_size(1, 0, 2, 64, 64, 64, F32, ctypes.byref(z)) == OK
    assert z.value == 0
    assert lib.kda_chunk_backward_phase_workspace_size(1, 64, 2, 16, 64, 64, F32, ctypes.byref(z)) == UNSUP

    def bp(ptrs=None, T=64, Dk=64, chunk=64, mode=1, flags=0, ws=True, wsb=None):
        p = ptrs if ptrs is not None else [f() for _ in range(16)]
        return lib.kda_chunk_backward_phase(*p, 1, T, 2, Dk, 64, chunk, F32, mode, flags,
                                            f(need + 4096) if ws else None,
                                            need if wsb is None else wsb, None)

    # q k v alpha theta beta S0 dO dST dq dk dv dalpha dtheta dbeta dS0
    base = [f() for _ in range(16)]
    for i in (0, 3, 4, 7, 9, 12, 13, 14):
        assert bp(ptrs=base[:i] + [None] + base[i + 1:]) == NULLP, i
    assert bp(ws=False) == NULLP
    assert bp(wsb=need - 1) == WS
    assert bp(chunk=16) == UNSUP
    assert bp(Dk=16) == UNSUP
    assert bp(mode=2) == UNSUP
    assert bp(flags=4) == UNSUP
    al = list(base)
    al[13] = base[4]                                              # d_theta == theta
    assert bp(ptrs=al) == ALIAS
    al = list(base)
    al[12] = base[13]                                             # d_alpha == d_theta
    assert bp(ptrs=al) == ALIAS
    opt = list(base)
    opt[8] = opt[15] = None
    assert bp(ptrs=opt, T=0) == OK                                # nothing to do, no HIP call
