"""gated_delta_rule_forward_amd — KDA / CKDA recurrence on AMD MI355X (gfx950).

Thin ctypes binding over libkda.so (C ABI in include/kda.h).  This module only
marshals arguments: it passes tensor data pointers, sizes and the current HIP
stream to the library, and allocates outputs / workspace with torch when the
caller does not supply them.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If libkda.so is missing the first call raises.

Recurrence ("Semidirect Fourier Delta Attention", §1 eq. (1), §3 eq. (14)):
    S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KDA", "CKDA", "KdaError", "library_path", "load", "abi_version", "workspace_size",
    "chunk_forward_save", "chunk_backward_saved", "chunk_backward_phase",
    "backward_phase_workspace_size",
    "chunk_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "SideStream", "SIDE_EVENTS",
    "chunk_forward", "chunk_forward_prologue", "chunk_forward_varlen", "chunk_forward_phase",
    "decode_step", "decode_step_phase", "decode_step_prologue", "gate_prep", "last_stage_times",
    "chunk_backward", "chunk_backward_prologue", "chunk_backward_varlen",
    "chunk_backward_varlen_prologue", "backward_workspace_size",
    "VALIDATE_RANGES", "STAGE_EVENTS", "NO_SEGMENTS", "SINGLE_STREAM",
]

KDA, CKDA = 0, 1
STAGE_EVENTS = 2
VALIDATE_RANGES = 1    # KDA_FLAG_VALIDATE_RANGES
NO_SEGMENTS = 4        # KDA_FLAG_NO_SEGMENTS
SINGLE_STREAM = 8      # KDA_FLAG_SINGLE_STREAM
STREAMED = 16          # KDA_FLAG_STREAMED
_DT = {torch.float32: 0, torch.bfloat16: 1}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None

_STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "unsupported", 4: "misaligned",
           5: "workspace too small", 6: "alias", 7: "hip error",
           8: "input out of range", 9: "workspace above the built-in scratch"}
NOALLOC_SCRATCH_BYTES = 32 << 20     # KDA_NOALLOC_SCRATCH_BYTES


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({_STATUS.get(status, 'unknown')})")


SIDE_EVENTS = 9    # KDA_SIDE_EVENTS


class _Side(ctypes.Structure):
    """kda_side_t (include/kda.h)."""
    _fields_ = [("stream", ctypes.c_void_p), ("events", ctypes.c_void_p * SIDE_EVENTS)]


class SideStream:
    """A second stream and its events (kda_side_stream_create: a stream with a
    hardware queue of its own), owned here and lent to kda_chunk_forward_side
    (chunk_forward(..., side=...)).  `stream` wraps it for torch
    (torch.cuda.ExternalStream).  The streamed form is not taken for calls
    on the null stream (torch's default current stream): launch those calls
    on a torch.cuda.Stream()."""

    def __init__(self, device=None):
        lib = load()
        self._c = _Side()
        with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
            _check("kda_side_stream_create", lib.kda_side_stream_create(ctypes.byref(self._c)))
        # (kept for __del__, which may run while the interpreter shuts down)
        self._destroy, self._byref = lib.kda_side_stream_destroy, ctypes.byref
        self.stream = torch.cuda.ExternalStream(self._c.stream, device=device)

    def _as_arg(self):
        return ctypes.byref(self._c)

    def __del__(self):
        c = getattr(self, "_c", None)
        if c is not None and c.stream and getattr(self, "_destroy", None) is not None:
            self._destroy(self._byref(c))


class Prologue(ctypes.Structure):
    """kda_prologue_t (include/kda.h)."""
    _fields_ = [("alpha_min", ctypes.c_float), ("alpha_max", ctypes.c_float),
                ("beta_max", ctypes.c_float), ("eps", ctypes.c_float),
                ("normalize_q", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libkda.so (built by gated_delta_rule_forward_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libkda.so not built ({_LIB_PATH}); run "
                           "`python -m gated_delta_rule_forward_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.kda_abi_version.restype = i
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_forward_workspace_size.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.kda_chunk_forward_workspace_size.restype = i
    lib.kda_chunk_forward.argtypes = [vp] * 8 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_forward.restype = i
    lib.kda_chunk_forward_side.argtypes = [vp] * 8 + [i] * 8 + [u, vp, sz, vp, ctypes.POINTER(_Side)]
    lib.kda_chunk_forward_side.restype = i
    lib.kda_side_stream_create.argtypes = [ctypes.POINTER(_Side)]
    lib.kda_side_stream_create.restype = i
    lib.kda_side_stream_destroy.argtypes = [ctypes.POINTER(_Side)]
    lib.kda_side_stream_destroy.restype = i
    lib.kda_chunk_forward_noalloc.argtypes = [vp] * 8 + [i] * 8 + [u, vp]
    lib.kda_chunk_forward_noalloc.restype = i
    lib.kda_chunk_forward_states.argtypes = [vp] * 9 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_forward_states.restype = i
    lib.kda_chunk_forward_prologue.argtypes = [vp] * 5 + [ctypes.POINTER(Prologue)] + [vp] * 3 + \
        [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_forward_prologue.restype = i
    lib.kda_chunk_forward_phase.argtypes = [vp] * 9 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_forward_phase.restype = i
    lib.kda_decode_step_phase.argtypes = [vp] * 8 + [i] * 6 + [u, vp]
    lib.kda_decode_step_phase.restype = i
    lib.kda_chunk_forward_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.kda_chunk_forward_varlen_workspace_size.restype = i
    lib.kda_chunk_forward_varlen.argtypes = [vp] * 5 + [ctypes.POINTER(Prologue), vp, i, vp, vp,
                                                         vp] + [i] * 7 + [u, vp, sz, vp]
    lib.kda_chunk_forward_varlen.restype = i
    lib.kda_decode_step.argtypes = [vp] * 7 + [i] * 6 + [u, vp]
    lib.kda_decode_step.restype = i
    lib.kda_decode_step_prologue.argtypes = [vp] * 5 + [ctypes.POINTER(Prologue)] + [vp] * 2 + \
        [i] * 6 + [u, vp]
    lib.kda_decode_step_prologue.restype = i
    lib.kda_chunk_backward_workspace_size.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.kda_chunk_backward_workspace_size.restype = i
    lib.kda_chunk_backward.argtypes = [vp] * 14 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_backward.restype = i
    lib.kda_chunk_backward_phase_workspace_size.argtypes = [i, i, i, i, i, i, i,
                                                            ctypes.POINTER(sz)]
    lib.kda_chunk_backward_phase_workspace_size.restype = i
    lib.kda_chunk_backward_phase.argtypes = [vp] * 16 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_backward_phase.restype = i
    lib.kda_chunk_forward_save.argtypes = [vp] * 8 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_forward_save.restype = i
    lib.kda_chunk_backward_saved.argtypes = [vp] * 13 + [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_backward_saved.restype = i
    lib.kda_chunk_backward_prologue_workspace_size.argtypes = [i, i, i, i, i, i, i,
                                                               ctypes.POINTER(sz)]
    lib.kda_chunk_backward_prologue_workspace_size.restype = i
    lib.kda_chunk_backward_prologue.argtypes = [vp] * 8 + [ctypes.POINTER(Prologue)] + [vp] * 6 + \
        [i] * 8 + [u, vp, sz, vp]
    lib.kda_chunk_backward_prologue.restype = i
    lib.kda_chunk_backward_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i,
                                                             ctypes.POINTER(sz)]
    lib.kda_chunk_backward_varlen_workspace_size.restype = i
    lib.kda_chunk_backward_varlen.argtypes = [vp] * 6 + [i] + [vp] * 9 + [i] * 7 + [u, vp, sz, vp]
    lib.kda_chunk_backward_varlen.restype = i
    lib.kda_chunk_backward_varlen_prologue_workspace_size.argtypes = [i, i, i, i, i, i, i,
                                                                      ctypes.POINTER(sz)]
    lib.kda_chunk_backward_varlen_prologue_workspace_size.restype = i
    lib.kda_chunk_backward_varlen_prologue.argtypes = [vp] * 6 + [i] + [vp] * 3 + \
        [ctypes.POINTER(Prologue)] + [vp] * 6 + [i] * 7 + [u, vp, sz, vp]
    lib.kda_chunk_backward_varlen_prologue.restype = i
    lib.kda_gate_prep.argtypes = [vp] * 4 + [i] * 5 + [vp]
    lib.kda_gate_prep.restype = i
    lib.kda_last_stage_times.argtypes = [ctypes.POINTER(ctypes.c_float),
                                         ctypes.POINTER(ctypes.c_char_p), i, ctypes.POINTER(i)]
    lib.kda_last_stage_times.restype = i
    _lib = lib
    return lib


def abi_version() -> int:
    return load().kda_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int):
    if status != 0:
        raise KdaError(fn, status)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, chunk: int, dtype: torch.dtype) -> int:
    n = ctypes.c_size_t(0)
    _check("kda_chunk_forward_workspace_size",
           load().kda_chunk_forward_workspace_size(B, T, H, Dk, Dv, chunk, _DT[dtype],
                                                   ctypes.byref(n)))
    return n.value


def chunk_forward(q, k, v, alpha, beta, initial_state=None, *, chunk: int = 64, mode: int = CKDA,
                  out=None, final_state=None, output_final_state: bool = True, workspace=None,
                  chunk_states=None, stream=None, flags: int = 0, side=None):
    """Chunked forward.  q, k: [B,T,H,Dk]; v: [B,T,H,Dv] (fp32 or bf16, same dtype);
    alpha: [B,T,H,Dk] fp32; beta: [B,T,H] fp32; initial_state: [B,H,Dk,Dv] fp32 or None.
    chunk_states: None, or a [B,H,ceil(T/chunk),Dk,Dv] tensor of q's dtype that
    receives the state entering every chunk (kda_chunk_forward_states).
    side: None, or a SideStream lent to kda_chunk_forward_side (not with
    chunk_states).  Returns (out [B,T,H,Dv], final_state [B,H,Dk,Dv] fp32 or None)."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = workspace_size(B, T, H, Dk, Dv, chunk, q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, alpha, beta, initial_state, out, final_state, workspace, chunk_states)
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, k, v and out must share one dtype (float32 or bfloat16)")
    wsb = workspace.numel() * workspace.element_size()
    if side is not None and chunk_states is not None:
        raise ValueError("chunk_states and side cannot be combined")
    if side is not None:
        st = lib.kda_chunk_forward_side(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                        _ptr(initial_state), _ptr(out), _ptr(final_state),
                                        B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                        _ptr(workspace), wsb, _stream(stream), side._as_arg())
        _check("kda_chunk_forward_side", st)
    elif chunk_states is None:
        st = lib.kda_chunk_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(initial_state), _ptr(out), _ptr(final_state),
                                   B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                   _ptr(workspace), wsb, _stream(stream))
        _check("kda_chunk_forward", st)
    else:
        nc = (T + chunk - 1) // chunk
        if chunk_states.dtype != q.dtype or tuple(chunk_states.shape) != (B, H, nc, Dk, Dv):
            raise ValueError("chunk_states must be [B,H,ceil(T/chunk),Dk,Dv] in q's dtype")
        st = lib.kda_chunk_forward_states(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(initial_state), _ptr(out), _ptr(final_state),
                                          _ptr(chunk_states), B, T, H, Dk, Dv, chunk,
                                          _DT[q.dtype], mode, flags, _ptr(workspace), wsb,
                                          _stream(stream))
        _check("kda_chunk_forward_states", st)
    return out, final_state


def chunk_forward_noalloc(q, k, v, alpha, beta, initial_state, out, final_state=None, *,
                          chunk: int = 64, mode: int = CKDA, stream=None, flags: int = 0):
    """kda_chunk_forward_noalloc: the chunked forward with the library's built-in
    scratch in place of a workspace.  The caller passes every tensor (out, and
    final_state or None); nothing is allocated here or in the library.  Returns
    (out, final_state)."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _dev(q, k, v, alpha, beta, initial_state, out, final_state)
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, k, v and out must share one dtype (float32 or bfloat16)")
    st = lib.kda_chunk_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(initial_state), _ptr(out), _ptr(final_state),
                                       B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                       _stream(stream))
    _check("kda_chunk_forward_noalloc", st)
    return out, final_state


def chunk_forward_prologue(q_raw, k_raw, v, gate, beta_logit, initial_state=None, *,
                           alpha_min: float, alpha_max: float, beta_max: float,
                           eps: float = 1e-6, normalize_q: bool = True, chunk: int = 64,
                           mode: int = CKDA, out=None, final_state=None,
                           output_final_state: bool = True, workspace=None, stream=None,
                           flags: int = 0):
    """Chunked forward from raw inputs (kda_chunk_forward_prologue): gate
    [B,T,H,Dk] fp32 and beta_logit [B,T,H] fp32 logits, q_raw / k_raw
    unnormalised; alpha = alpha_min + (alpha_max - alpha_min) sigmoid(gate),
    beta = beta_max sigmoid(beta_logit), k = k_raw / (|k_raw| + eps) and q
    likewise when normalize_q.  Returns (out, final_state)."""
    lib = load()
    B, T, H, Dk = q_raw.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q_raw.dtype, device=q_raw.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q_raw.device)
    if workspace is None:
        nbytes = workspace_size(B, T, H, Dk, Dv, chunk, q_raw.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q_raw.device)
    _dev(q_raw, k_raw, v, gate, beta_logit, initial_state, out, final_state, workspace)
    if q_raw.dtype not in _DT or k_raw.dtype != q_raw.dtype or v.dtype != q_raw.dtype or \
            out.dtype != q_raw.dtype:
        raise ValueError("q_raw, k_raw, v and out must share one dtype (float32 or bfloat16)")
    pro = Prologue(alpha_min, alpha_max, beta_max, eps, int(bool(normalize_q)))
    st = lib.kda_chunk_forward_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(gate),
                                        _ptr(beta_logit), ctypes.byref(pro),
                                        _ptr(initial_state), _ptr(out), _ptr(final_state),
                                        B, T, H, Dk, Dv, chunk, _DT[q_raw.dtype], mode, flags,
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream))
    _check("kda_chunk_forward_prologue", st)
    return out, final_state


def chunk_forward_varlen(q, k, v, alpha, beta, cu_seqlens, initial_state=None, *,
                         chunk: int = 64, mode: int = CKDA, prologue: dict | None = None,
                         out=None, final_state=None, output_final_state: bool = True,
                         workspace=None, stream=None, flags: int = 0):
    """Packed batch (kda_chunk_forward_varlen): q, k, alpha [total_T,H,Dk]
    (or [1,total_T,H,Dk]); v [.., total_T,H,Dv]; beta [.., total_T,H];
    cu_seqlens int32 [N+1] on the GPU; initial_state [N,H,Dk,Dv] fp32 or
    None.  prologue: None or dict(alpha_min=, alpha_max=, beta_max=, eps=,
    normalize_q=) (alpha, beta are then logits).  Returns (out shaped like v,
    final_state [N,H,Dk,Dv] or None)."""
    lib = load()
    H, Dk = q.shape[-2], q.shape[-1]
    total_T = q.shape[-3]
    Dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or N < 1:
        raise ValueError("cu_seqlens must be an int32 tensor of N + 1 offsets, N >= 1")
    if out is None:
        out = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check("kda_chunk_forward_varlen_workspace_size",
               lib.kda_chunk_forward_varlen_workspace_size(N, total_T, H, Dk, Dv, chunk,
                                                           _DT[q.dtype], ctypes.byref(n)))
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, alpha, beta, cu_seqlens, initial_state, out, final_state, workspace)
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("q, k, v and out must share one dtype (float32 or bfloat16)")
    pro = None if prologue is None else ctypes.byref(Prologue(
        prologue["alpha_min"], prologue["alpha_max"], prologue["beta_max"],
        prologue.get("eps", 1e-6), int(bool(prologue.get("normalize_q", True)))))
    st = lib.kda_chunk_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), pro,
                                      _ptr(cu_seqlens), N, _ptr(initial_state), _ptr(out),
                                      _ptr(final_state), total_T, H, Dk, Dv, chunk, _DT[q.dtype],
                                      mode, flags, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    _check("kda_chunk_forward_varlen", st)
    return out, final_state


def chunk_forward_phase(q, k, v, alpha, theta, beta, initial_state=None, *, chunk: int = 64,
                        mode: int = CKDA, out=None, final_state=None,
                        output_final_state: bool = True, workspace=None, stream=None,
                        flags: int = 0):
    """Phase variant (kda_chunk_forward_phase): alpha and theta [B,T,H,Dk/2]
    fp32, one decay and one phase per channel pair; everything else as
    chunk_forward.  Returns (out, final_state)."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = workspace_size(B, T, H, Dk, Dv, chunk, q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, alpha, theta, beta, initial_state, out, final_state, workspace)
    st = lib.kda_chunk_forward_phase(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(theta),
                                     _ptr(beta), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                     B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    _check("kda_chunk_forward_phase", st)
    return out, final_state


def decode_step_phase(q, k, v, alpha, theta, beta, state, *, out=None, mode: int = CKDA,
                      stream=None, flags: int = 0):
    """Phase-variant decode (kda_decode_step_phase): alpha, theta [B,H,Dk/2];
    state [B,H,Dk,Dv] fp32 updated in place.  Returns out [B,H,Dv]."""
    lib = load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _dev(q, k, v, alpha, theta, beta, state, out)
    st = lib.kda_decode_step_phase(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(theta),
                                   _ptr(beta), _ptr(state), _ptr(out), B, H, Dk, Dv,
                                   _DT[q.dtype], mode, flags, _stream(stream))
    _check("kda_decode_step_phase", st)
    return out


def decode_step(q, k, v, alpha, beta, state, *, out=None, mode: int = CKDA, stream=None,
                flags: int = 0):
    """One token for every (b, h): q, k: [B,H,Dk]; v: [B,H,Dv]; alpha: [B,H,Dk] fp32;
    beta: [B,H] fp32; state: [B,H,Dk,Dv] fp32, updated in place.  Returns out [B,H,Dv]."""
    lib = load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _dev(q, k, v, alpha, beta, state, out)
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
                             _ptr(out), B, H, Dk, Dv, _DT[q.dtype], mode, flags, _stream(stream))
    _check("kda_decode_step", st)
    return out


def decode_step_prologue(q_raw, k_raw, v, gate, beta_logit, state, *, alpha_min: float,
                         alpha_max: float, beta_max: float, eps: float = 1e-6,
                         normalize_q: bool = True, out=None, mode: int = CKDA, stream=None,
                         flags: int = 0):
    """One token for every (b, h) from raw inputs (kda_decode_step_prologue):
    gate [B,H,Dk] and beta_logit [B,H] fp32 logits, q_raw / k_raw
    unnormalised; the transforms of chunk_forward_prologue.  state [B,H,Dk,Dv]
    fp32 is updated in place.  Returns out [B,H,Dv]."""
    lib = load()
    B, H, Dk = q_raw.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q_raw.dtype, device=q_raw.device)
    _dev(q_raw, k_raw, v, gate, beta_logit, state, out)
    pro = Prologue(alpha_min, alpha_max, beta_max, eps, 1 if normalize_q else 0)
    st = lib.kda_decode_step_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(gate),
                                      _ptr(beta_logit), ctypes.byref(pro), _ptr(state), _ptr(out),
                                      B, H, Dk, Dv, _DT[q_raw.dtype], mode, flags, _stream(stream))
    _check("kda_decode_step_prologue", st)
    return out


def backward_workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, chunk: int,
                            dtype: torch.dtype) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    st = lib.kda_chunk_backward_workspace_size(B, T, H, Dk, Dv, chunk, _DT[dtype], ctypes.byref(n))
    _check("kda_chunk_backward_workspace_size", st)
    return n.value


def chunk_backward(q, k, v, alpha, beta, d_out, initial_state=None, d_final_state=None, *,
                   chunk: int = 64, mode: int = CKDA, want_d_initial_state: bool = True,
                   grads=None, workspace=None, stream=None, flags: int = 0):
    """Backward of chunk_forward (kda_chunk_backward): gradients of
    sum <out, d_out> + <final_state, d_final_state> with respect to q, k, v,
    alpha, beta and initial_state.  Layouts as chunk_forward; d_out like out,
    d_final_state [B,H,Dk,Dv] fp32 or None.  grads: optional dict of output
    tensors.  Returns a dict dq, dk, dv (q's dtype), d_alpha, d_beta,
    d_initial_state (fp32; None unless wanted)."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    g = dict(grads or {})
    g.setdefault("dq", torch.empty((B, T, H, Dk), dtype=q.dtype, device=dev))
    g.setdefault("dk", torch.empty((B, T, H, Dk), dtype=q.dtype, device=dev))
    g.setdefault("dv", torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev))
    g.setdefault("d_alpha", torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev))
    g.setdefault("d_beta", torch.empty((B, T, H), dtype=torch.float32, device=dev))
    if want_d_initial_state:
        g.setdefault("d_initial_state", torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev))
    else:
        g["d_initial_state"] = None
    if workspace is None:
        nbytes = backward_workspace_size(B, T, H, Dk, Dv, chunk, q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _dev(q, k, v, alpha, beta, d_out, initial_state, d_final_state, workspace, *g.values())
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or d_out.dtype != q.dtype:
        raise ValueError("q, k, v and d_out must share one dtype (float32 or bfloat16)")
    wsb = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(initial_state), _ptr(d_out), _ptr(d_final_state),
                                _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["d_alpha"]),
                                _ptr(g["d_beta"]), _ptr(g["d_initial_state"]),
                                B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                _ptr(workspace), wsb, _stream(stream))
    _check("kda_chunk_backward", st)
    return g


def backward_phase_workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, chunk: int,
                                  dtype: torch.dtype) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    st = lib.kda_chunk_backward_phase_workspace_size(B, T, H, Dk, Dv, chunk, _DT[dtype],
                                                     ctypes.byref(n))
    _check("kda_chunk_backward_phase_workspace_size", st)
    return n.value


def chunk_backward_phase(q, k, v, alpha, theta, beta, d_out, initial_state=None,
                         d_final_state=None, *, chunk: int = 64, mode: int = CKDA,
                         want_d_initial_state: bool = True, grads=None, workspace=None,
                         stream=None, flags: int = 0):
    """Backward of chunk_forward_phase (kda_chunk_backward_phase): gradients
    with respect to q, k, v, alpha, theta ([B,T,H,Dk/2]), beta and
    initial_state.  Returns a dict dq, dk, dv (q's dtype), d_alpha, d_theta,
    d_beta, d_initial_state (fp32; None unless wanted)."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    g = dict(grads or {})
    g.setdefault("dq", torch.empty((B, T, H, Dk), dtype=q.dtype, device=dev))
    g.setdefault("dk", torch.empty((B, T, H, Dk), dtype=q.dtype, device=dev))
    g.setdefault("dv", torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev))
    g.setdefault("d_alpha", torch.empty((B, T, H, Dk // 2), dtype=torch.float32, device=dev))
    g.setdefault("d_theta", torch.empty((B, T, H, Dk // 2), dtype=torch.float32, device=dev))
    g.setdefault("d_beta", torch.empty((B, T, H), dtype=torch.float32, device=dev))
    if want_d_initial_state:
        g.setdefault("d_initial_state", torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev))
    else:
        g["d_initial_state"] = None
    if workspace is None:
        nbytes = backward_phase_workspace_size(B, T, H, Dk, Dv, chunk, q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _dev(q, k, v, alpha, theta, beta, d_out, initial_state, d_final_state, workspace, *g.values())
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or d_out.dtype != q.dtype:
        raise ValueError("q, k, v and d_out must share one dtype (float32 or bfloat16)")
    wsb = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_backward_phase(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(theta),
                                      _ptr(beta), _ptr(initial_state), _ptr(d_out),
                                      _ptr(d_final_state), _ptr(g["dq"]), _ptr(g["dk"]),
                                      _ptr(g["dv"]), _ptr(g["d_alpha"]), _ptr(g["d_theta"]),
                                      _ptr(g["d_beta"]), _ptr(g["d_initial_state"]),
                                      B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                      _ptr(workspace), wsb, _stream(stream))
    _check("kda_chunk_backward_phase", st)
    return g


def chunk_forward_save(q, k, v, alpha, beta, initial_state=None, *, chunk: int = 64,
                       mode: int = CKDA, out=None, final_state=None, want_final_state: bool = True,
                       saved=None, stream=None, flags: int = 0):
    """kda_chunk_forward_save: the forward of chunk_forward that also leaves in
    `saved` (uint8, backward_workspace_size bytes; allocated when None) what
    chunk_backward_saved needs.  Returns (out, final_state, saved)."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    if saved is None:
        saved = torch.empty(max(backward_workspace_size(B, T, H, Dk, Dv, chunk, q.dtype), 1),
                            dtype=torch.uint8, device=dev)
    _dev(q, k, v, alpha, beta, initial_state, out, final_state, saved)
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype (float32 or bfloat16)")
    st = lib.kda_chunk_forward_save(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(initial_state), _ptr(out), _ptr(final_state),
                                    B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                    _ptr(saved), saved.numel() * saved.element_size(),
                                    _stream(stream))
    _check("kda_chunk_forward_save", st)
    return out, final_state, saved


def chunk_backward_saved(q, k, v, alpha, beta, d_out, saved, d_final_state=None, *,
                         chunk: int = 64, mode: int = CKDA, want_d_initial_state: bool = True,
                         grads=None, stream=None, flags: int = 0):
    """kda_chunk_backward_saved: chunk_backward's gradients from the workspace
    a chunk_forward_save call on the same inputs filled (used up by this
    call).  Returns the dict of chunk_backward."""
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    g = dict(grads or {})
    g.setdefault("dq", torch.empty((B, T, H, Dk), dtype=q.dtype, device=dev))
    g.setdefault("dk", torch.empty((B, T, H, Dk), dtype=q.dtype, device=dev))
    g.setdefault("dv", torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev))
    g.setdefault("d_alpha", torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev))
    g.setdefault("d_beta", torch.empty((B, T, H), dtype=torch.float32, device=dev))
    if want_d_initial_state:
        g.setdefault("d_initial_state", torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev))
    else:
        g["d_initial_state"] = None
    _dev(q, k, v, alpha, beta, d_out, d_final_state, saved, *g.values())
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or d_out.dtype != q.dtype:
        raise ValueError("q, k, v and d_out must share one dtype (float32 or bfloat16)")
    st = lib.kda_chunk_backward_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                      _ptr(d_out), _ptr(d_final_state),
                                      _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                                      _ptr(g["d_alpha"]), _ptr(g["d_beta"]),
                                      _ptr(g["d_initial_state"]),
                                      B, T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags,
                                      _ptr(saved), saved.numel() * saved.element_size(),
                                      _stream(stream))
    _check("kda_chunk_backward_saved", st)
    return g


def chunk_backward_prologue(q_raw, k_raw, v, gate, beta_logit, d_out, initial_state=None,
                            d_final_state=None, *, alpha_min: float, alpha_max: float,
                            beta_max: float, eps: float = 1e-6, normalize_q: bool = True,
                            chunk: int = 64, mode: int = CKDA, want_d_initial_state: bool = True,
                            workspace=None, stream=None, flags: int = 0):
    """Backward of chunk_forward_prologue (kda_chunk_backward_prologue):
    gradients with respect to q_raw, k_raw, v, the gate logits, the beta logits
    and initial_state.  Returns a dict dq, dk, dv (q_raw's dtype), d_gate,
    d_beta_logit, d_initial_state (fp32; None unless wanted)."""
    lib = load()
    B, T, H, Dk = q_raw.shape
    Dv = v.shape[-1]
    dev = q_raw.device
    g = {"dq": torch.empty((B, T, H, Dk), dtype=q_raw.dtype, device=dev),
         "dk": torch.empty((B, T, H, Dk), dtype=q_raw.dtype, device=dev),
         "dv": torch.empty((B, T, H, Dv), dtype=q_raw.dtype, device=dev),
         "d_gate": torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev),
         "d_beta_logit": torch.empty((B, T, H), dtype=torch.float32, device=dev),
         "d_initial_state": (torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
                             if want_d_initial_state else None)}
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check("kda_chunk_backward_prologue_workspace_size",
               lib.kda_chunk_backward_prologue_workspace_size(B, T, H, Dk, Dv, chunk,
                                                               _DT[q_raw.dtype], ctypes.byref(n)))
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    _dev(q_raw, k_raw, v, gate, beta_logit, d_out, initial_state, d_final_state, workspace,
         *g.values())
    if (q_raw.dtype not in _DT or k_raw.dtype != q_raw.dtype or v.dtype != q_raw.dtype
            or d_out.dtype != q_raw.dtype):
        raise ValueError("q_raw, k_raw, v and d_out must share one dtype (float32 or bfloat16)")
    pro = Prologue(alpha_min, alpha_max, beta_max, eps, int(bool(normalize_q)))
    wsb = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_backward_prologue(
        _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(gate), _ptr(beta_logit), _ptr(initial_state),
        _ptr(d_out), _ptr(d_final_state), ctypes.byref(pro), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g["d_gate"]), _ptr(g["d_beta_logit"]), _ptr(g["d_initial_state"]),
        B, T, H, Dk, Dv, chunk, _DT[q_raw.dtype], mode, flags, _ptr(workspace), wsb,
        _stream(stream))
    _check("kda_chunk_backward_prologue", st)
    return g


def chunk_backward_varlen(q, k, v, alpha, beta, cu_seqlens, d_out, initial_state=None,
                          d_final_state=None, *, chunk: int = 64, mode: int = CKDA,
                          want_d_initial_state: bool = True, workspace=None, stream=None,
                          flags: int = 0):
    """Backward of chunk_forward_varlen (kda_chunk_backward_varlen): layouts as
    chunk_forward_varlen, d_out like v, d_final_state [N,H,Dk,Dv] fp32 or None.
    Returns a dict dq, dk, dv (q's dtype, q's / v's shape), d_alpha, d_beta
    (fp32) and d_initial_state ([N,H,Dk,Dv] fp32; None unless wanted)."""
    lib = load()
    H, Dk = q.shape[-2], q.shape[-1]
    total_T = q.shape[-3]
    Dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or N < 1:
        raise ValueError("cu_seqlens must be an int32 tensor of N + 1 offsets, N >= 1")
    dev = q.device
    g = {"dq": torch.empty(q.shape, dtype=q.dtype, device=dev),
         "dk": torch.empty(k.shape, dtype=q.dtype, device=dev),
         "dv": torch.empty(v.shape, dtype=q.dtype, device=dev),
         "d_alpha": torch.empty(alpha.shape, dtype=torch.float32, device=dev),
         "d_beta": torch.empty(beta.shape, dtype=torch.float32, device=dev),
         "d_initial_state": (torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
                             if want_d_initial_state else None)}
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check("kda_chunk_backward_varlen_workspace_size",
               lib.kda_chunk_backward_varlen_workspace_size(N, total_T, H, Dk, Dv, chunk,
                                                             _DT[q.dtype], ctypes.byref(n)))
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    _dev(q, k, v, alpha, beta, cu_seqlens, d_out, initial_state, d_final_state, workspace,
         *g.values())
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype or d_out.dtype != q.dtype:
        raise ValueError("q, k, v and d_out must share one dtype (float32 or bfloat16)")
    st = lib.kda_chunk_backward_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_seqlens), N,
        _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g["d_alpha"]), _ptr(g["d_beta"]), _ptr(g["d_initial_state"]),
        total_T, H, Dk, Dv, chunk, _DT[q.dtype], mode, flags, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("kda_chunk_backward_varlen", st)
    return g


def chunk_backward_varlen_prologue(q_raw, k_raw, v, gate, beta_logit, cu_seqlens, d_out,
                                   initial_state=None, d_final_state=None, *, alpha_min: float,
                                   alpha_max: float, beta_max: float, eps: float = 1e-6,
                                   normalize_q: bool = True, chunk: int = 64, mode: int = CKDA,
                                   want_d_initial_state: bool = True, workspace=None,
                                   stream=None, flags: int = 0):
    """Raw-input backward of a packed batch (kda_chunk_backward_varlen_prologue):
    layouts as chunk_backward_varlen, inputs and parameterisation as
    chunk_backward_prologue.  Returns a dict dq, dk, dv (q_raw's dtype), d_gate,
    d_beta_logit and d_initial_state ([N,H,Dk,Dv] fp32; None unless wanted)."""
    lib = load()
    H, Dk = q_raw.shape[-2], q_raw.shape[-1]
    total_T = q_raw.shape[-3]
    Dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or N < 1:
        raise ValueError("cu_seqlens must be an int32 tensor of N + 1 offsets, N >= 1")
    dev = q_raw.device
    g = {"dq": torch.empty(q_raw.shape, dtype=q_raw.dtype, device=dev),
         "dk": torch.empty(k_raw.shape, dtype=q_raw.dtype, device=dev),
         "dv": torch.empty(v.shape, dtype=q_raw.dtype, device=dev),
         "d_gate": torch.empty(gate.shape, dtype=torch.float32, device=dev),
         "d_beta_logit": torch.empty(beta_logit.shape, dtype=torch.float32, device=dev),
         "d_initial_state": (torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
                             if want_d_initial_state else None)}
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check("kda_chunk_backward_varlen_prologue_workspace_size",
               lib.kda_chunk_backward_varlen_prologue_workspace_size(
                   N, total_T, H, Dk, Dv, chunk, _DT[q_raw.dtype], ctypes.byref(n)))
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=dev)
    _dev(q_raw, k_raw, v, gate, beta_logit, cu_seqlens, d_out, initial_state, d_final_state,
         workspace, *g.values())
    if (q_raw.dtype not in _DT or k_raw.dtype != q_raw.dtype or v.dtype != q_raw.dtype
            or d_out.dtype != q_raw.dtype):
        raise ValueError("q_raw, k_raw, v and d_out must share one dtype (float32 or bfloat16)")
    pro = Prologue(alpha_min, alpha_max, beta_max, eps, int(bool(normalize_q)))
    st = lib.kda_chunk_backward_varlen_prologue(
        _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(gate), _ptr(beta_logit), _ptr(cu_seqlens), N,
        _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), ctypes.byref(pro), _ptr(g["dq"]),
        _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["d_gate"]), _ptr(g["d_beta_logit"]),
        _ptr(g["d_initial_state"]), total_T, H, Dk, Dv, chunk, _DT[q_raw.dtype], mode, flags,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("kda_chunk_backward_varlen_prologue", st)
    return g


def gate_prep(alpha, chunk: int, *, stream=None):
    """Chunk-local gate summary of alpha [B,T,H,Dk] fp32.  Returns (L [B,H,NC,C,Dk] fp32,
    meta [B,H,NC,C,Dk] uint8 = zpos << 1 | parity, gend [B,H,NC,Dk] fp32)."""
    lib = load()
    B, T, H, Dk = alpha.shape
    NC = (T + chunk - 1) // chunk
    L = torch.empty((B, H, NC, chunk, Dk), dtype=torch.float32, device=alpha.device)
    meta = torch.empty((B, H, NC, chunk, Dk), dtype=torch.uint8, device=alpha.device)
    gend = torch.empty((B, H, NC, Dk), dtype=torch.float32, device=alpha.device)
    _dev(alpha, L, meta, gend)
    _check("kda_gate_prep", lib.kda_gate_prep(_ptr(alpha), _ptr(L), _ptr(meta), _ptr(gend),
                                              B, T, H, Dk, chunk, _stream(stream)))
    return L, meta, gend


def last_stage_times():
    """[(kernel name, ms)] of the last call made with flags=STAGE_EVENTS, one
    entry per kernel launch in launch order (a name repeats when a call
    launches that kernel more than once)."""
    lib = load()
    cap = 32
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    n = ctypes.c_int(0)
    _check("kda_last_stage_times", lib.kda_last_stage_times(ms, names, cap, ctypes.byref(n)))
    return [(names[i].decode(), float(ms[i])) for i in range(min(n.value, cap))]
