"""Seeded synthetic inputs for the KDA / CKDA workloads.

This module is shared by the tests, the smoke check and the benchmark, and it
feeds the HIP library and the CPU oracle the *same* tensors.  It holds none of
the recurrence's arithmetic: it only draws random numbers, normalises keys and
queries per token (an input property the workloads ask for), maps normals to
gates and step sizes, and casts.

Workloads (H = heads, D = d_k = d_v, C = chunk length):
  0  KDA fp32 tiny        B=1   H=1  T=64     D=16  C=16
  1  CKDA fp32            B=2   H=4  T=1024   D=64  C=64
  2  KDA bf16 prefill     B=1   H=32 T=8192   D=128 C=64
  3  CKDA bf16 long ctx   B=1   H=16 T=65536  D=128 C=64   S0 ~ N(0, 0.02^2)
  4  CKDA bf16 decode     B=256 H=32 D=128, 1000 single-token steps, resident
                          fp32 state ~ N(0, 0.02^2) updated in place

Recipes.  q, k ~ N(0,1) then L2-normalised per token in fp32, then cast; v ~
N(0,1) cast.  KDA gate alpha = exp(-softplus(x)), x ~ N(0,1) per element, so
alpha in (0,1); KDA beta = sigmoid(N(0,1)).  CKDA gate alpha = s * exp(-softplus
(x)) with s = -1 with probability 0.3, then each element independently set to
exactly -1 with probability 0.01 or exactly 0 with probability 0.01 (mutually
exclusive); CKDA beta = 2 sigmoid(N(0,1)), each (t, h) set to exactly 2 with
probability 0.01.  Workload i uses seed i.  Draw order: q, k, v, x, sign,
gate-special, beta-normal, beta-special, S0.  The decode workload draws its
initial state first and then the stacked per-step inputs in the same order.

The pages train and evaluate on public corpora and synthetic state-tracking
tasks; none of those are used or needed: these seeded tensors stand in for
them at the pages' head geometry.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

KDA, CKDA = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int
    chunk: int
    dtype: torch.dtype
    mode: int
    s0_std: float | None
    seed: int
    steps: int = 0          # decode workloads: number of single-token steps

    @property
    def Dk(self) -> int:
        return self.D

    @property
    def Dv(self) -> int:
        return self.D


WORKLOADS = {
    0: Workload("kda_fp32_tiny", 1, 1, 64, 16, 16, torch.float32, KDA, None, 0),
    1: Workload("ckda_fp32", 2, 4, 1024, 64, 64, torch.float32, CKDA, None, 1),
    2: Workload("kda_bf16_prefill", 1, 32, 8192, 128, 64, torch.bfloat16, KDA, None, 2),
    3: Workload("ckda_bf16_long_ctx", 1, 16, 65536, 128, 64, torch.bfloat16, CKDA, 0.02, 3),
    4: Workload("ckda_bf16_decode", 256, 32, 1, 128, 0, torch.bfloat16, CKDA, 0.02, 4,
                steps=1000),
}


def workload(i: int, **overrides) -> Workload:
    """Workload i, optionally with fields replaced (e.g. T=67 for a ragged tail)."""
    return replace(WORKLOADS[i], **overrides) if overrides else WORKLOADS[i]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(shape, g, device, dtype):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    return x.to(dtype)


def _gates(shape, mode, g, device):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    a = torch.exp(-torch.nn.functional.softplus(x))
    if mode == CKDA:
        s = torch.rand(shape, generator=g, device=device) < 0.3
        a = torch.where(s, -a, a)
        u = torch.rand(shape, generator=g, device=device)
        a = torch.where(u < 0.01, torch.full_like(a, -1.0), a)
        a = torch.where((u >= 0.01) & (u < 0.02), torch.zeros_like(a), a)
    return a.contiguous()


def _betas(shape, mode, g, device):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    b = torch.sigmoid(x)
    if mode == CKDA:
        b = 2.0 * b
        u = torch.rand(shape, generator=g, device=device)
        b = torch.where(u < 0.01, torch.full_like(b, 2.0), b)
    return b.contiguous()


def make_prefill(w: Workload, device="cpu", seed: int | None = None):
    """Inputs for a chunked forward: dict of q, k, v ([B,T,H,D], w.dtype),
    alpha ([B,T,H,D] fp32), beta ([B,T,H] fp32), S0 ([B,H,D,D] fp32 or None)."""
    g = _gen(w.seed if seed is None else seed, device)
    B, T, H, D = w.B, w.T, w.H, w.D
    q = _unit_rows((B, T, H, D), g, device, w.dtype)
    k = _unit_rows((B, T, H, D), g, device, w.dtype)
    v = torch.randn((B, T, H, D), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    alpha = _gates((B, T, H, D), w.mode, g, device)
    beta = _betas((B, T, H), w.mode, g, device)
    S0 = None
    if w.s0_std is not None:
        S0 = (w.s0_std * torch.randn((B, H, D, D), generator=g, device=device,
                                     dtype=torch.float32)).contiguous()
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "alpha": alpha, "beta": beta, "S0": S0}


def make_prefill_raw(w: Workload, device="cpu", seed: int | None = None, gate_std: float = 2.0,
                     forget_frac: float = 0.0):
    """Raw inputs for the forward with the fused input parameterisation: q, k
    N(0,1) per element (not normalised) and v N(0,1), all rounded to w.dtype;
    gate logits N(0, gate_std^2) fp32 [B,T,H,D], with a fraction forget_frac
    of them set to -200 (a gate of 0 after any range-sigmoid with alpha_min =
    0); beta logits N(0,1) fp32 [B,T,H]; S0 as in make_prefill."""
    g = _gen(w.seed if seed is None else seed, device)
    B, T, H, D = w.B, w.T, w.H, w.D
    f32 = torch.float32
    q = torch.randn((B, T, H, D), generator=g, device=device, dtype=f32).to(w.dtype)
    k = torch.randn((B, T, H, D), generator=g, device=device, dtype=f32).to(w.dtype)
    v = torch.randn((B, T, H, D), generator=g, device=device, dtype=f32).to(w.dtype)
    gate = gate_std * torch.randn((B, T, H, D), generator=g, device=device, dtype=f32)
    if forget_frac > 0:
        u = torch.rand((B, T, H, D), generator=g, device=device)
        gate = torch.where(u < forget_frac, torch.full_like(gate, -200.0), gate)
    blog = torch.randn((B, T, H), generator=g, device=device, dtype=f32)
    S0 = None
    if w.s0_std is not None:
        S0 = (w.s0_std * torch.randn((B, H, D, D), generator=g, device=device,
                                     dtype=f32)).contiguous()
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "gate": gate.contiguous(), "beta_logit": blog.contiguous(), "S0": S0}


def make_varlen(w: Workload, lengths, device="cpu", seed: int | None = None):
    """A packed batch of len(lengths) sequences (w.B is ignored): the inputs of
    make_prefill for B = 1, T = sum(lengths), plus cu_seqlens (int32 [N+1])
    and, when w.s0_std is set, one initial state per sequence [N,H,D,D]."""
    total = int(sum(lengths))
    inp = make_prefill(replace(w, B=1, T=total, s0_std=None), device=device, seed=seed)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    inp["cu_seqlens"] = cu.to(device)
    inp["S0"] = None
    if w.s0_std is not None:
        g = _gen((w.seed if seed is None else seed) + 1000, device)
        inp["S0"] = (w.s0_std * torch.randn((len(lengths), w.H, w.D, w.D), generator=g,
                                            device=device, dtype=torch.float32)).contiguous()
    return inp


def make_prefill_phase(w: Workload, theta_max: float = 3.0, device="cpu", seed: int | None = None):
    """Inputs of the phase variant: those of make_prefill, except alpha, now
    one gate per channel pair [B,T,H,D/2] (drawn like make_prefill's gates),
    plus phases theta = theta_max * tanh(x), x ~ N(0,1), [B,T,H,D/2] fp32."""
    inp = make_prefill(w, device=device, seed=seed)
    g = _gen((w.seed if seed is None else seed) + 2000, device)
    B, T, H, D = w.B, w.T, w.H, w.D
    inp["alpha"] = _gates((B, T, H, D // 2), w.mode, g, device)
    inp["theta"] = (theta_max * torch.tanh(torch.randn((B, T, H, D // 2), generator=g,
                                                       device=device, dtype=torch.float32))).contiguous()
    return inp


def make_backward_seeds(w: Workload, device="cpu", seed: int | None = None, dst: bool = True):
    """Loss gradients for a backward pass: dO [B,T,H,D] ~ N(0,1) in w.dtype and
    dST [B,H,D,D] ~ N(0,1) fp32 (None unless dst), from seed w.seed + 1000 (so
    the forward inputs of the same workload are unchanged).  Draw order: dO,
    dST."""
    g = _gen((w.seed if seed is None else seed) + 1000, device)
    B, T, H, D = w.B, w.T, w.H, w.D
    dO = torch.randn((B, T, H, D), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    dST = None
    if dst:
        dST = torch.randn((B, H, D, D), generator=g, device=device, dtype=torch.float32)
    return dO.contiguous(), dST


def make_decode(w: Workload, steps: int | None = None, device="cpu", seed: int | None = None):
    """Inputs for stacked decode steps: S0 [B,H,D,D] fp32, then per step
    q, k, v [N,B,H,D] (w.dtype), alpha [N,B,H,D] fp32, beta [N,B,H] fp32."""
    g = _gen(w.seed if seed is None else seed, device)
    N = w.steps if steps is None else steps
    B, H, D = w.B, w.H, w.D
    S0 = ((w.s0_std or 0.0) * torch.randn((B, H, D, D), generator=g, device=device,
                                          dtype=torch.float32)).contiguous()
    q = _unit_rows((N, B, H, D), g, device, w.dtype)
    k = _unit_rows((N, B, H, D), g, device, w.dtype)
    v = torch.randn((N, B, H, D), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    alpha = _gates((N, B, H, D), w.mode, g, device)
    beta = _betas((N, B, H), w.mode, g, device)
    return {"S0": S0, "q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "alpha": alpha, "beta": beta}
