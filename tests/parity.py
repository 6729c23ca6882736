"""Helpers for GPU-vs-oracle parity tests (test-side only).

Error measure (the pages state no precision; this is the reading the tests
use): for every (b, h) slice separately, max |gpu - oracle| / max |oracle| over
that slice's outputs (T x Dv) and, separately, over its final state
(Dk x Dv); the test bound applies to the largest such ratio.  fp32 workloads
must stay within 1e-4, bf16 workloads within 2e-2.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def np32(t):
    return t.detach().float().cpu().numpy()


def slice_err_out(gpu, ref):
    """gpu, ref: [B,T,H,Dv] -> max over (b,h) of normwise max error."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for b in range(r.shape[0]):
        for h in range(r.shape[2]):
            den = np.abs(r[b, :, h]).max()
            num = np.abs(g[b, :, h] - r[b, :, h]).max()
            worst = max(worst, num / den if den > 0 else num)
    return worst


def slice_err_state(gpu, ref):
    """[B,H,Dk,Dv] -> max over (b,h) of normwise max error."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for b in range(r.shape[0]):
        for h in range(r.shape[1]):
            den = np.abs(r[b, h]).max()
            num = np.abs(g[b, h] - r[b, h]).max()
            worst = max(worst, num / den if den > 0 else num)
    return worst


def oracle_threads():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))
