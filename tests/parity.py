"""Helpers for GPU-vs-oracle parity tests (test-side only).

Error measure (the pages state no precision; this is the reading the tests
use): for every (b, h) slice separately, max |gpu - oracle| / max |oracle| over
that slice's outputs (T x Dv) and, separately, over its final state
(Dk x Dv); the test bound applies to the largest such ratio.  fp32 workloads
must stay within 1e-4, bf16 workloads within 2e-2.

For information only, the same calls also record the elementwise relative
error max |gpu - oracle| / max(|oracle|, 1e-3 max |oracle|) (the floor keeps
entries near zero from dominating), per slice and maximised over slices;
elem_note() formats the latest pair for the test log.
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


ELEM = {"out": None, "state": None}


def _slice_errs(g, r):
    """(normwise, elementwise) relative error of one slice."""
    ar = np.abs(r)
    den = ar.max()
    diff = np.abs(g - r)
    num = diff.max()
    if den == 0:
        return num, num
    return num / den, (diff / np.maximum(ar, 1e-3 * den)).max()


def slice_err_out(gpu, ref):
    """gpu, ref: [B,T,H,Dv] -> max over (b,h) of normwise max error."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    worst = welem = 0.0
    for b in range(r.shape[0]):
        for h in range(r.shape[2]):
            n, e = _slice_errs(g[b, :, h], r[b, :, h])
            worst, welem = max(worst, n), max(welem, e)
    ELEM["out"] = welem
    return worst


def slice_err_state(gpu, ref):
    """[B,H,Dk,Dv] -> max over (b,h) of normwise max error."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    worst = welem = 0.0
    for b in range(r.shape[0]):
        for h in range(r.shape[1]):
            n, e = _slice_errs(g[b, h], r[b, h])
            worst, welem = max(worst, n), max(welem, e)
    ELEM["state"] = welem
    return worst


def elem_note():
    """The latest elementwise errors (information only, not asserted)."""
    f = lambda x: "-" if x is None else f"{x:.3e}"
    return f" (elementwise, floor 1e-3 max: out {f(ELEM['out'])} state {f(ELEM['state'])})"


def oracle_threads():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))
