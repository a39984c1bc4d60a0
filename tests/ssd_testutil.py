"""Helpers shared by the GPU parity tests: oracle on sampled heads, error
metrics, tolerance bar.

Tolerance bar (per output tensor, global): max|got - ref| <= tol * max|ref|
with tol = 2e-2 for bf16 inputs (bf16 operands, fp32 accumulation) and
tol = 1e-4 for the fp32 io dtype. The same bar applies to y and to the final
state, each against its own maximum.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import ssd_recurrent

TOL = {"bf16": 2e-2, "fp32": 1e-4, torch.bfloat16: 2e-2, torch.float32: 1e-4}


def np64(t):
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def note(msg: str):
    """Print and flush a progress line naming the case about to run on the GPU."""
    print(msg, file=sys.stderr, flush=True)


def oracle_sampled(inp: dict, pairs):
    """Oracle outputs for selected (b, h) pairs over the full sequence.

    Slices each head with its own B/C group (one group per sampled head) and
    runs the fp64 recurrence. Returns {(b, h): (y [L, P], hT [P, N])}.
    """
    x, dt, A, B, C, D, h0 = (inp[k] for k in ("x", "dt", "A", "B", "C", "D", "init_state"))
    H = x.shape[2]
    G = B.shape[2]
    by_b = {}
    for b, h in pairs:
        by_b.setdefault(b, []).append(h)
    out = {}
    for b, hs in by_b.items():
        gs = [h // (H // G) for h in hs]
        xs = np64(x[b:b + 1, :, hs])
        dts = np64(dt[b:b + 1, :, hs])
        As = np64(A[hs])
        Bs = np64(B[b:b + 1, :, gs])
        Cs = np64(C[b:b + 1, :, gs])
        Ds = None if D is None else np64(D[hs])
        h0s = None if h0 is None else np64(h0[b:b + 1, hs])
        y, hT = ssd_recurrent(xs, dts, As, Bs, Cs, Ds, h0s)
        for k, h in enumerate(hs):
            out[(b, h)] = (y[0, :, k], hT[0, k])
    return out


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / max(scale, 1e-30)


OUT_EPS = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -23}


def check_ssm_part(y_got, y_ref, dx, tol, what, out_eps):
    """The bar applied to the state-space part y - D x, against its own
    maximum. The skip term D x can dominate max|y| and would otherwise hide
    errors in the state-space part; y itself is stored in the io dtype, so
    each element may also carry one rounding of |y_ref| * out_eps."""
    y_got = np.asarray(y_got, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    ssm = y_ref - (0.0 if dx is None else np.asarray(dx, np.float64))
    excess = np.maximum(np.abs(y_got - y_ref) - out_eps * np.abs(y_ref), 0.0)
    e = float(np.max(excess)) / max(float(np.max(np.abs(ssm))), 1e-30)
    note(f"    {what} (ssm part, beyond output rounding): {e:.3e} (bar {tol:.0e})")
    assert e <= tol, f"{what}: state-space part error {e:.3e} > {tol:.0e}"
    return e


def check_rel(got, ref, tol, what):
    e = rel_err(got, ref)
    note(f"    {what}: max|err|/max|ref| = {e:.3e} (bar {tol:.0e})")
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: relative error {e:.3e} > {tol:.0e}"
    return e
