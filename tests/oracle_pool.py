"""Whole-output parity at full size on the host cores.

The fp64 oracle (``oracle.ssd_recurrent``) is run over every (batch, head)
chain of a workload, or a chosen subset, in a pool of worker processes. Each
task takes one batch element and a block of heads, computes the oracle on
them, compares with the GPU's y and final state for the same chains, and
returns only the error maxima, so the parent combines them into the global
per-tensor measures of the tolerance bar:

  y            max|y_gpu - y_ref|                        / max|y_ref|
  ssm part     max(|y_gpu - y_ref| - out_eps |y_ref|, 0) / max|y_ref - D x|
  final state  max|hT_gpu - hT_ref|                      / max|hT_ref|

This module imports numpy and the oracle only, so spawned workers start
quickly and never touch the GPU. The pool has at most 16 workers.
"""

from __future__ import annotations

import atexit
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

from oracle import ssd_recurrent

_POOL = None


def pool_size() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ProcessPoolExecutor(max_workers=pool_size(), mp_context=mp.get_context("spawn"))
        atexit.register(_POOL.shutdown, wait=False, cancel_futures=True)
    return _POOL


def _task(args):
    x, dt, A, B, C, D, h0, y_gpu, h_gpu, out_eps = args
    y_ref, h_ref = ssd_recurrent(x[None], dt[None], A, B[None], C[None], D, None if h0 is None else h0[None])
    y_ref, h_ref = y_ref[0], h_ref[0]
    y_gpu = y_gpu.astype(np.float64)
    diff = np.abs(y_gpu - y_ref)
    ssm = y_ref if D is None else y_ref - D.astype(np.float64)[None, :, None] * x.astype(np.float64)
    out = {
        "y_err": float(diff.max()),
        "y_ref": float(np.abs(y_ref).max()),
        "ssm_excess": float(np.maximum(diff - out_eps * np.abs(y_ref), 0.0).max()),
        "ssm_ref": float(np.abs(ssm).max()),
        "finite": bool(np.isfinite(y_gpu).all()),
    }
    if h_gpu is not None:
        h_gpu = h_gpu.astype(np.float64)
        out["h_err"] = float(np.abs(h_gpu - h_ref).max())
        out["h_ref"] = float(np.abs(h_ref).max())
        out["finite"] = out["finite"] and bool(np.isfinite(h_gpu).all())
    return out


def head_blocks(H: int, G: int, block: int):
    """Contiguous head blocks [h0, h1) that either lie inside one B/C group or
    cover whole groups, so the block's heads map onto the sliced groups with
    the same contiguous rule (g = h // (heads per group))."""
    hpg = H // G
    step = block if hpg % block == 0 or block % hpg == 0 else hpg
    step = min(step, H)
    return [(h0, min(h0 + step, H)) for h0 in range(0, H, step)]


def compare_all(inp: dict, y, hT, out_eps: float, batches=None, heads=None, block: int = 16) -> dict:
    """Oracle vs GPU over the chains of ``batches`` (default all) x ``heads``
    (default all), heads taken in contiguous blocks. ``inp`` holds the CPU
    input tensors (torch or numpy), ``y`` and ``hT`` the GPU outputs copied to
    the host. Returns the global error measures and the chain count."""
    to_np = _to_numpy
    x, dt, A, Bm, Cm = (to_np(inp[k]) for k in ("x", "dt", "A", "B", "C"))
    D = None if inp["D"] is None else to_np(inp["D"])
    h0 = None if inp["init_state"] is None else to_np(inp["init_state"])
    yg = to_np(y)
    hg = None if hT is None else to_np(hT)
    bsz, L, H, P = x.shape
    G = Bm.shape[2]
    hpg = H // G
    batches = range(bsz) if batches is None else batches
    blocks = head_blocks(H, G, block)
    if heads is not None:
        keep = set(heads)
        blocks = [(a, e) for a, e in blocks if any(a <= h < e for h in keep)]
    tasks = []
    for b in batches:
        for a, e in blocks:
            ga, ge = a // hpg, (e - 1) // hpg + 1
            tasks.append((x[b, :, a:e], dt[b, :, a:e], A[a:e], Bm[b, :, ga:ge], Cm[b, :, ga:ge],
                           None if D is None else D[a:e], None if h0 is None else h0[b, a:e],
                           yg[b, :, a:e], None if hg is None else hg[b, a:e], out_eps))
    res = list(_pool().map(_task, tasks))
    agg = {
        "y": max(r["y_err"] for r in res) / max(max(r["y_ref"] for r in res), 1e-30),
        "ssm": max(r["ssm_excess"] for r in res) / max(max(r["ssm_ref"] for r in res), 1e-30),
        "finite": all(r["finite"] for r in res),
        "chains": sum((e - a) for a, e in blocks) * len(list(batches)),
    }
    if hg is not None:
        agg["final_state"] = max(r["h_err"] for r in res) / max(max(r["h_ref"] for r in res), 1e-30)
    return agg


def compare_packed(inp: dict, cu, y, hT, out_eps: float, init_states=None, block: int = 16) -> dict:
    """compare_all for packed sequences: ``inp`` holds [1, T, ...] inputs,
    ``cu`` the S + 1 offsets, ``y`` [1, T, H, P] and ``hT`` [S, H, P, N] the
    GPU outputs, ``init_states`` [S, H, P, N] or None. Every (sequence, head)
    chain runs the oracle recurrence on its own tokens; an empty sequence's
    final state must equal its initial state (zeros without one) exactly."""
    to_np = _to_numpy
    x, dt, Bm, Cm = (to_np(inp[k])[0] for k in ("x", "dt", "B", "C"))
    A = to_np(inp["A"])
    D = None if inp["D"] is None else to_np(inp["D"])
    h0 = None if init_states is None else to_np(init_states)
    yg = to_np(y)[0]
    hg = None if hT is None else to_np(hT)
    cu = [int(v) for v in cu]
    T, H, P = x.shape
    G = Bm.shape[1]
    hpg = H // G
    blocks = head_blocks(H, G, block)
    tasks, empty_ok = [], True
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        if e == a:
            if hg is not None:
                want = np.zeros_like(hg[s]) if h0 is None else h0[s]
                empty_ok = empty_ok and np.array_equal(hg[s], want)
            continue
        for ha, he in blocks:
            ga, ge = ha // hpg, (he - 1) // hpg + 1
            tasks.append((x[a:e, ha:he], dt[a:e, ha:he], A[ha:he], Bm[a:e, ga:ge], Cm[a:e, ga:ge],
                          None if D is None else D[ha:he], None if h0 is None else h0[s, ha:he],
                          yg[a:e, ha:he], None if hg is None else hg[s, ha:he], out_eps))
    res = list(_pool().map(_task, tasks))
    agg = {
        "y": max(r["y_err"] for r in res) / max(max(r["y_ref"] for r in res), 1e-30),
        "ssm": max(r["ssm_excess"] for r in res) / max(max(r["ssm_ref"] for r in res), 1e-30),
        "finite": all(r["finite"] for r in res),
        "chains": sum(1 for s in range(len(cu) - 1) if cu[s + 1] > cu[s]) * H,
        "empty_ok": empty_ok,
    }
    if hg is not None:
        agg["final_state"] = max(r["h_err"] for r in res) / max(max(r["h_ref"] for r in res), 1e-30)
    return agg


def _to_numpy(t):
    if isinstance(t, np.ndarray):
        return t
    t = t.detach().cpu()
    if str(t.dtype) == "torch.bfloat16":
        t = t.float()  # exact: every bf16 value is an fp32 value
    return t.numpy()
