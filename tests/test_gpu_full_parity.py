"""Whole-output GPU parity at the workloads' full sizes.

Every (batch, head) chain of every bf16 workload, at its full size and in the
launch configuration the benchmark times, is compared element by element with
the fp64 oracle recurrence (computed on the host cores by a pool of worker
processes, tests/oracle_pool.py): y, its state-space part y - D x, and the
final state, each to the tolerance bar (max|err| <= 2e-2 max|ref| per output
tensor). Both forward paths are covered on the shapes where each runs:
ssd_forward's own choice (split, split with segmented state passing, or the
one-pass kernel over several rounds of workgroups), and the other path forced
through ssd_forward_split / ssd_forward_fused. After every call the status
record the call left in its workspace (ssd_workspace_status) must report the
expected path and no cut-off wait or incomplete hand-over chain.

The blocked algorithm these paths implement computes per-chunk states in
parallel and recombines them ("Mamba-2 vs Transformers: SSMs, structured state
space duality", section "Mamba-2 and the SSD paper: what changed in
practice"); the oracle is the plain recurrence of the same operator.
"""

import pytest
import torch

from oracle_pool import compare_all
from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import OUT_EPS, TOL, note

pytestmark = pytest.mark.gpu

DEV = "cuda"


def ssd():
    import mamba_ssd_scan_fwd_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def run_recorded(cfg, inp, entry):
    """One forward call with a caller-owned workspace; returns y and the final
    state on the host plus the (path, status) the call recorded."""
    lib = ssd()
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    desc = lib.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.io_dtype)
    ws = torch.empty(lib.workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    kw = {"fused": entry == "fused", "split": entry == "split"}
    y, hT = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], workspace=ws, **kw)
    path, status = lib.workspace_status(desc, ws)
    torch.cuda.synchronize()
    out = (y.cpu(), hT.cpu(), path, status)
    del d, y, hT, ws
    torch.cuda.empty_cache()
    return out


# (workload index, batch override, entry point, path the call must take,
#  heads per oracle task)
FULL = [
    (1, None, "auto", "split", 16),            # the headline: split path, one round
    (1, None, "fused", "one-pass", 16),        # the headline through the one-pass kernel
    (1, 32, "fused", "one-pass", 16),          # headline layer at batch 32: several rounds
    (1, 32, "split", "split", 16),
    (2, None, "auto", "split-segmented", 4),   # one 64K-token sequence: segmented state passing
    (2, None, "fused", "one-pass", 4),         # 64 chains of 256 chunks in the one-pass kernel
    (3, None, "auto", "split", 16),            # N = 256, 8 groups
    (4, None, "auto", "one-pass", 16),         # 32 x 4096, N = 64: ssd_forward takes the one-pass path
    (4, None, "split", "split", 16),
]


@pytest.mark.parametrize("idx,batch,entry,path,block", FULL,
                         ids=[f"{CONFIGS[i].name}-b{b or CONFIGS[i].batch}-{e}" for i, b, e, _, _ in FULL])
def test_every_chain_at_full_size(idx, batch, entry, path, block):
    cfg = CONFIGS[idx] if batch is None else CONFIGS[idx].with_(batch=batch)
    inp = make_inputs(cfg, seed=idx)
    note(f"[gpu] full size, every chain: {cfg.name} B={cfg.batch} L={cfg.seqlen} H={cfg.nheads} "
         f"P={cfg.headdim} N={cfg.dstate} G={cfg.ngroups} entry={entry}")
    y, hT, got_path, status = run_recorded(cfg, inp, entry)
    note(f"    path {got_path}, status {status}")
    assert got_path == path, f"took the {got_path} path, expected {path}"
    assert status == 0, f"the call's status record reports {status:#x}"
    tol = TOL[cfg.io_dtype]
    r = compare_all(inp, y, hT, OUT_EPS[cfg.io_dtype], block=block)
    note(f"    {r['chains']} chains: y {r['y']:.3e}, ssm part {r['ssm']:.3e}, final state "
         f"{r['final_state']:.3e} (bar {tol:.0e})")
    assert r["chains"] == cfg.batch * cfg.nheads
    assert r["finite"], "non-finite output"
    assert r["y"] <= tol and r["ssm"] <= tol and r["final_state"] <= tol, r


def test_status_record_of_each_path():
    """The record names the path each entry point took, and reads clean, on
    small shapes of each path (the long-chain shape takes the segmented state
    passing)."""
    lib = ssd()
    cases = [(CONFIGS[1].with_(batch=2, seqlen=1100), "split", "split"),
             (CONFIGS[1].with_(batch=2, seqlen=1100), "fused", "one-pass"),
             (CONFIGS[1].with_(batch=1, seqlen=70 * 256 + 5, nheads=4, init_state=True), "auto", "split-segmented"),
             (CONFIGS[0], "auto", "split")]
    for cfg, entry, path in cases:
        inp = make_inputs(cfg, seed=3)
        note(f"[gpu] status record: {cfg.name} B={cfg.batch} L={cfg.seqlen} entry={entry}")
        _, _, got, status = run_recorded(cfg, inp, entry)
        assert (got, status) == (path, 0), (got, status)
    # a workspace no forward call has written: no record
    cfg = CONFIGS[1].with_(batch=2, seqlen=1100)
    desc = lib.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.io_dtype)
    ws = torch.zeros(lib.workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    assert lib.workspace_status(desc, ws) == ("none", lib.STATUS_NO_RECORD)
