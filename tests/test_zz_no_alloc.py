"""The no-allocation entry point (ssd_forward_noalloc) against ssd_forward.

ssd_forward_noalloc runs ssd_forward's kernels with the workspace taken from
the library's fixed per-GPU scratch array. Two calls in a row, the second on
a smaller problem than the first (the scratch keeps the first call's
contents, so whatever must start at zero has to be cleared by the second
call itself), must each give ssd_forward's y and final state bit for bit:
the first on the one-pass path (the headline layer at batch 16: two rounds
of workgroups, hand-over counters in the scratch), the second on the split
path. A third call on a problem larger than the scratch returns
SSD_ERR_SCRATCH_LIMIT and writes nothing.
"""

import pytest
import torch

from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import note

pytestmark = pytest.mark.gpu

DEV = "cuda"


def ssd():
    import mamba_ssd_scan_fwd_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def both(cfg, seed):
    lib = ssd()
    inp = make_inputs(cfg, seed=seed)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    args = [d[k] for k in ("x", "dt", "A", "B", "C", "D", "init_state")]
    desc = lib.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.io_dtype)
    ws = torch.empty(lib.workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    y_ref, h_ref = lib.forward(*args, workspace=ws)
    path, status = lib.workspace_status(desc, ws)
    y = torch.full_like(y_ref, float("nan"))
    h = torch.full_like(h_ref, float("nan"))
    lib.forward_noalloc(*args, y=y, final_state=h)
    torch.cuda.synchronize()
    return (y, h), (y_ref, h_ref), path, status


def test_no_allocation_entry_matches_ssd_forward_on_two_calls():
    big = CONFIGS[1].with_(batch=16)  # two rounds of workgroups: ssd_forward takes the one-pass path
    small = CONFIGS[1].with_(batch=2, seqlen=700, nheads=8, init_state=True)
    for cfg, want in ((big, "one-pass"), (small, "split")):
        note(f"[gpu] no-allocation entry: B={cfg.batch} L={cfg.seqlen} H={cfg.nheads}")
        (y, h), (y_ref, h_ref), path, status = both(cfg, seed=cfg.batch + 7)
        assert (path, status) == (want, 0)
        assert torch.equal(y, y_ref), "y differs from ssd_forward"
        assert torch.equal(h, h_ref), "final state differs from ssd_forward"


def test_no_allocation_entry_rejects_a_problem_larger_than_its_scratch():
    lib = ssd()
    cfg = CONFIGS[3].with_(seqlen=4096)  # 4 x 4096, 128 heads, N = 256: 272 MiB of workspace
    desc = lib.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.io_dtype)
    assert lib.workspace_bytes(desc) > (256 << 20)
    inp = make_inputs(cfg, seed=9)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y = torch.full_like(d["x"], 7.0)
    note("[gpu] no-allocation entry: a problem larger than the scratch")
    with pytest.raises(lib.SSDError, match="SCRATCH_LIMIT"):
        lib.forward_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None, y=y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "the rejected call wrote to y"
