"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every case draws seeded synthetic inputs (ssd_inputs), runs the library on
the GPU, and compares element by element with the oracle on the same inputs:
  * the small fp32 workload in full;
  * each bf16 workload at reduced batch/length (several chunks and a ragged
    tail) and at its full size in the launch configuration the benchmark
    times, both on sampled (batch, head) pairs over the whole sequence;
  * edge shapes (L = 1, L < Q, L = Q +- 1, every P, N, group layout, chunk
    length, both io dtypes) in full;
  * API options (no D, no/zero initial state, no final state, in-place state,
    library-allocated workspace, a non-default stream);
  * hygiene: every output element written, guard bands intact, bitwise
    run-to-run determinism;
  * each step of the chunked path on its own against the oracle's definition
    of that step's output.
"""

import numpy as np
import pytest
import torch

from oracle import chunk_cumsum as o_cumsum
from oracle import chunk_entry_states as o_entry
from oracle import chunk_local_states as o_local
from oracle import ssd_recurrent
from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import OUT_EPS, TOL, check_rel, check_ssm_part, note, np64, oracle_sampled

pytestmark = pytest.mark.gpu

DEV = "cuda"


def ssd():
    import mamba_ssd_scan_fwd_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def to_dev(inp):
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


def run(inp, **kw):
    d = to_dev(inp)
    y, hT = ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], **kw)
    torch.cuda.synchronize()
    return y.cpu(), (hT.cpu() if hT is not None else None)


def full_check(inp, tol, tag, **kw):
    note(f"[gpu] {tag}: x{tuple(inp['x'].shape)} B{tuple(inp['B'].shape)} {inp['x'].dtype} {kw}")
    y, hT = run(inp, **kw)
    yr, hr = ssd_recurrent(*(np64(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    check_rel(np64(y), yr, tol, f"{tag} y")
    io = "bf16" if inp["x"].dtype == torch.bfloat16 else "fp32"
    dx = None if inp["D"] is None else np64(inp["x"]) * np64(inp["D"])[:, None]
    check_ssm_part(np64(y), yr, dx, tol, f"{tag} y", OUT_EPS[io])
    if hT is not None:
        check_rel(np64(hT), hr, tol, f"{tag} final_state")
    return y, hT


def sampled_check(inp, pairs, tol, tag, **kw):
    note(f"[gpu] {tag}: x{tuple(inp['x'].shape)} B{tuple(inp['B'].shape)} {inp['x'].dtype} pairs={pairs}")
    y, hT = run(inp, **kw)
    ref = oracle_sampled(inp, pairs)
    yg = np.stack([np64(y[b, :, h]) for b, h in pairs])
    yo = np.stack([ref[p][0] for p in pairs])
    ey = check_rel(yg, yo, tol, f"{tag} y (sampled)")
    dx = None
    if inp["D"] is not None:
        xs = np.stack([np64(inp["x"][b, :, h]) for b, h in pairs])
        dx = np.array([float(inp["D"][h]) for b, h in pairs])[:, None, None] * xs
    io = "bf16" if inp["x"].dtype == torch.bfloat16 else "fp32"
    check_ssm_part(yg, yo, dx, tol, f"{tag} y (sampled)", OUT_EPS[io])
    eh = check_rel(np.stack([np64(hT[b, h]) for b, h in pairs]),
                   np.stack([ref[p][1] for p in pairs]), tol, f"{tag} final_state (sampled)")
    assert torch.isfinite(y.float()).all() and torch.isfinite(hT).all()
    return ey, eh


def pairs_for(cfg, n=3):
    b, H = cfg.batch, cfg.nheads
    cand = [(0, 0), (b - 1, H - 1), (b // 2, H // 2 + 1 if H > 2 else 0), (0, H // 3)]
    out = []
    for p in cand:
        if p not in out:
            out.append(p)
    return out[:n]


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def test_tiny_fp32_workload_in_full():
    cfg = CONFIGS[0]
    full_check(make_inputs(cfg, seed=0), TOL["fp32"], cfg.name)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_workloads_reduced_length(idx):
    cfg = CONFIGS[idx]
    small = cfg.with_(batch=min(cfg.batch, 2), seqlen=2 * 256 + 77)
    inp = make_inputs(small, seed=100 + idx)
    sampled_check(inp, pairs_for(small, 4), TOL[cfg.io_dtype], f"{cfg.name} reduced")


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_workloads_full_size(idx):
    cfg = CONFIGS[idx]
    inp = make_inputs(cfg, seed=idx)
    sampled_check(inp, pairs_for(cfg, 3), TOL[cfg.io_dtype], f"{cfg.name} full size")


@pytest.mark.parametrize("idx,batch", [(4, None), (1, 32)])
def test_split_entry_full_size_where_forward_takes_one_pass(idx, batch):
    """ssd_forward takes the one-pass kernel on these shapes (several rounds
    of workgroups); ssd_forward_split runs the separate steps on them."""
    cfg = CONFIGS[idx] if batch is None else CONFIGS[idx].with_(name=f"{CONFIGS[idx].name} batch {batch}", batch=batch)
    inp = make_inputs(cfg, seed=40 + idx)
    sampled_check(inp, pairs_for(cfg, 3), TOL[cfg.io_dtype], f"{cfg.name} split entry", split=True)


def test_split_entry_is_what_forward_runs_on_the_headline():
    cfg = CONFIGS[1]
    inp = make_inputs(cfg, seed=41)
    note("[gpu] split entry vs ssd_forward, headline")
    ys, hs = run(inp, split=True)
    ya, ha = run(inp)
    assert torch.equal(ys, ya) and torch.equal(hs, ha)


# --------------------------------------------------------------------------
# edge shapes, every P / N / group layout / chunk length, both dtypes
# --------------------------------------------------------------------------

BASE = CONFIGS[1].with_(batch=2, seqlen=256, nheads=4, headdim=64, dstate=128, ngroups=1)

EDGE = [
    # (L, P, N, H, G, io, Q, init)
    (1, 64, 128, 4, 1, "bf16", 0, True),
    (15, 64, 128, 4, 1, "bf16", 0, False),
    (255, 64, 128, 4, 1, "bf16", 256, True),
    (256, 64, 128, 4, 1, "bf16", 256, False),
    (257, 64, 128, 4, 1, "bf16", 256, True),
    (773, 64, 128, 4, 2, "bf16", 256, True),
    (200, 64, 128, 4, 1, "bf16", 64, True),
    (333, 64, 128, 4, 4, "bf16", 128, False),
    (300, 16, 128, 4, 1, "bf16", 0, True),
    (300, 32, 64, 4, 2, "bf16", 0, True),
    (300, 128, 128, 2, 1, "bf16", 0, True),
    (300, 64, 16, 4, 1, "bf16", 0, True),
    (300, 64, 32, 4, 1, "bf16", 0, True),
    (300, 64, 256, 4, 2, "bf16", 0, True),
    (300, 128, 256, 2, 1, "bf16", 128, True),
    (300, 16, 256, 4, 1, "bf16", 0, True),   # headdim 16, dstate 256: default chunk 128
    # Hin smaller than one 1 KB load block; B tile with fewer load blocks
    # than wavefronts; one LDS buffer per head (P = 128 at Q = 256)
    (300, 16, 16, 4, 1, "bf16", 0, True),
    (200, 32, 16, 4, 1, "bf16", 64, True),
    (200, 32, 32, 4, 2, "bf16", 64, False),
    (300, 16, 64, 4, 1, "bf16", 128, True),
    (300, 128, 128, 2, 1, "bf16", 64, False),
    (300, 128, 32, 2, 1, "bf16", 256, True),
    (1, 16, 16, 4, 1, "fp32", 0, True),
    (300, 16, 16, 4, 1, "fp32", 0, True),
    (300, 64, 128, 4, 2, "fp32", 0, True),
    (257, 128, 256, 2, 1, "fp32", 64, True),
    (130, 32, 64, 4, 4, "fp32", 128, False),
]


@pytest.mark.parametrize("L,P,N,H,G,io,Q,init", EDGE)
def test_edge_shapes(L, P, N, H, G, io, Q, init):
    cfg = BASE.with_(seqlen=L, headdim=P, dstate=N, nheads=H, ngroups=G, io_dtype=io, init_state=init)
    inp = make_inputs(cfg, seed=L + P + N + H + G + Q)
    full_check(inp, TOL[io], f"edge L={L} P={P} N={N} H={H} G={G} {io} Q={Q}", chunk_size=Q)


def _bf16_refused(P, N, Q):
    """The bf16 shapes the plan refuses (their register tiles would spill)."""
    return (P == 128 and ((Q == 256 and N >= 64) or (Q == 64 and N == 256))) or (P == 16 and N == 256 and Q == 256)


def _random_split_shapes(n=24, seed=4242):
    """Seeded shapes over the supported set: every head dimension, state size
    and chunk length the plan accepts (0: the shape's default), grouped heads,
    ragged lengths from one token to several chunks, with and without an
    initial state; small enough for the fp64 recurrence on every chain."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        P = int(rng.choice([16, 32, 64, 128]))
        N = int(rng.choice([16, 32, 64, 128, 256]))
        Q = int(rng.choice([0, 64, 128, 256]))
        io = "bf16" if rng.random() < 0.75 else "fp32"
        if io == "bf16" and Q != 0 and _bf16_refused(P, N, Q):
            continue
        G = int(rng.choice([1, 2]))
        H = G * int(rng.choice([1, 2, 4]))
        L = int(rng.integers(1, 900))
        out.append((L, P, N, H, G, io, Q, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("L,P,N,H,G,io,Q,init", _random_split_shapes())
def test_random_shapes_in_full(L, P, N, H, G, io, Q, init):
    """Every output of seeded random shapes through ssd_forward_split (the
    path of every bf16 kernel instantiation these shapes reach, including the
    uneven row-group deal of the eight-wavefront chunk scan) against the fp64
    recurrence."""
    cfg = BASE.with_(seqlen=L, headdim=P, dstate=N, nheads=H, ngroups=G, io_dtype=io, init_state=init)
    inp = make_inputs(cfg, seed=3 * L + P + N + H + Q)
    full_check(inp, TOL[io], f"random L={L} P={P} N={N} H={H} G={G} {io} Q={Q} init={init}", chunk_size=Q,
               split=True)


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_every_chunk_length_gives_the_same_result(Q, io):
    cfg = BASE.with_(seqlen=700, io_dtype=io, init_state=True)
    inp = make_inputs(cfg, seed=7)
    full_check(inp, TOL[io], f"Q={Q} {io}", chunk_size=Q)


def test_memoryless_limit_on_gpu():
    # A -> -inf: every chunk boundary and decay factor underflows to 0; the
    # result must be the memoryless closed form (checked by the oracle pins).
    cfg = BASE.with_(seqlen=300, init_state=True)
    inp = make_inputs(cfg, seed=11)
    inp["A"] = torch.full_like(inp["A"], -1e5)
    full_check(inp, TOL["bf16"], "A=-1e5")


def test_zero_dt_carries_state_on_gpu():
    cfg = BASE.with_(seqlen=300, init_state=True)
    inp = make_inputs(cfg, seed=12)
    inp["dt"] = torch.zeros_like(inp["dt"])
    y, hT = full_check(inp, TOL["bf16"], "dt=0")
    assert torch.equal(hT, inp["init_state"])  # exp(0) = 1 and nothing added


# --------------------------------------------------------------------------
# API options
# --------------------------------------------------------------------------

def test_no_D_and_no_final_state():
    cfg = BASE.with_(seqlen=300, init_state=True)
    inp = make_inputs(cfg, seed=13)
    inp["D"] = None
    y, hT = full_check(inp, TOL["bf16"], "D=None, final=None", return_final_state=False)
    assert hT is None


def test_null_initial_state_equals_zero_initial_state_bitwise():
    cfg = BASE.with_(seqlen=300, init_state=False)
    inp = make_inputs(cfg, seed=14)
    y0, h0 = run(inp)
    inp2 = dict(inp)
    inp2["init_state"] = torch.zeros((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate))
    y1, h1 = run(inp2)
    assert torch.equal(y0, y1) and torch.equal(h0, h1)


def test_in_place_state_update():
    cfg = BASE.with_(seqlen=300, init_state=True)
    inp = make_inputs(cfg, seed=15)
    d = to_dev(inp)
    ref_y, ref_h = run(inp)
    state = d["init_state"].clone()
    y, hT = ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], state, final_state=state)
    torch.cuda.synchronize()
    assert hT.data_ptr() == state.data_ptr()
    assert torch.equal(y.cpu(), ref_y) and torch.equal(state.cpu(), ref_h)


def test_library_allocated_workspace_and_side_stream():
    cfg = BASE.with_(seqlen=400, init_state=True)
    inp = make_inputs(cfg, seed=16)
    ref_y, ref_h = run(inp)
    d = to_dev(inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y, hT = ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"],
                              library_workspace=True)
    s.synchronize()
    assert torch.equal(y.cpu(), ref_y) and torch.equal(hT.cpu(), ref_h)


def test_state_chaining_across_calls():
    cfg = BASE.with_(seqlen=700, init_state=True)
    inp = make_inputs(cfg, seed=17)
    y, hT = run(inp)
    cut = 300

    def part(sl, h0):
        p = dict(inp)
        for k in ("x", "dt", "B", "C"):
            p[k] = inp[k][:, sl].contiguous()
        p["init_state"] = h0
        return run(p)

    y1, h1 = part(slice(0, cut), inp["init_state"])
    y2, h2 = part(slice(cut, None), h1)
    yr, hr = ssd_recurrent(*(np64(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    check_rel(np64(torch.cat([y1, y2], 1)), yr, TOL["bf16"], "chained y")
    check_rel(np64(h2), hr, TOL["bf16"], "chained final_state")


# --------------------------------------------------------------------------
# hygiene
# --------------------------------------------------------------------------

@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_every_output_written_and_guard_bands_intact(io):
    cfg = BASE.with_(seqlen=517, io_dtype=io, init_state=True, ngroups=2)
    inp = make_inputs(cfg, seed=18)
    d = to_dev(inp)
    ny, nh, pad = d["x"].numel(), cfg.batch * cfg.nheads * cfg.headdim * cfg.dstate, 4096
    ybuf = torch.full((ny + 2 * pad,), float("nan"), dtype=d["x"].dtype, device=DEV)
    hbuf = torch.full((nh + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    y = ybuf[pad:pad + ny].view_as(d["x"])
    hT = hbuf[pad:pad + nh].view(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate)
    ws_n = ssd().workspace_bytes(ssd().make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim,
                                                 cfg.dstate, cfg.ngroups, io))
    ws = torch.full((ws_n // 4,), float("nan"), dtype=torch.float32, device=DEV)
    ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], y=y, final_state=hT,
                  workspace=ws.view(torch.uint8))
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(hT).all()
    assert torch.isnan(ybuf[:pad].float()).all() and torch.isnan(ybuf[pad + ny:].float()).all()
    assert torch.isnan(hbuf[:pad]).all() and torch.isnan(hbuf[pad + nh:]).all()


def test_bitwise_deterministic():
    cfg = CONFIGS[1].with_(batch=2, seqlen=1100)
    inp = make_inputs(cfg, seed=19)
    y0, h0 = run(inp)
    y1, h1 = run(inp)
    assert torch.equal(y0, y1) and torch.equal(h0, h1)


# --------------------------------------------------------------------------
# each step on its own against the oracle's definition of its output
# --------------------------------------------------------------------------

STEP_CASES = [("bf16", 256, 600), ("bf16", 64, 300), ("fp32", 128, 333)]


@pytest.mark.parametrize("io,Q,L", STEP_CASES)
def test_step_chunk_cumsum(io, Q, L):
    cfg = BASE.with_(seqlen=L, io_dtype=io, ngroups=2)
    inp = make_inputs(cfg, seed=20)
    d = to_dev(inp)
    note(f"[gpu] step1 cumsum {io} Q={Q} L={L}")
    cs, dtc = ssd().chunk_cumsum(d["dt"], d["A"], headdim=cfg.headdim, dstate=cfg.dstate, ngroups=2,
                                 io_dtype=io, chunk_size=Q)
    torch.cuda.synchronize()
    ref = o_cumsum(np64(inp["dt"]), np64(inp["A"]), Q)
    # fp32 running sum of at most Q terms of magnitude <= 1.6
    assert np.max(np.abs(np64(cs) - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))
    dref = np.zeros(ref.shape)
    dtn = np64(inp["dt"])
    for c in range(ref.shape[2]):
        n = min(Q, L - c * Q)
        dref[:, :, c, :n] = dtn[:, c * Q:c * Q + n, :].transpose(0, 2, 1)
    assert np.array_equal(np64(dtc), dref)


@pytest.mark.parametrize("io,Q,L", STEP_CASES)
def test_step_chunk_state(io, Q, L):
    cfg = BASE.with_(seqlen=L, io_dtype=io, ngroups=2)
    inp = make_inputs(cfg, seed=21)
    d = to_dev(inp)
    note(f"[gpu] step2 chunk_state {io} Q={Q} L={L}")
    cs, dtc = ssd().chunk_cumsum(d["dt"], d["A"], headdim=cfg.headdim, dstate=cfg.dstate, ngroups=2,
                                 io_dtype=io, chunk_size=Q)
    st = ssd().chunk_state(d["x"], d["B"], cs, dtc, chunk_size=Q)
    torch.cuda.synchronize()
    ref = o_local(np64(inp["x"]), np64(inp["dt"]), np64(inp["A"]), np64(inp["B"]), Q)
    check_rel(np64(st), ref, TOL[io], f"chunk states {io} Q={Q}")


@pytest.mark.parametrize("io,Q,L", STEP_CASES)
def test_step_state_passing(io, Q, L):
    cfg = BASE.with_(seqlen=L, io_dtype=io, ngroups=2, init_state=True)
    inp = make_inputs(cfg, seed=22)
    d = to_dev(inp)
    args = [np64(inp[k]) for k in ("x", "dt", "A", "B")]
    local = o_local(*args, Q)
    entry, final = o_entry(*args, Q, np64(inp["init_state"]))
    cs = torch.tensor(o_cumsum(args[1], args[2], Q), dtype=torch.float32, device=DEV)
    st = torch.tensor(local, dtype=torch.float32).to(inp["x"].dtype).to(DEV)
    note(f"[gpu] step3 state_passing {io} Q={Q} L={L}")
    st, hT = ssd().state_passing(st, cs, d["init_state"], seqlen=L, ngroups=2, chunk_size=Q)
    torch.cuda.synchronize()
    check_rel(np64(st), entry, TOL[io], f"entry states {io} Q={Q}")
    check_rel(np64(hT), final, TOL[io], f"final state {io} Q={Q}")


@pytest.mark.parametrize("io,Q,L", STEP_CASES)
def test_step_chunk_scan(io, Q, L):
    cfg = BASE.with_(seqlen=L, io_dtype=io, ngroups=2, init_state=True)
    inp = make_inputs(cfg, seed=23)
    d = to_dev(inp)
    args = [np64(inp[k]) for k in ("x", "dt", "A", "B")]
    entry, _ = o_entry(*args, Q, np64(inp["init_state"]))
    cs = torch.tensor(o_cumsum(args[1], args[2], Q), dtype=torch.float32, device=DEV)
    _, dtc = ssd().chunk_cumsum(d["dt"], d["A"], headdim=cfg.headdim, dstate=cfg.dstate, ngroups=2,
                                io_dtype=io, chunk_size=Q)
    st = torch.tensor(entry, dtype=torch.float32).to(inp["x"].dtype).to(DEV)
    note(f"[gpu] step4+5 chunk_scan {io} Q={Q} L={L}")
    y = ssd().chunk_scan(d["x"], d["B"], d["C"], d["D"], cs, dtc, st, chunk_size=Q)
    torch.cuda.synchronize()
    yr, _ = ssd_recurrent(*(np64(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    check_rel(np64(y), yr, TOL[io], f"chunk scan y {io} Q={Q}")


@pytest.mark.parametrize("io,Q,L,G", [("bf16", 256, 600, 2), ("bf16", 128, 333, 1), ("bf16", 64, 200, 4),
                                      ("fp32", 128, 333, 2)])
def test_forward_equals_its_steps_bitwise(io, Q, L, G):
    """ssd_forward (which may fuse steps into fewer launches) leaves in its
    workspace exactly what the stand-alone steps compute, and returns the
    same y and final state, bit for bit."""
    cfg = BASE.with_(seqlen=L, io_dtype=io, ngroups=G, nheads=8, init_state=True)
    inp = make_inputs(cfg, seed=24)
    d = to_dev(inp)
    lib = ssd()
    desc = lib.make_desc(cfg.batch, L, cfg.nheads, cfg.headdim, cfg.dstate, G, io, Q)
    nws = lib.workspace_bytes(desc)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device=DEV)
    note(f"[gpu] forward vs steps {io} Q={Q} L={L} G={G}")
    y, hT = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], chunk_size=Q,
                        workspace=ws)
    cs, dtc = lib.chunk_cumsum(d["dt"], d["A"], headdim=cfg.headdim, dstate=cfg.dstate, ngroups=G,
                               io_dtype=io, chunk_size=Q)
    st = lib.chunk_state(d["x"], d["B"], cs, dtc, chunk_size=Q)
    cs3, dtc3, st3 = lib.cumsum_chunk_state(d["x"], d["B"], d["dt"], d["A"], chunk_size=Q)
    torch.cuda.synchronize()
    assert torch.equal(cs3, cs) and torch.equal(dtc3, dtc) and torch.equal(st3, st)
    st, hT2 = lib.state_passing(st, cs, d["init_state"], seqlen=L, ngroups=G, chunk_size=Q)
    y2 = lib.chunk_scan(d["x"], d["B"], d["C"], d["D"], cs, dtc, st, chunk_size=Q)
    torch.cuda.synchronize()
    # workspace layout: dA_cumsum, dt_chunked, states, each on a 256-byte boundary
    n = cs.numel() * 4
    off_dt = (n + 255) // 256 * 256
    ws_cs = ws[:n].view(torch.float32).view(cs.shape)
    ws_dt = ws[off_dt:off_dt + n].view(torch.float32).view(cs.shape)
    assert torch.equal(ws_cs, cs), "dA_cumsum in the workspace differs from step 1"
    assert torch.equal(ws_dt, dtc), "dt_chunked in the workspace differs from step 1"
    assert torch.equal(y, y2) and torch.equal(hT, hT2)


# ---- the recurrent (decode) step -----------------------------------------

def _decode_inputs(cfg, seed):
    """One token per sequence: the L = 1 slice of the seeded recipe, plus a
    0.1 N(0,1) state."""
    inp = make_inputs(cfg.with_(seqlen=1, init_state=True), seed=seed)
    return inp


@pytest.mark.parametrize("io,P,N,H,G,withD", [("bf16", 64, 128, 8, 1, True), ("bf16", 16, 16, 4, 2, True),
                                              ("bf16", 32, 256, 4, 4, False), ("bf16", 128, 64, 2, 1, True),
                                              ("fp32", 64, 32, 4, 2, True)])
def test_decode_step_matches_oracle(io, P, N, H, G, withD):
    cfg = BASE.with_(batch=3, io_dtype=io, headdim=P, dstate=N, nheads=H, ngroups=G)
    inp = _decode_inputs(cfg, seed=30)
    if not withD:
        inp["D"] = None
    d = to_dev(inp)
    state = d["init_state"].clone()
    note(f"[gpu] decode step {io} P={P} N={N} H={H} G={G} D={withD}")
    y = ssd().decode_step(d["x"][:, 0], d["dt"][:, 0], d["A"], d["B"][:, 0], d["C"][:, 0], d["D"], state)
    torch.cuda.synchronize()
    yr, hr = ssd_recurrent(*(np64(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    tol = TOL[io]
    check_rel(np64(y), yr[:, 0], tol, f"decode y {io}")
    # the state stays fp32: only fp32 rounding of one update
    check_rel(np64(state), hr, 1e-6, f"decode state {io}")


def test_decode_steps_continue_a_prefill():
    """Prefill L0 tokens with ssd_forward, then decode the next T tokens one
    at a time from its final state: every y and the last state match the
    oracle recurrence over all L0 + T tokens."""
    L0, T = 300, 24
    cfg = BASE.with_(seqlen=L0 + T, nheads=4, ngroups=2, init_state=True)
    inp = make_inputs(cfg, seed=31)
    d = to_dev(inp)
    note(f"[gpu] prefill {L0} + decode {T}")
    _, state = ssd().forward(*(d[k][:, :L0].contiguous() if k in ("x", "dt", "B", "C") else d[k]
                               for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    ys = []
    for t in range(L0, L0 + T):
        ys.append(ssd().decode_step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                                    d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"], state))
    torch.cuda.synchronize()
    yr, hr = ssd_recurrent(*(np64(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    got = np.stack([np64(v) for v in ys], axis=1)
    check_rel(got, yr[:, L0:], TOL["bf16"], "decoded y after prefill")
    check_rel(np64(state), hr, TOL["bf16"], "state after prefill + decode")


def test_decode_step_large_batch_sampled():
    """The decode workload bench.py times (batch 256 of the headline layer),
    checked on sampled sequences."""
    cfg = CONFIGS[1].with_(batch=256)
    inp = _decode_inputs(cfg, seed=32)
    d = to_dev(inp)
    state = d["init_state"].clone()
    note("[gpu] decode step batch 256 H=64 P=64 N=128")
    y = ssd().decode_step(d["x"][:, 0], d["dt"][:, 0], d["A"], d["B"][:, 0], d["C"][:, 0], d["D"], state)
    torch.cuda.synchronize()
    for b in (0, 77, 255):
        sl = {k: (v[b:b + 1] if k in ("x", "dt", "B", "C", "init_state") else v) for k, v in inp.items()}
        yr, hr = ssd_recurrent(*(np64(sl[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
        check_rel(np64(y[b:b + 1]), yr[:, 0], TOL["bf16"], f"decode y b={b}")
        check_rel(np64(state[b:b + 1]), hr, 1e-6, f"decode state b={b}")


# ---- dt preprocessing (bias, softplus, clamp) on every entry point -----------

def _raw_dt_case(cfg, seed):
    """The workload's inputs with dt replaced by raw pre-activation values
    z ~ N(mu, 1) and a per-head bias ~ N(0, 0.5^2), both drawn from a seeded
    CPU generator."""
    inp = make_inputs(cfg, seed=seed)
    g = torch.Generator().manual_seed(1000 + seed)
    inp["dt"] = torch.randn(inp["dt"].shape, generator=g) + cfg.dt_mu
    bias = 0.5 * torch.randn(cfg.nheads, generator=g)
    return inp, bias


@pytest.mark.parametrize("io,Q,L,G,limit", [("bf16", 256, 600, 2, (1e-3, 0.1)), ("bf16", 128, 333, 1, None),
                                            ("fp32", 64, 150, 2, (1e-3, 0.1))])
def test_forward_with_dt_preprocessing(io, Q, L, G, limit):
    from oracle import dt_preprocess
    cfg = BASE.with_(seqlen=L, io_dtype=io, ngroups=G, nheads=4, init_state=True)
    inp, bias = _raw_dt_case(cfg, seed=33)
    d = to_dev(inp)
    pre = dict(bias=bias.to(DEV), softplus=True, limit=limit)
    note(f"[gpu] forward with dt preprocessing {io} Q={Q} L={L} limit={limit}")
    y, hT = ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], chunk_size=Q,
                          dt_pre=pre)
    cs, dtc = ssd().chunk_cumsum(d["dt"], d["A"], headdim=cfg.headdim, dstate=cfg.dstate, ngroups=G,
                                 io_dtype=io, chunk_size=Q, dt_pre=pre)
    torch.cuda.synchronize()
    dt_eff = dt_preprocess(np64(inp["dt"]), np64(bias), softplus=True, limit=limit)
    yr, hr = ssd_recurrent(np64(inp["x"]), dt_eff, *(np64(inp[k]) for k in ("A", "B", "C", "D", "init_state")))
    check_rel(np64(y), yr, TOL[io], f"y with dt preprocessing {io}")
    check_rel(np64(hT), hr, TOL[io], f"final state with dt preprocessing {io}")
    # step 1 alone: dt_chunked is the preprocessed dt (fp32 softplus), 0 past the end
    dref = np.zeros(np64(dtc).shape)
    for c in range(dref.shape[2]):
        n = min(Q, L - c * Q)
        dref[:, :, c, :n] = dt_eff[:, c * Q:c * Q + n, :].transpose(0, 2, 1)
    assert np.max(np.abs(np64(dtc) - dref)) <= 2e-6 * np.max(np.abs(dref))
    assert np.all(np64(dtc)[:, :, -1, L - (dref.shape[2] - 1) * Q:] == 0)


def test_decode_step_with_dt_preprocessing():
    from oracle import dt_preprocess
    cfg = BASE.with_(batch=3, seqlen=1, nheads=4, ngroups=2, init_state=True)
    inp, bias = _raw_dt_case(cfg, seed=34)
    d = to_dev(inp)
    state = d["init_state"].clone()
    pre = dict(bias=bias.to(DEV), softplus=True, limit=(1e-3, 0.1))
    note("[gpu] decode step with dt preprocessing")
    y = ssd().decode_step(d["x"][:, 0], d["dt"][:, 0], d["A"], d["B"][:, 0], d["C"][:, 0], d["D"], state,
                          dt_pre=pre)
    torch.cuda.synchronize()
    dt_eff = dt_preprocess(np64(inp["dt"]), np64(bias), softplus=True, limit=(1e-3, 0.1))
    yr, hr = ssd_recurrent(np64(inp["x"]), dt_eff, *(np64(inp[k]) for k in ("A", "B", "C", "D", "init_state")))
    check_rel(np64(y), yr[:, 0], TOL["bf16"], "decode y with dt preprocessing")
    check_rel(np64(state), hr, 1e-6, "decode state with dt preprocessing")


def test_fused_steps_with_dt_preprocessing_bitwise():
    cfg = BASE.with_(seqlen=500, nheads=8, ngroups=2)
    inp, bias = _raw_dt_case(cfg, seed=35)
    d = to_dev(inp)
    pre = dict(bias=bias.to(DEV), softplus=True, limit=(1e-3, 0.1))
    note("[gpu] fused steps 1+2 with dt preprocessing, bitwise")
    cs, dtc = ssd().chunk_cumsum(d["dt"], d["A"], headdim=cfg.headdim, dstate=cfg.dstate, ngroups=2,
                                 io_dtype="bf16", dt_pre=pre)
    st = ssd().chunk_state(d["x"], d["B"], cs, dtc)
    cs2, dtc2, st2 = ssd().cumsum_chunk_state(d["x"], d["B"], d["dt"], d["A"], dt_pre=pre)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs2) and torch.equal(dtc, dtc2) and torch.equal(st, st2)


# ---- packed variable-length sequences ---------------------------------------

def _packed_case(lengths, cfg, seed, init):
    """Seeded inputs for sum(lengths) packed tokens (the workload recipe on a
    [1, T] batch) and the int32 offsets."""
    T = int(sum(lengths))
    inp = make_inputs(cfg.with_(batch=1, seqlen=max(T, 1), init_state=False), seed=seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h0 = None
    if init:
        g = torch.Generator().manual_seed(2000 + seed)
        h0 = 0.1 * torch.randn((len(lengths), cfg.nheads, cfg.headdim, cfg.dstate), generator=g)
    return inp, cu, h0


@pytest.mark.parametrize("io,Q,init", [("bf16", 256, True), ("bf16", 64, False), ("fp32", 128, True)])
def test_varlen_matches_oracle_per_sequence(io, Q, init):
    lengths = [1, 300, 0, 64, 255, 256, 257, 17, 0, 700, 3]
    cfg = BASE.with_(io_dtype=io, nheads=4, ngroups=2)
    inp, cu, h0 = _packed_case(lengths, cfg, seed=36, init=init)
    d = to_dev(inp)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=DEV)
    note(f"[gpu] varlen {io} Q={Q} init={init} lengths={lengths}")
    y, hT = ssd().forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu_d,
                                 init_states=None if h0 is None else h0.to(DEV), chunk_size=Q)
    torch.cuda.synchronize()
    yg, hg = np64(y), np64(hT)
    for s, n in enumerate(lengths):
        a, e = int(cu[s]), int(cu[s + 1])
        h0s = None if h0 is None else np64(h0[s:s + 1])
        if n == 0:
            ref_h = np.zeros_like(hg[s]) if h0 is None else h0s[0]
            assert np.array_equal(hg[s], ref_h), f"empty sequence {s}: final state must be its initial state"
            continue
        yr, hr = ssd_recurrent(*(np64(inp[k][:, a:e]) for k in ("x", "dt")), np64(inp["A"]),
                               *(np64(inp[k][:, a:e]) for k in ("B", "C")), np64(inp["D"]), h0s)
        check_rel(yg[:, a:e], yr, TOL[io], f"varlen y seq {s} (len {n})")
        check_rel(hg[s:s + 1], hr, TOL[io], f"varlen final state seq {s} (len {n})")


@pytest.mark.parametrize("L,Q", [(700, 256), (256, 256), (300, 64)])
def test_varlen_with_equal_lengths_equals_batched_bitwise(L, Q):
    """Equal lengths: every sequence starts where the batched layout's does,
    so the packed path must give the batched path's bits."""
    S = 3
    cfg = BASE.with_(batch=S, seqlen=L, nheads=4, ngroups=2, init_state=True)
    inp = make_inputs(cfg, seed=37)
    d = to_dev(inp)
    note(f"[gpu] varlen vs batched bitwise L={L} Q={Q}")
    y1, h1 = ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], chunk_size=Q)
    pk = {k: d[k].reshape(1, S * L, *d[k].shape[2:]) for k in ("x", "dt", "B", "C")}
    cu = torch.arange(0, S * L + 1, L, dtype=torch.int32, device=DEV)
    y2, h2 = ssd().forward_varlen(pk["x"], pk["dt"], d["A"], pk["B"], pk["C"], d["D"], cu_seqlens=cu,
                                  init_states=d["init_state"], chunk_size=Q)
    torch.cuda.synchronize()
    assert torch.equal(y2.reshape(y1.shape), y1) and torch.equal(h2, h1)


# ---- the short causal convolution (split into x, B, C) ------------------------

@pytest.mark.parametrize("io,K,silu,bias,state", [("bf16", 4, True, True, True), ("bf16", 1, False, False, False),
                                                  ("bf16", 2, True, False, True), ("fp32", 3, True, True, False)])
def test_conv1d_split_matches_oracle(io, K, silu, bias, state):
    from oracle import causal_conv1d
    b, L, H, P, G, N = 2, 150, 4, 32, 2, 16
    CH = H * P + 2 * G * N
    g = torch.Generator().manual_seed(60 + K)
    dt_ = torch.bfloat16 if io == "bf16" else torch.float32
    u = torch.randn((b, L, CH), generator=g).to(dt_)
    w = (torch.randn((CH, K), generator=g) / K).float()
    bv = torch.randn(CH, generator=g).float() if bias else None
    s0 = torch.randn((b, CH, K - 1), generator=g).float() if state else None
    s_out = torch.full((b, CH, max(K - 1, 1)), float("nan"), device=DEV) if K > 1 else None
    note(f"[gpu] conv1d split {io} K={K} silu={silu} bias={bias} state={state}")
    x, B, C = ssd().conv1d_split(u.to(DEV), w.to(DEV), None if bv is None else bv.to(DEV), nheads=H, headdim=P,
                                 ngroups=G, dstate=N, silu=silu, conv_state_in=None if s0 is None else s0.to(DEV),
                                 conv_state_out=s_out)
    torch.cuda.synchronize()
    ref, last = causal_conv1d(np64(u), np64(w), None if bv is None else np64(bv), silu,
                              None if s0 is None else np64(s0))
    got = np.concatenate([np64(x).reshape(b, L, H * P), np64(B).reshape(b, L, G * N),
                          np64(C).reshape(b, L, G * N)], axis=2)
    check_rel(got, ref, TOL[io], f"conv1d {io} K={K}")
    if K > 1:
        assert np.array_equal(np64(s_out)[:, :, :K - 1], last), "carried state = last K-1 inputs"


def test_conv1d_split_continues_across_calls_bitwise():
    b, L, H, P, G, N, K, cut = 1, 200, 2, 16, 1, 16, 4, 70
    CH = H * P + 2 * G * N
    g = torch.Generator().manual_seed(70)
    u = torch.randn((b, L, CH), generator=g).to(torch.bfloat16).to(DEV)
    w = torch.randn((CH, K), generator=g).float().to(DEV)
    kw = dict(nheads=H, headdim=P, ngroups=G, dstate=N, silu=True)
    note("[gpu] conv1d split continuation")
    whole = ssd().conv1d_split(u, w, **kw)
    s = torch.empty((b, CH, K - 1), device=DEV)
    a = ssd().conv1d_split(u[:, :cut].contiguous(), w, conv_state_out=s, **kw)
    c = ssd().conv1d_split(u[:, cut:].contiguous(), w, conv_state_in=s, **kw)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(torch.cat([a[i], c[i]], dim=1), whole[i])


# ---- HIP graph capture ----------------------------------------------------

@pytest.mark.parametrize("fused", [False, True])
def test_forward_replays_from_a_captured_graph(fused):
    """ssd_forward (and the one-pass entry point) enqueue kernels only, so a
    call can be captured into a HIP graph with a preallocated workspace and
    replayed. Every replay, with eager work and synchronisations in between,
    gives the eager result bit for bit."""
    cfg = CONFIGS[1].with_(batch=2, seqlen=1100, init_state=True)
    inp = make_inputs(cfg, seed=41)
    d = to_dev(inp)
    lib = ssd()
    desc = lib.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, "bf16")
    ws = torch.empty(lib.workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(d["x"])
    hT = torch.empty((cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device=DEV)

    def call():
        lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], y=y, final_state=hT,
                    workspace=ws, fused=fused)

    note(f"[gpu] graph capture and replay (fused={fused})")
    call()
    torch.cuda.synchronize()
    y_ref, h_ref = y.clone(), hT.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        y.fill_(float("nan"))
        hT.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hT, h_ref), f"replay {r} differs from the eager result"


# ---- state passing cut into segments (a few long sequences) ---------------

@pytest.mark.parametrize("L,H,P,N,io,init", [(64 * 256 + 77, 4, 64, 128, "bf16", True),
                                             (96 * 256 + 3, 2, 32, 64, "bf16", False),
                                             (79 * 256 - 40, 2, 16, 16, "fp32", True)])
def test_long_sequence_segmented_state_passing(L, H, P, N, io, init):
    """Few chains of many chunks: ssd_forward cuts each chain into segments
    of 32 chunks that run in parallel. Checked in full against the oracle,
    with a ragged last segment."""
    cfg = BASE.with_(batch=1, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=1, io_dtype=io, init_state=init)
    inp = make_inputs(cfg, seed=L + H)
    full_check(inp, TOL[io], f"segmented state passing L={L} H={H} P={P} N={N} {io}")


def test_segmented_state_passing_in_place_and_against_the_plain_chain():
    """The segmented state passing of ssd_forward with the final state written
    over the initial state, against the plain chain of the step entry point:
    the same entering states and final state up to fp32 rounding order."""
    L, H = 70 * 256 + 11, 4
    cfg = BASE.with_(batch=1, seqlen=L, nheads=H, init_state=True)
    inp = make_inputs(cfg, seed=43)
    d = to_dev(inp)
    lib = ssd()
    note(f"[gpu] segmented state passing in place, L={L}")
    state = d["init_state"].clone()
    y, hT = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], state, final_state=state)
    cs, dtc, st = lib.cumsum_chunk_state(d["x"], d["B"], d["dt"], d["A"])
    st, h2 = lib.state_passing(st, cs, d["init_state"], seqlen=L)
    y2 = lib.chunk_scan(d["x"], d["B"], d["C"], d["D"], cs, dtc, st)
    torch.cuda.synchronize()
    assert hT.data_ptr() == state.data_ptr()
    check_rel(np64(state), np64(h2), 1e-5, "final state: segmented vs plain chain")
    check_rel(np64(y), np64(y2), 1e-2, "y: segmented vs plain chain (entering states rounded to bf16)")
