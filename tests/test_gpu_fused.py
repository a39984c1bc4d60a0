"""GPU parity of the one-pass path (ssd_forward_fused) against the fp64 oracle.

The one-pass kernel computes every chunk's state, hands it to the next
chunk's workgroup and writes y in one launch (after the dt cumsum). These
cases run it through the C ABI on seeded inputs and compare with the oracle
element by element (in full at small sizes, on sampled heads over the whole
sequence at the workloads' sizes), check that every state hand-over
happened (the per-head counters, the ticket count and the status word it
leaves in the workspace), and compare it with the split path.
"""

import numpy as np
import pytest
import torch

from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import TOL, check_rel, note, np64
from test_gpu_parity import BASE, DEV, full_check, pairs_for, run, sampled_check, ssd, to_dev

pytestmark = pytest.mark.gpu

# workloads the one-pass kernel supports (bf16, chunk 256, headdim 32/64, dstate 32..128)
FUSED_IDX = [i for i, c in enumerate(CONFIGS)
             if c.io_dtype == "bf16" and c.headdim in (32, 64) and 32 <= c.dstate <= 128
             and not (c.headdim == 32 and c.dstate == 32)]


def up(v):
    return -(-v // 256) * 256


def sync_words(ws, cfg, desc, Q=256):
    """The per-head counters and the ticket the one-pass kernel leaves in the
    workspace (after dA_cumsum and dt_chunked, each 256-byte aligned, the
    states region starts with the hand-over ring, then the counters), and
    the status bits of the call's status record (ssd_workspace_status)."""
    nc = -(-cfg.seqlen // Q)
    cs = cfg.batch * cfg.nheads * nc * Q * 4
    st_off = up(up(cs) + cs)
    ring = cfg.batch * cfg.nheads * 2 * cfg.headdim * cfg.dstate * 4
    off = st_off + up(ring)
    n = cfg.batch * cfg.nheads + 1
    w = ws[off:off + 4 * n].view(torch.int32).cpu().numpy()
    path, status = ssd().workspace_status(desc, ws)
    assert path == "one-pass"
    return w[:-1], int(w[-1]), status, nc


def test_fused_covers_the_headline_workload():
    assert 1 in FUSED_IDX and len(FUSED_IDX) >= 2


@pytest.mark.parametrize("idx", FUSED_IDX)
def test_fused_workloads_reduced_length(idx):
    cfg = CONFIGS[idx]
    small = cfg.with_(batch=min(cfg.batch, 2), seqlen=3 * 256 + 77)
    inp = make_inputs(small, seed=200 + idx)
    sampled_check(inp, pairs_for(small, 4), TOL[cfg.io_dtype], f"fused {cfg.name} reduced", fused=True)


@pytest.mark.parametrize("idx", FUSED_IDX)
def test_fused_workloads_full_size(idx):
    cfg = CONFIGS[idx]
    inp = make_inputs(cfg, seed=idx)
    sampled_check(inp, pairs_for(cfg, 3), TOL[cfg.io_dtype], f"fused {cfg.name} full size", fused=True)


FUSED_EDGE = [
    # (L, P, N, H, G, init)
    (1, 64, 128, 4, 1, True),            # one chunk: one workgroup reads the initial state, writes the final
    (255, 64, 128, 4, 1, True),
    (256, 64, 128, 4, 1, False),
    (257, 64, 128, 4, 1, True),          # two chunks, one token in the second
    (773, 64, 128, 4, 2, True),
    (300, 32, 64, 4, 2, True),
    (300, 32, 128, 8, 1, True),
    (300, 64, 32, 4, 1, True),
    (300, 64, 64, 8, 4, False),
    (600, 64, 128, 16, 16, True),        # one head per group
    (41 * 256 - 243, 64, 128, 4, 1, True),  # a chain of 41 chunks
    (3000, 32, 64, 32, 2, True),         # 16 heads per group
]


@pytest.mark.parametrize("L,P,N,H,G,init", FUSED_EDGE)
def test_fused_edge_shapes(L, P, N, H, G, init):
    cfg = BASE.with_(seqlen=L, headdim=P, dstate=N, nheads=H, ngroups=G, io_dtype="bf16", init_state=init)
    inp = make_inputs(cfg, seed=L + 3 * P + N + H + G)
    full_check(inp, TOL["bf16"], f"fused edge L={L} P={P} N={N} H={H} G={G}", fused=True)


@pytest.mark.parametrize("L,H,G,batch,N", [(1, 4, 1, 2, 128), (257, 4, 2, 2, 128), (3000, 32, 2, 2, 128),
                                           (41 * 256 - 243, 4, 1, 2, 128), (1100, 64, 1, 8, 128),
                                           (2048, 64, 1, 8, 128), (2048, 64, 1, 32, 128), (4096, 32, 1, 32, 64)])
def test_fused_chain_completed(L, H, G, batch, N):
    """Every head's counter ends at the last hand-over (nc - 1), the tickets
    cover the grid, and no wait was cut off (batch 8 with 64 heads: the
    headline's 32 chains of 16 heads; batch 32: the same layer over several
    rounds of workgroups; 32 x 4096 with N = 64: the small-state workload)."""
    cfg = BASE.with_(seqlen=L, nheads=H, ngroups=G, batch=batch, dstate=N, init_state=True)
    inp = make_inputs(cfg, seed=L + H)
    d = to_dev(inp)
    lib = ssd()
    desc = lib.make_desc(cfg.batch, L, H, cfg.headdim, cfg.dstate, G, "bf16", 0)
    ws = torch.full((lib.workspace_bytes(desc),), 0xA5, dtype=torch.uint8, device=DEV)
    note(f"[gpu] fused chain counters B={batch} L={L} H={H} G={G} N={N}")
    lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], workspace=ws, fused=True)
    torch.cuda.synchronize()
    flags, ticket, status, nc = sync_words(ws, cfg, desc)
    assert status == 0
    assert np.all(flags == (nc - 1 if nc > 1 else 0)), flags
    units = cfg.batch * nc * H
    assert ticket > 0 and units % ticket == 0 and (units // ticket) in (1, 2, 4, 8, 16)


def test_fused_matches_split_path():
    cfg = CONFIGS[1].with_(batch=2, seqlen=5 * 256 + 31, init_state=True)
    inp = make_inputs(cfg, seed=31)
    note("[gpu] fused vs split")
    ys, hs = run(inp)
    yf, hf = run(inp, fused=True)
    # both are within the bar of the oracle; against each other they differ
    # only by where bf16 rounding happens (the chunk states stay fp32 here)
    check_rel(np64(yf), np64(ys), TOL["bf16"], "fused vs split y")
    check_rel(np64(hf), np64(hs), TOL["bf16"], "fused vs split final_state")


def test_fused_api_options():
    cfg = BASE.with_(seqlen=700, init_state=True)
    inp = make_inputs(cfg, seed=32)
    ref_y, ref_h = run(inp, fused=True)
    d = to_dev(inp)
    lib = ssd()
    note("[gpu] fused in-place state, no D, no final state, library workspace")
    # in-place state update gives the same bits
    state = d["init_state"].clone()
    y, hT = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], state, final_state=state, fused=True)
    torch.cuda.synchronize()
    assert hT.data_ptr() == state.data_ptr()
    assert torch.equal(y.cpu(), ref_y) and torch.equal(state.cpu(), ref_h)
    # library-allocated workspace on a side stream
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y2, h2 = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"],
                             library_workspace=True, fused=True)
    s.synchronize()
    assert torch.equal(y2.cpu(), ref_y) and torch.equal(h2.cpu(), ref_h)
    # no D, no final state
    inp2 = dict(inp)
    inp2["D"] = None
    y3, h3 = full_check(inp2, TOL["bf16"], "fused D=None final=None", fused=True, return_final_state=False)
    assert h3 is None


def test_fused_bitwise_deterministic_and_workspace_reuse():
    cfg = CONFIGS[1].with_(batch=2, seqlen=1100)
    inp = make_inputs(cfg, seed=33)
    d = to_dev(inp)
    lib = ssd()
    desc = lib.make_desc(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, "bf16", 0)
    ws = torch.empty((lib.workspace_bytes(desc),), dtype=torch.uint8, device=DEV)
    note("[gpu] fused determinism, one workspace for three calls")
    outs = []
    for _ in range(3):
        y, hT = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], workspace=ws,
                            fused=True)
        torch.cuda.synchronize()
        outs.append((y.cpu(), hT.cpu()))
    for y, hT in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(hT, outs[0][1])


def test_fused_rejects_unsupported_shapes():
    lib = ssd()
    for kw in (dict(io_dtype="fp32"), dict(chunk_size=128), dict(headdim=128), dict(dstate=256),
               dict(headdim=32, dstate=32)):
        cfg = BASE.with_(seqlen=300, io_dtype=kw.get("io_dtype", "bf16"), headdim=kw.get("headdim", 64),
                         dstate=kw.get("dstate", 128))
        inp = make_inputs(cfg, seed=34)
        d = to_dev(inp)
        with pytest.raises(lib.SSDError, match="UNSUPPORTED"):
            lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"],
                        chunk_size=kw.get("chunk_size", 0), fused=True)


def _random_fused_shapes(n=10, seed=2024):
    """Seeded shapes inside the supported set, from one chunk to multi-round
    grids (more workgroups than compute units, so chains continue across
    rounds of workgroups)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        P = int(rng.choice([32, 64]))
        N = int(rng.choice([32, 64, 128]))
        if P == 32 and N == 32:
            continue
        G = int(rng.choice([1, 2, 4]))
        H = G * int(rng.choice([1, 2, 4, 8, 16]))
        B = int(rng.integers(1, 13))
        L = int(rng.integers(1, 12 * 256))
        out.append((B, L, H, P, N, G))
    # multi-round at the headline layer shape: 384 and 768 workgroups
    out += [(12, 2048, 64, 64, 128, 1), (24, 2048, 64, 64, 128, 1)]
    return out


@pytest.mark.parametrize("B,L,H,P,N,G", _random_fused_shapes())
def test_fused_random_shapes(B, L, H, P, N, G):
    cfg = BASE.with_(batch=B, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, init_state=bool(L % 2))
    inp = make_inputs(cfg, seed=B * 7 + L)
    pairs = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    pairs = list(dict.fromkeys(pairs))
    sampled_check(inp, pairs, TOL["bf16"], f"fused random B={B} L={L} H={H} P={P} N={N} G={G}", fused=True)


def test_fused_debug_mode_checks_the_status_word():
    """With SSD_DEBUG set, the one-pass call waits for its kernel and checks
    the hand-over status word (a separate process: the setting is read once
    per process)."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch, mamba_ssd_scan_fwd_amd as m\n"
        "from ssd_inputs import CONFIGS, make_inputs\n"
        "cfg = CONFIGS[1].with_(batch=2, seqlen=700)\n"
        "d = {k: (v.cuda() if v is not None else None) for k, v in make_inputs(cfg, seed=5).items()}\n"
        "y, h = m.forward(d['x'], d['dt'], d['A'], d['B'], d['C'], d['D'], d['init_state'], fused=True)\n"
        "torch.cuda.synchronize()\n"
        "print('finite', bool(torch.isfinite(y.float()).all()))\n" % root)
    note("[gpu] one-pass path with SSD_DEBUG=1 in a subprocess")
    env = dict(os.environ, SSD_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "path=fused" in r.stderr and "cut off" not in r.stderr, r.stderr[-2000:]
    assert "finite True" in r.stdout
