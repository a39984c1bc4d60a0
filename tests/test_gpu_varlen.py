"""Packed sequences cut into fixed chunks of the packed stream (the varlen
entry point with bf16 io and without initial states; fp32 io keeps chunks per
sequence), on the GPU, through the C ABI.

Each sequence runs the recurrence of the SSD layer on its own tokens ("Mamba-2
vs Transformers: SSMs, structured state space duality", section "How we
compared Mamba-2, Transformers, and mixed SSD+attention models"); the chunks
are those of one sequence of T tokens, so one chunk may hold the end of one
sequence and the starts of several others. Every sequence's y and final state
are compared with the fp64 oracle recurrence run on that sequence alone; a
single sequence must give the batched split path's bits; the status record
must report the state-passing path taken and no cut-off wait.
"""

import numpy as np
import pytest
import torch

from oracle_pool import compare_packed
from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import OUT_EPS, TOL, note

pytestmark = pytest.mark.gpu

DEV = "cuda"
BASE = CONFIGS[1].with_(headdim=64, dstate=128)


def ssd():
    import mamba_ssd_scan_fwd_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def packed_run(cfg, lengths, Q, seed, finals=True):
    """Seeded [1, T] inputs for the lengths; one varlen call with a
    caller-owned workspace. Returns inputs, offsets, y, final states (host)
    and the recorded (path, status)."""
    lib = ssd()
    T = int(sum(lengths))
    inp = make_inputs(cfg.with_(batch=1, seqlen=T, init_state=False), seed=seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    cu_d = torch.tensor(cu, device=DEV)
    desc = lib.make_desc(1, T, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, cfg.io_dtype, Q)
    S = len(lengths)
    ws = torch.empty(lib.workspace_bytes_varlen(desc, S), dtype=torch.uint8, device=DEV)
    y, hT = lib.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu_d, chunk_size=Q,
                               return_final_states=finals, workspace=ws)
    path, status = lib.workspace_status_varlen(desc, S, ws)
    torch.cuda.synchronize()
    return inp, cu, y.cpu(), None if hT is None else hT.cpu(), path, status


# (io, chunk length, lengths, state-passing path)
CASES = [
    ("bf16", 256, [1, 3, 0, 17, 64, 5, 200, 2, 0, 31, 256, 1, 90, 0], "split"),  # many sequences per chunk
    ("bf16", 64, [64, 64, 128, 0, 192, 1, 63, 65], "split"),  # starts on chunk boundaries
    ("fp32", 128, [300, 7, 129, 0, 0, 511, 2], "split"),  # (fp32 io: chunks per sequence)
    ("bf16", 128, [0, 100, 0], "split"),  # empty sequences at both ends
    ("bf16", 64, [1] * 70 + [500], "split"),  # 63 starts within one chunk
    ("fp32", 64, [1] * 70 + [500], "split"),
    ("bf16", 256, [1] * 250 + [700], "split"),  # 249 starts, then a long sequence in the same chunk
    ("bf16", 256, [5000, 3, 9000, 250, 2500], "split-segmented"),  # 66 chunks: segments of 32
]


@pytest.mark.parametrize("io,Q,lengths,path", CASES,
                         ids=[f"{io}-Q{Q}-S{len(l)}-T{sum(l)}" for io, Q, l, _ in CASES])
def test_fixed_chunks_match_the_oracle_per_sequence(io, Q, lengths, path):
    cfg = BASE.with_(io_dtype=io, nheads=4, ngroups=2)
    note(f"[gpu] varlen fixed chunks {io} Q={Q} S={len(lengths)} T={sum(lengths)}")
    inp, cu, y, hT, got_path, status = packed_run(cfg, lengths, Q, seed=80 + Q)
    note(f"    path {got_path}, status {status}")
    assert got_path == path and status == 0
    r = compare_packed(inp, cu, y, hT, OUT_EPS[io], block=2)
    note(f"    {r}")
    assert r["finite"] and r["empty_ok"]
    for k in ("y", "ssm", "final_state"):
        assert r[k] <= TOL[io], f"{k}: {r[k]:.3e} > {TOL[io]}"


def test_final_states_do_not_change_y():
    """Asking for the final states adds work after the chunk scan only."""
    cfg = BASE.with_(nheads=4, ngroups=2)
    lengths = [40, 300, 1, 0, 222]
    _, _, y1, _, _, _ = packed_run(cfg, lengths, 64, seed=90, finals=True)
    _, _, y2, h2, _, _ = packed_run(cfg, lengths, 64, seed=90, finals=False)
    assert h2 is None and torch.equal(y1, y2)


@pytest.mark.parametrize("L,Q,H", [(700, 256, 4), (300, 64, 4), (16700, 256, 4)])
def test_one_sequence_equals_the_batched_split_path(L, Q, H):
    """One sequence: no start after token 0, so the fixed chunks are the
    batched layout's at batch 1 and y has the batched split path's bits (at
    16700 tokens both cut state passing into segments). The final state
    differs in two roundings: the end window keeps its local state in fp32
    where the batched path rounds the last chunk state to bf16, and carries
    the entering state as stored for the chunk scan (bf16) where the batched
    path keeps it in fp32: within 2^-7 of max|final state|."""
    lib = ssd()
    cfg = BASE.with_(batch=1, seqlen=L, nheads=H, ngroups=2, init_state=False)
    inp = make_inputs(cfg, seed=91)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    note(f"[gpu] varlen one sequence vs batched split L={L} Q={Q}")
    y1, h1 = lib.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None, chunk_size=Q, split=True)
    cu = torch.tensor([0, L], dtype=torch.int32, device=DEV)
    y2, h2 = lib.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu, chunk_size=Q)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    scale = h1.abs().max().item()
    assert (h2 - h1).abs().max().item() <= 2.0 ** -7 * scale


@pytest.mark.parametrize("Q", [64, 256])
def test_changing_one_sequence_leaves_the_others_bit_for_bit(Q):
    """Sequence isolation in fixed chunks: every decay across a sequence start
    is exactly 0, so the other sequences' y and final states must not change
    by a single bit when one sequence's x, B and C change (including
    sequences that share a chunk with it). (Its dt is left alone: dt enters
    the chunk's dA cumsum, and a later sequence in the same chunk sees the
    offset of its start rounded with it, so its decays may move by a
    rounding.)"""
    lib = ssd()
    cfg = BASE.with_(nheads=4, ngroups=2)
    lengths = [70, 3, 130, 1, 0, 200, 45]
    T = sum(lengths)
    inp = make_inputs(cfg.with_(batch=1, seqlen=T, init_state=False), seed=95)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cu_d = torch.tensor(cu, device=DEV)
    note(f"[gpu] varlen sequence isolation Q={Q}")

    def run(d):
        y, hT = lib.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu_d, chunk_size=Q)
        torch.cuda.synchronize()
        return y.cpu(), hT.cpu()

    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y0, h0 = run(d)
    for s in (1, 2, 5):  # a 3-token sequence inside a chunk, one spanning chunks, the one after an empty one
        a, e = int(cu[s]), int(cu[s + 1])
        g = torch.Generator().manual_seed(96 + s)
        d2 = {k: (v.clone() if v is not None else None) for k, v in d.items()}
        for k in ("x", "B", "C"):
            d2[k][:, a:e] = torch.randn(d2[k][:, a:e].shape, generator=g).to(d2[k].dtype).to(DEV)
        y1, h1 = run(d2)
        keep = torch.ones(T, dtype=torch.bool)
        keep[a:e] = False
        assert torch.equal(y1[:, keep], y0[:, keep]), f"changing sequence {s} changed another sequence's y"
        others = [q for q in range(len(lengths)) if q != s]
        assert torch.equal(h1[others], h0[others]), f"changing sequence {s} changed another final state"
        assert not torch.equal(y1[:, a:e], y0[:, a:e])


@pytest.mark.parametrize("init,T", [(False, 700), (False, 17000), (True, 700)])
def test_varlen_replays_from_a_captured_graph(init, T):
    """ssd_forward_varlen enqueues kernels only (the tables and the cleared
    words come from kernels, not memsets), so a call can be captured into a
    HIP graph with a preallocated workspace and replayed; every replay, with
    eager work in between, gives the eager bits. Both cuts (fixed chunks
    without initial states, with the segmented state passing at 17000
    tokens; chunks per sequence with them)."""
    lib = ssd()
    cfg = BASE.with_(nheads=4, ngroups=2)
    lengths = [T // 3, 5, T - T // 3 - 5 - 40, 0, 40]
    inp = make_inputs(cfg.with_(batch=1, seqlen=T, init_state=False), seed=97)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=DEV)
    S = len(lengths)
    h0 = (0.1 * torch.randn((S, cfg.nheads, cfg.headdim, cfg.dstate), generator=torch.Generator().manual_seed(98))
          ).to(DEV) if init else None
    desc = lib.make_desc(1, T, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, "bf16", 0)
    ws = torch.empty(lib.workspace_bytes_varlen(desc, S), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(d["x"])
    hT = torch.empty((S, cfg.nheads, cfg.headdim, cfg.dstate), dtype=torch.float32, device=DEV)

    def call():
        lib.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu_seqlens=cu, init_states=h0, y=y,
                           final_states=hT, workspace=ws)

    note(f"[gpu] varlen graph capture and replay init={init} T={T}")
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
        path, status = lib.workspace_status_varlen(desc, S, ws)
        assert status == 0
