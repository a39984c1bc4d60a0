"""The short causal convolution fused into the forward pass (ssd_forward_conv),
on the GPU, through the C ABI.

The convolution is the Mamba-2 block's input step in front of the SSM
(Telegram post "Mamba3", paragraph on the removed short causal convolution).
ssd_forward_conv applies it inside the forward's first kernel; it must give
the bits of the two-call path (ssd_conv1d_split, then ssd_forward_split) for
y, the final state, the convolved x, B, C and the carried convolution state,
and match the oracle's convolution followed by its recurrence.
"""

import numpy as np
import pytest
import torch

from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import OUT_EPS, TOL, check_rel, note, np64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def ssd():
    import mamba_ssd_scan_fwd_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def conv_case(b, L, H, P, N, G, K, bias, state, seed):
    """Seeded packed activations (bf16, the B and C channels scaled by
    1/sqrt(N) like the workloads' B and C), weights, bias, a carried state
    whose values are bf16 numbers (as a state this library writes), and the
    forward's dt, A, D and initial state from the workload recipe."""
    CH = H * P + 2 * G * N
    g = torch.Generator().manual_seed(seed)
    xbc = torch.randn((b, L, CH), generator=g)
    xbc[:, :, H * P:] /= N ** 0.5
    xbc = xbc.to(torch.bfloat16)
    w = (torch.randn((CH, K), generator=g) / K ** 0.5).float()
    bv = (0.1 * torch.randn(CH, generator=g)).float() if bias else None
    s0 = torch.randn((b, CH, K - 1), generator=g).to(torch.bfloat16).float() if state and K > 1 else None
    cfg = CONFIGS[1].with_(batch=b, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G, init_state=True)
    inp = make_inputs(cfg, seed=seed + 1)
    return xbc, w, bv, s0, inp


def dev(t):
    return None if t is None else t.to(DEV)


# (b, L, H, P, N, G, Q, K, silu, bias, carried state)
CASES = [
    (2, 700, 8, 64, 128, 2, 256, 4, True, True, True),   # ragged last chunk, state in and out
    (1, 300, 4, 32, 64, 1, 64, 3, True, False, False),
    (2, 513, 4, 64, 256, 2, 256, 2, False, True, True),  # N = 256: two blocks of state columns
    (1, 130, 4, 16, 16, 4, 128, 1, True, True, False),   # width 1, G = H
    (3, 256, 8, 128, 32, 2, 128, 4, True, True, True),   # P = 128
    (1, 2, 4, 64, 128, 1, 64, 4, True, True, True),      # shorter than the convolution: state carried through
    (2, 1100, 16, 64, 128, 1, 256, 4, True, True, True),  # 16 heads per group: several head groups
]


@pytest.mark.parametrize("b,L,H,P,N,G,Q,K,silu,bias,state", CASES,
                         ids=[f"b{c[0]}-L{c[1]}-H{c[2]}-P{c[3]}-N{c[4]}-G{c[5]}-Q{c[6]}-K{c[7]}" for c in CASES])
def test_fused_convolution_gives_the_two_call_bits(b, L, H, P, N, G, Q, K, silu, bias, state):
    m = ssd()
    xbc, w, bv, s0, inp = conv_case(b, L, H, P, N, G, K, bias, state, seed=300 + L)
    d = {k: dev(v) for k, v in inp.items()}
    CH = H * P + 2 * G * N
    note(f"[gpu] forward_conv vs two calls b={b} L={L} H={H} P={P} N={N} G={G} Q={Q} K={K}")
    so1 = torch.full((b, CH, max(K - 1, 1)), float("nan"), device=DEV) if K > 1 else None
    so2 = torch.full_like(so1, float("nan")) if K > 1 else None
    x1, B1, C1 = m.conv1d_split(dev(xbc), dev(w), dev(bv), nheads=H, headdim=P, ngroups=G, dstate=N, silu=silu,
                                conv_state_in=dev(s0), conv_state_out=so1)
    y1, h1 = m.forward(x1, d["dt"], d["A"], B1, C1, d["D"], d["init_state"], chunk_size=Q, split=True)
    desc = m.make_desc(b, L, H, P, N, G, "bf16", Q)
    ws = torch.empty(m.workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    y2, h2, x2, B2, C2 = m.forward_conv(dev(xbc), dev(w), d["dt"], d["A"], d["D"], d["init_state"], nheads=H,
                                        headdim=P, ngroups=G, dstate=N, bias=dev(bv), silu=silu,
                                        conv_state_in=dev(s0), conv_state_out=so2, chunk_size=Q, workspace=ws)
    path, status = m.workspace_status(desc, ws)
    torch.cuda.synchronize()
    assert path in ("split", "split-segmented") and status == 0
    assert torch.equal(x1, x2) and torch.equal(B1, B2) and torch.equal(C1, C2), "convolved x, B, C differ"
    if K > 1:
        assert torch.equal(so1, so2), "carried convolution state differs"
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_fused_convolution_matches_the_oracle():
    from oracle import causal_conv1d, ssd_recurrent
    m = ssd()
    b, L, H, P, N, G, K = 2, 333, 4, 32, 64, 2, 4
    xbc, w, bv, s0, inp = conv_case(b, L, H, P, N, G, K, True, True, seed=401)
    d = {k: dev(v) for k, v in inp.items()}
    note("[gpu] forward_conv vs oracle convolution + recurrence")
    y, hT, _, _, _ = m.forward_conv(dev(xbc), dev(w), d["dt"], d["A"], d["D"], d["init_state"], nheads=H, headdim=P,
                                    ngroups=G, dstate=N, bias=dev(bv), silu=True, conv_state_in=dev(s0))
    torch.cuda.synchronize()
    u, _ = causal_conv1d(np64(xbc), np64(w), np64(bv), True, np64(s0))
    x = u[:, :, :H * P].reshape(b, L, H, P)
    Bm = u[:, :, H * P:H * P + G * N].reshape(b, L, G, N)
    Cm = u[:, :, H * P + G * N:].reshape(b, L, G, N)
    yr, hr = ssd_recurrent(x, np64(inp["dt"]), np64(inp["A"]), Bm, Cm, np64(inp["D"]), np64(inp["init_state"]))
    check_rel(np64(y), yr, TOL["bf16"], "y of convolution + forward")
    check_rel(np64(hT), hr, TOL["bf16"], "final state of convolution + forward")


def test_fused_convolution_at_the_headline_size():
    """The headline layer (8 x 2048, 64 heads, P 64, N 128) with a width-4
    SiLU convolution: the fused call against the two-call path, bit for bit."""
    m = ssd()
    cfg = CONFIGS[1]
    b, L, H, P, N, G, K = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups, 4
    xbc, w, bv, _, inp = conv_case(b, L, H, P, N, G, K, True, False, seed=402)
    d = {k: dev(v) for k, v in inp.items()}
    note("[gpu] forward_conv at the headline size")
    x1, B1, C1 = m.conv1d_split(dev(xbc), dev(w), dev(bv), nheads=H, headdim=P, ngroups=G, dstate=N, silu=True)
    y1, h1 = m.forward(x1, d["dt"], d["A"], B1, C1, d["D"], d["init_state"], split=True)
    y2, h2, x2, B2, C2 = m.forward_conv(dev(xbc), dev(w), d["dt"], d["A"], d["D"], d["init_state"], nheads=H,
                                        headdim=P, ngroups=G, dstate=N, bias=dev(bv), silu=True)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2) and torch.equal(B1, B2) and torch.equal(C1, C2)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
