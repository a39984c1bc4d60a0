"""Properties of the operator checked on the HIP path itself (through the C
ABI), on both forward paths.

The SSD layer is one lower-triangular (semiseparable) matrix acting on x
plus the contribution of the initial state ("Mamba-2 vs Transformers: SSMs,
structured state space duality", section "How we compared Mamba-2,
Transformers, and mixed SSD+attention models": the same matrix contracted as
a recurrence or as masked attention). At fixed dt, A, B, C that makes:
  * y linear in (x, h0) jointly: scaling both by 2 scales y and the final
    state by 2 exactly (every rounding in the path commutes with a power of
    two), and y(x1 + x2, h01 + h02) = y(x1, h01) + y(x2, h02) to the
    tolerance bar;
  * y causal: changing x at token t0 leaves y before t0 bit for bit
    unchanged (the masked weights are exact zeros) and changes y at t0.
Left padding for batched generation ("Mamba-2 vs Transformers", section
"Why speed is not the same as end-to-end serving wins"): a prefix of tokens
with dt = 0 and x = 0 carries the state through unchanged (the decay is
exp(0) = 1 and the input term is 0), so the real tokens' y and the final
state equal those of the unpadded sequence.
"""

import pytest
import torch

from ssd_inputs import CONFIGS, make_inputs
from ssd_testutil import TOL, check_rel, note, np64

pytestmark = pytest.mark.gpu

DEV = "cuda"
PATHS = ["split", "fused"]
CASE = CONFIGS[1].with_(batch=2, seqlen=3 * 256 + 41, nheads=8, init_state=True)


def ssd():
    import mamba_ssd_scan_fwd_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def fwd(inp, path, **over):
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    d.update({k: v.to(DEV) for k, v in over.items()})
    y, hT = ssd().forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"],
                          fused=path == "fused", split=path == "split")
    torch.cuda.synchronize()
    return y.cpu(), hT.cpu()


@pytest.mark.parametrize("path", PATHS)
def test_scaling_x_and_h0_by_two_scales_the_outputs_exactly(path):
    inp = make_inputs(CASE, seed=51)
    note(f"[gpu] homogeneity, {path}")
    y1, h1 = fwd(inp, path)
    y2, h2 = fwd(inp, path, x=inp["x"] * 2, init_state=inp["init_state"] * 2)
    assert torch.equal(y2, y1 * 2) and torch.equal(h2, h1 * 2)


@pytest.mark.parametrize("path", PATHS)
def test_additive_in_x_and_h0(path):
    """x1 holds the even tokens and x2 the odd ones, so x1 + x2 is exact in
    bf16; the two initial states are independent draws."""
    inp = make_inputs(CASE, seed=52)
    x = inp["x"]
    even = (torch.arange(CASE.seqlen) % 2 == 0)[None, :, None, None]
    x1 = torch.where(even, x, torch.zeros_like(x))
    x2 = torch.where(even, torch.zeros_like(x), x)
    g = torch.Generator().manual_seed(53)
    h02 = 0.1 * torch.randn(inp["init_state"].shape, generator=g)
    note(f"[gpu] additivity, {path}")
    ya, ha = fwd(inp, path, x=x1)
    yb, hb = fwd(inp, path, x=x2, init_state=h02)
    ys, hs = fwd(inp, path, x=x, init_state=inp["init_state"] + h02)
    check_rel(np64(ya) + np64(yb), np64(ys), TOL["bf16"], f"y(x1) + y(x2) vs y(x1 + x2), {path}")
    check_rel(np64(ha) + np64(hb), np64(hs), TOL["bf16"], f"final states, {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("t0", [0, 255, 256, 300, CASE.seqlen - 1])
def test_changing_x_at_t0_leaves_earlier_outputs_unchanged(path, t0):
    inp = make_inputs(CASE, seed=54)
    x2 = inp["x"].clone()
    x2[:, t0] = (x2[:, t0].float() + 1.0).to(x2.dtype)
    note(f"[gpu] causality t0={t0}, {path}")
    y1, h1 = fwd(inp, path)
    y2, h2 = fwd(inp, path, x=x2)
    assert torch.equal(y1[:, :t0], y2[:, :t0]), "an output before t0 changed"
    assert not torch.equal(y1[:, t0], y2[:, t0]), "the output at t0 did not change"
    if t0 == CASE.seqlen - 1:
        # (an earlier token's share of the final state can decay below fp32
        # resolution over the rest of the sequence)
        assert not torch.equal(h1, h2), "the final state did not change"


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pad", [1, 200, 256, 333])
def test_left_padding_leaves_the_real_tokens_unchanged(path, pad):
    inp = make_inputs(CASE, seed=55)
    L = CASE.seqlen
    g = torch.Generator().manual_seed(56 + pad)
    padded = {}
    for k in ("x", "dt", "B", "C"):
        v = inp[k]
        if k in ("x", "dt"):
            head = torch.zeros((v.shape[0], pad) + tuple(v.shape[2:]), dtype=v.dtype)
        else:  # B and C of the pad tokens are arbitrary: dt = 0 and x = 0 cancel them
            head = (torch.randn((v.shape[0], pad) + tuple(v.shape[2:]), generator=g) / CASE.dstate ** 0.5).to(v.dtype)
        padded[k] = torch.cat([head, v], dim=1)
    padded.update({k: inp[k] for k in ("A", "D", "init_state")})
    note(f"[gpu] left padding {pad} tokens, {path}")
    y0, h0 = fwd(inp, path)
    yp, hp = fwd(padded, path)
    assert yp.shape[1] == pad + L
    check_rel(np64(yp[:, pad:]), np64(y0), TOL["bf16"], f"real tokens' y after {pad} pad tokens, {path}")
    check_rel(np64(hp), np64(h0), TOL["bf16"], f"final state after {pad} pad tokens, {path}")
