"""The seeded input recipe: shapes, dtypes, ranges, moments, reproducibility."""

import math

import pytest
import torch

from ssd_inputs import CONFIGS, make_inputs


def small(cfg):
    # same distributions, fewer tokens, so the test stays fast
    return cfg.with_(batch=min(cfg.batch, 2), seqlen=min(cfg.seqlen, 512))


@pytest.mark.parametrize("idx", range(len(CONFIGS)))
def test_shapes_dtypes_and_ranges(idx):
    cfg = small(CONFIGS[idx])
    t = make_inputs(cfg, seed=idx)
    b, L, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
    assert t["x"].shape == (b, L, H, P) and t["x"].dtype == io
    assert t["B"].shape == (b, L, G, N) and t["B"].dtype == io
    assert t["C"].shape == (b, L, G, N) and t["C"].dtype == io
    assert t["dt"].shape == (b, L, H) and t["dt"].dtype == torch.float32
    assert t["A"].shape == (H,) and t["D"].shape == (H,)
    assert float(t["dt"].min()) >= cfg.dt_lo and float(t["dt"].max()) <= cfg.dt_hi * (1 + 1e-6)
    assert float(t["A"].max()) <= -1.0 + 1e-6 and float(t["A"].min()) >= -16.0 - 1e-4
    if cfg.init_state:
        assert t["init_state"].shape == (b, H, P, N)
        assert abs(float(t["init_state"].std()) - 0.1) < 0.01
    else:
        assert t["init_state"] is None
    # x ~ N(0,1), B ~ N(0,1)/sqrt(N)
    assert abs(float(t["x"].float().std()) - 1.0) < 0.02
    assert abs(float(t["B"].float().std()) * math.sqrt(N) - 1.0) < 0.05


def test_dt_fraction_at_upper_clamp():
    # softplus(z) > 0.1  <=>  z > log(e^0.1 - 1) = -2.2522; with z ~ N(-2, 1)
    # about 60% of dt sits exactly at the clamp
    t = make_inputs(small(CONFIGS[1]), seed=1)
    frac = float((t["dt"] == torch.tensor(0.1, dtype=torch.float32)).float().mean())
    thr = math.log(math.expm1(0.1))
    expect = 0.5 * math.erfc((thr + 2.0) / math.sqrt(2))
    assert abs(frac - expect) < 0.01


def test_reproducible_and_seed_dependent():
    cfg = small(CONFIGS[4])
    a = make_inputs(cfg, seed=3)
    b = make_inputs(cfg, seed=3)
    c = make_inputs(cfg, seed=4)
    for k in a:
        if a[k] is None:
            continue
        assert torch.equal(a[k], b[k])
    assert not torch.equal(a["x"], c["x"])
