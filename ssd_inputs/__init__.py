"""Seeded synthetic inputs for the SSD forward pass.

This module is shared by the tests, the benchmark and the oracle-side scripts.
It draws random inputs and nothing else: it holds none of the operator's
arithmetic (no decay, no cumulative sum, no contraction).

The five workloads
------------------
``CONFIGS`` lists the five workloads used for parity and measurement, named by
what they are. Every workload draws, in this order, from one CPU
``torch.Generator`` seeded with the workload's index (or the given seed):

  x    ~ N(0, 1)                                    [batch, L, H, P]
  dt   = clamp(softplus(N(dt_mu, 1)), dt_lo, dt_hi) [batch, L, H]
  A_h  = -exp(U(ln 1, ln 16))                       [H]
  B, C ~ N(0, 1) / sqrt(N)                          [batch, L, G, N]
  D    ~ N(0, 1)                                    [H]
  h0   ~ 0.1 * N(0, 1)  (only where the workload has an initial state)
                                                    [batch, H, P, N]

all drawn in fp32; x, B and C are then rounded to bf16 (round to nearest even)
for the bf16 workloads. dt, A, D and the states always stay fp32. softplus is
log(1 + e^z) with beta = 1, applied before the clamp. The dt distribution is
an input recipe (the operator itself takes dt as given).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import torch

__all__ = ["SSDConfig", "CONFIGS", "make_inputs", "config_by_name"]


@dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    io_dtype: str          # "fp32" or "bf16" (dtype of x, B, C, y)
    dt_mu: float = -2.0
    dt_lo: float = 1e-3
    dt_hi: float = 0.1
    init_state: bool = False

    def as_dict(self):
        return asdict(self)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "SSDConfig":
        d = asdict(self)
        d.update(kw)
        return SSDConfig(**d)


CONFIGS = [
    SSDConfig("tiny-fp32", 1, 256, 4, 16, 16, 1, "fp32"),
    SSDConfig("mamba2-1.3b-layer", 8, 2048, 64, 64, 128, 1, "bf16"),
    SSDConfig("long-prefill-64k", 1, 65536, 64, 64, 128, 1, "bf16", init_state=True),
    SSDConfig("large-state-grouped", 4, 8192, 128, 64, 256, 8, "bf16"),
    SSDConfig("small-state-many-seq", 32, 4096, 32, 64, 64, 1, "bf16",
              dt_mu=-3.0, dt_lo=1e-4, dt_hi=0.1, init_state=True),
]


def config_by_name(name: str) -> SSDConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def make_inputs(cfg: SSDConfig, seed: int | None = None, device="cpu"):
    """Draw one batch of inputs for ``cfg``.

    Returns a dict of tensors: x, dt, A, B, C, D, init_state (None when the
    workload has none). Draws happen on the CPU in the fixed order above, so
    the values do not depend on ``device``; they are then moved to it.
    """
    if seed is None:
        seed = CONFIGS.index(cfg) if cfg in CONFIGS else 0
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    b, L, H, P, N, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.dstate, cfg.ngroups
    f32 = torch.float32
    x = torch.randn((b, L, H, P), generator=g, dtype=f32)
    z = torch.randn((b, L, H), generator=g, dtype=f32) + cfg.dt_mu
    dt = torch.nn.functional.softplus(z).clamp_(cfg.dt_lo, cfg.dt_hi)
    u = torch.rand((H,), generator=g, dtype=f32)
    A = -torch.exp(u * (math.log(16.0) - math.log(1.0)) + math.log(1.0))
    Bm = torch.randn((b, L, G, N), generator=g, dtype=f32) / math.sqrt(N)
    Cm = torch.randn((b, L, G, N), generator=g, dtype=f32) / math.sqrt(N)
    D = torch.randn((H,), generator=g, dtype=f32)
    h0 = 0.1 * torch.randn((b, H, P, N), generator=g, dtype=f32) if cfg.init_state else None
    if cfg.io_dtype == "bf16":
        x, Bm, Cm = x.to(torch.bfloat16), Bm.to(torch.bfloat16), Cm.to(torch.bfloat16)
    elif cfg.io_dtype != "fp32":
        raise ValueError(cfg.io_dtype)
    out = dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, init_state=h0)
    if device != "cpu":
        out = {k: (v.to(device) if v is not None else None) for k, v in out.items()}
    return out
