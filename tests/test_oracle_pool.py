"""CPU checks of the whole-output parity machinery (tests/oracle_pool.py):
the head blocks it hands to workers map heads to the right B/C groups, the
pooled comparison of the oracle's own outputs gives zero error, and one
changed element in any single chain is caught."""

import numpy as np
import pytest
import torch

from oracle import ssd_recurrent
from oracle_pool import compare_all, head_blocks
from ssd_inputs import CONFIGS, make_inputs


@pytest.mark.parametrize("H,G,block", [(64, 1, 16), (128, 8, 16), (16, 16, 16), (6, 2, 16), (32, 4, 4), (12, 3, 8)])
def test_head_blocks_stay_inside_or_cover_whole_groups(H, G, block):
    hpg = H // G
    blocks = head_blocks(H, G, block)
    assert [h for a, e in blocks for h in range(a, e)] == list(range(H))
    for a, e in blocks:
        groups = {h // hpg for h in range(a, e)}
        if len(groups) > 1:  # whole groups only
            assert a % hpg == 0 and e % hpg == 0


def _case(G, H, seed):
    cfg = CONFIGS[1].with_(batch=2, seqlen=67, nheads=H, headdim=16, dstate=16, ngroups=G, init_state=True)
    inp = make_inputs(cfg, seed=seed)
    y, hT = ssd_recurrent(*(inp[k] for k in ("x", "dt", "A", "B", "C", "D", "init_state")))
    return inp, y, hT


@pytest.mark.parametrize("G,H", [(1, 8), (2, 8), (8, 8)])
def test_pooled_comparison_of_the_oracle_with_itself_is_exact(G, H):
    inp, y, hT = _case(G, H, seed=5)
    r = compare_all(inp, torch.tensor(y), torch.tensor(hT), 2.0 ** -8, block=4)
    assert r["chains"] == 2 * H and r["finite"]
    assert r["y"] == 0.0 and r["ssm"] == 0.0 and r["final_state"] == 0.0


@pytest.mark.parametrize("where", ["y", "state"])
def test_one_changed_element_in_one_chain_is_caught(where):
    inp, y, hT = _case(2, 8, seed=6)
    y, hT = y.copy(), hT.copy()
    if where == "y":
        y[1, 40, 5, 3] += 0.05 * np.abs(y).max()
    else:
        hT[1, 6, 2, 9] += 0.05 * np.abs(hT).max()
    r = compare_all(inp, y, hT, 2.0 ** -8, block=4)
    key = "y" if where == "y" else "final_state"
    assert r[key] > 2e-2
