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


def _packed(lengths, seed):
    from ssd_inputs import make_inputs as mk
    cfg = CONFIGS[1].with_(batch=1, seqlen=sum(lengths), nheads=8, headdim=16, dstate=16, ngroups=2)
    inp = mk(cfg, seed=seed)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ys, hs = [], []
    for s in range(len(lengths)):
        a, e = cu[s], cu[s + 1]
        if a == e:
            ys.append(np.zeros((1, 0, 8, 16)))
            hs.append(np.zeros((1, 8, 16, 16)))
            continue
        y, hT = ssd_recurrent(*(inp[k][:, a:e] for k in ("x", "dt")), inp["A"],
                              *(inp[k][:, a:e] for k in ("B", "C")), inp["D"], None)
        ys.append(y)
        hs.append(hT)
    return inp, cu, np.concatenate(ys, axis=1), np.concatenate(hs, axis=0)


def test_packed_comparison_of_per_sequence_oracle_runs_is_exact():
    inp, cu, y, hT = _packed([5, 0, 17, 1, 0, 9], seed=7)
    from oracle_pool import compare_packed
    r = compare_packed(inp, cu, y, hT, 2.0 ** -8, block=4)
    assert r["chains"] == 4 * 8 and r["finite"] and r["empty_ok"]
    assert r["y"] == 0.0 and r["ssm"] == 0.0 and r["final_state"] == 0.0


@pytest.mark.parametrize("where", ["y", "state", "empty"])
def test_packed_comparison_catches_one_changed_element(where):
    from oracle_pool import compare_packed
    inp, cu, y, hT = _packed([5, 0, 17, 1, 0, 9], seed=8)
    y, hT = y.copy(), hT.copy()
    if where == "y":
        y[0, 22, 6, 3] += 0.05 * np.abs(y).max()  # the length-1 sequence's token
    elif where == "state":
        hT[5, 1, 2, 9] += 0.05 * np.abs(hT).max()
    else:
        hT[4, 0, 0, 0] = 1e-30  # an empty sequence's final state must be exactly zero
    r = compare_packed(inp, cu, y, hT, 2.0 ** -8, block=4)
    if where == "empty":
        assert not r["empty_ok"]
    else:
        assert r["y" if where == "y" else "final_state"] > 2e-2
