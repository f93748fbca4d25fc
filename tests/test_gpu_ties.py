"""GPU: exact ties in the proxy scores.

With every query zero, or every key row of a head the same vector, a pooled query row scores
the same against every key block.  Every block then attains the row maximum (the HRM flag goes
to the lowest index, block 0) and every block's MaxNorm sum is the same, so the visiting order
is decided by the block index alone.  Lists are compared with the oracle's element by element,
without the tie band the other parity tests allow: that pins the lowest-index rule of the row
argmax and the block-index tiebreak of the selection, which a tie band would accept in any
order.  Budgets of 0.3 and 1.0 make the radix select resolve its threshold in the block-index
bits of the sort key (every round of digits) or take every block.
"""
import numpy as np
import pytest

import oracle as O
from synth import config, make, ragged, shrink
from gpu_helpers import gpu_kap, oracle_lists, upload

pytestmark = pytest.mark.gpu


def _cfg(name):
    if name == "gqa_b128":
        return shrink(config(1), 2304, q_heads=4, kv_heads=2, n_salient=3)
    if name == "stress_b64":
        return shrink(config(4), 4096, q_heads=7, kv_heads=1)
    if name == "ragged_b128":
        return ragged(shrink(config(1), 2304, q_heads=4, kv_heads=2, n_salient=3), 2216)
    raise KeyError(name)


def _tied_inputs(name, how):
    cfg = _cfg(name)
    x = make(cfg)
    if how == "zero_q":
        x["q"] = np.zeros_like(x["q"])
    else:   # every key row of a head equal to its first row
        x["k"] = np.repeat(x["k"][:, :, :1, :], x["k"].shape[2], axis=2)
    return cfg, x, upload(x, cfg)


@pytest.mark.parametrize("name", ["gqa_b128", "stress_b64", "ragged_b128"])
@pytest.mark.parametrize("how", ["zero_q", "same_k"])
@pytest.mark.parametrize("kw", [dict(budget=0.3), dict(budget=1.0), dict(budget=0.3, agg_mode=O.AGG_MAX),
                                dict(budget=0.3, order_mode=O.ORDER_SCORE),
                                dict(budget=0.3, force_sink=True, force_diag=True)])
def test_tied_scores_order_by_block_index(name, how, kw):
    print(f"ties: {name} {how} {kw}", flush=True)
    cfg, x, xd = _tied_inputs(name, how)
    kp = O.KapParams(**kw)
    g = gpu_kap(xd, cfg, kp)
    idx, cnt, hrm = (g[n].cpu().numpy() for n in ("idx", "cnt", "hrm"))
    units = oracle_lists(x, cfg, kp)
    plain = not (kw.get("force_sink") or kw.get("force_diag"))
    for (b, h), us in units.items():
        for i, u in enumerate(us):
            k = u["k"]
            if plain:   # the oracle itself: HRM is block 0, the rest by index
                assert list(u["list"]) == list(range(k)), (b, h, i)
                assert u["hrm_cnt"] == 1
            assert int(cnt[b, h, i]) == k, (b, h, i)
            assert np.array_equal(idx[b, h, i, :k], u["list"]), (b, h, i, idx[b, h, i, :k], u["list"])
            assert (idx[b, h, i, k:] == -1).all()
            assert int(hrm[b, h, i]) == u["hrm_cnt"], (b, h, i)
