"""GPU: seeded random small problems, end to end against the oracle.

Each case draws its own shape and options from a fixed seed: block 64 or 128, head dim 64 or 128,
bf16 or fp32, query/KV head counts with GQA groups of 1 to 7, 2 to 9 blocks with a ragged last
block, causal or not, iid or planted-salient inputs, budgets, pooling size, SUM or MAX
aggregation, HRM-first or score-only order, MASS or MAXDIFF or no skip test, both caps and (bf16)
32-row votes.  The proxy's lists go through the tie-band comparator against the oracle's; the walk
runs on the oracle's lists and is checked by status-trace replay and output/LSE tolerance, the
same comparisons the named parity cases use.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import make, ragged
from gpu_helpers import check_lists, check_osk_units, gpu_kap, gpu_osk, oracle_lists, pack_lists

pytestmark = pytest.mark.gpu

SEEDS = list(range(96))


def _case(seed):
    r = np.random.default_rng(7000 + seed)
    block = int(r.choice([64, 128]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "bf16", "f32"]))
    hq, hk = [(1, 1), (2, 1), (4, 2), (3, 3), (7, 1), (8, 2)][int(r.integers(6))]
    nblk = int(r.integers(2, 10))
    full = nblk * block
    L = int(r.integers(full - block + 1, full + 1))
    budget = float(r.uniform(0.1, 1.0))
    tight = float(r.uniform(0.05, budget))
    cfg = dict(name=f"fuzz{seed}", batch=1, q_heads=hq, kv_heads=hk, seq_len=full, head_dim=D,
               block=block, dtype=dtype, budget=budget, tight_budget=tight, seed=9000 + seed)
    if r.random() < 0.5:
        cfg.update(structure="salient", n_salient=int(r.integers(1, nblk)), sink=bool(r.random() < 0.5),
                   window=int(r.integers(0, 3)), salient_gain=float(r.uniform(2.0, 12.0)))
    else:
        cfg.update(structure="iid")
    if L != full:
        cfg = ragged(cfg, L)
    kw_kap = dict(budget=budget, pool=int(r.choice([0, 0, 16])),
                  agg_mode=int(r.choice([O.AGG_SUM, O.AGG_SUM, O.AGG_MAX])),
                  order_mode=int(r.choice([O.ORDER_HRM_FIRST, O.ORDER_HRM_FIRST, O.ORDER_SCORE])))
    skip = int(r.choice([O.SKIP_OFF, O.SKIP_MASS, O.SKIP_MASS, O.SKIP_MAXDIFF]))
    kw_osk = dict(tight_budget=tight, skip_mode=skip,
                  skip_param=-2.0 if skip == O.SKIP_MAXDIFF else float(r.choice([1e-3, 1e-2])),
                  cap_mode=int(r.choice([O.COMPUTED, O.VISITED])),
                  vote_rows=int(r.choice([0, 32])) if dtype == "bf16" else 0)
    causal = bool(r.random() < 0.75)
    return cfg, kw_kap, kw_osk, causal


@pytest.mark.parametrize("seed", SEEDS)
def test_random_problem_matches_oracle(seed):
    cfg, kw_kap, kw_osk, causal = _case(seed)
    print(f"fuzz {seed}: {cfg} kap={kw_kap} osk={kw_osk} causal={causal}", flush=True)
    x = make(cfg)
    t = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    xd = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(t).cuda() for n in ("q", "k", "v")}
    kp = O.KapParams(**kw_kap)
    units = oracle_lists(x, cfg, kp, causal=causal)
    check_lists(units, gpu_kap(xd, cfg, kp, causal=causal))
    op = O.OskParams(**kw_osk)
    kmax = max(u["k"] for us in units.values() for u in us)
    idx, cnt = pack_lists(units, cfg, kmax)
    res = gpu_osk(xd, cfg, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), op, causal=causal)
    print(check_osk_units(x, cfg, op, idx, cnt, res, causal=causal), flush=True)
