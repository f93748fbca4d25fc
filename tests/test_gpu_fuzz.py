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

import block_sparse_attention_kap_amd as cosa
import oracle as O
from synth import make, ragged
from gpu_helpers import (check_lists, check_osk_units, gpu_kap, gpu_osk, oracle_lists, oshape,
                         pack_lists)

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


def _dev(x, cfg):
    t = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    return {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(t).cuda() for n in ("q", "k", "v")}


@pytest.mark.parametrize("seed", list(range(48)))
def test_random_shared_lists(seed):
    """GQA-shared lists on a random problem: the proxy's per-KV-head lists against the oracle's
    group selection, then the shared-list walk bitwise equal to the per-head walk handed the
    same list (outputs, LSE, status traces, tile counts)."""
    cfg, kw_kap, kw_osk, causal = _case(seed)
    print(f"fuzz shared {seed}: {cfg} kap={kw_kap} osk={kw_osk} causal={causal}", flush=True)
    x = make(cfg)
    xd = _dev(x, cfg)
    kp = O.KapParams(**kw_kap)
    B, G = cfg["block"], cfg["q_heads"] // cfg["kv_heads"]
    scale = float(np.float32(1.0 / np.sqrt(cfg["head_dim"])))
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=B, budget=kp.budget, pool=kp.pool,
                                 agg_mode=kp.agg_mode, order_mode=kp.order_mode, causal=causal,
                                 scale=scale, return_scores=True, share_kv=True)
    torch.cuda.synchronize()
    sh = oshape(cfg, causal)
    want = {(b, g): O.kap_kv_group(x["q"][b, g * G:(g + 1) * G], x["k"][b, g], sh, kp)
            for b in range(cfg["batch"]) for g in range(cfg["kv_heads"])}
    check_lists(want, dict(idx=idx, cnt=cnt, hrm=hrm, sc=sc))
    kw = dict(block=B, tight_budget=kw_osk["tight_budget"], cap_mode=kw_osk["cap_mode"],
              skip_mode=kw_osk["skip_mode"], skip_param=kw_osk["skip_param"], causal=causal,
              scale=scale, return_lse=True, return_status=True, return_counts=True,
              vote_rows=kw_osk["vote_rows"])
    shared = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, shared_lists=True, **kw)
    per_head = cosa.osk(xd["q"], xd["k"], xd["v"], idx.repeat_interleave(G, dim=1).contiguous(),
                        cnt.repeat_interleave(G, dim=1).contiguous(), **kw)
    torch.cuda.synchronize()
    for a, b_ in zip(shared, per_head):
        assert torch.equal(a, b_)


@pytest.mark.parametrize("seed", list(range(48)))
def test_random_prefill_equals_serial(seed):
    """cosa_prefill on a random problem (a random grouping of the KV heads, per-head or shared
    lists) gives bitwise the lists, outputs and LSE of the proxy and the walk called in turn."""
    cfg, kw_kap, kw_osk, causal = _case(seed)
    r = np.random.default_rng(11000 + seed)
    hk = cfg["kv_heads"]
    chunks = int(r.choice([c for c in range(1, hk + 1) if hk % c == 0]))
    share = bool(r.random() < 0.5)
    print(f"fuzz prefill {seed}: {cfg} chunks={chunks} share={share} causal={causal}", flush=True)
    xd = _dev(make(cfg), cfg)
    B = cfg["block"]
    scale = float(np.float32(1.0 / np.sqrt(cfg["head_dim"])))
    common = dict(block=B, scale=scale, causal=causal)
    walk = dict(tight_budget=kw_osk["tight_budget"], cap_mode=kw_osk["cap_mode"],
                skip_mode=kw_osk["skip_mode"], skip_param=kw_osk["skip_param"],
                vote_rows=kw_osk["vote_rows"])
    idx, cnt, hrm = cosa.kap(xd["q"], xd["k"], budget=kw_kap["budget"], share_kv=share, **common)
    out, lse = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, return_lse=True, shared_lists=share,
                        **common, **walk)
    torch.cuda.synchronize()
    out2, lse2, (idx2, cnt2, hrm2) = cosa.prefill(
        xd["q"], xd["k"], xd["v"], budget=kw_kap["budget"], head_chunks=chunks, share_kv=share,
        return_lse=True, return_lists=True, **common, **walk)
    torch.cuda.synchronize()
    for a, b_ in ((idx, idx2), (cnt, cnt2), (hrm, hrm2), (out, out2), (lse, lse2)):
        assert torch.equal(a, b_)


@pytest.mark.parametrize("seed", list(range(32)))
def test_random_varlen_batch(seed):
    """A random varlen batch (2 to 5 entries of random lengths, NaN in every padding row, so any
    read of one would reach the outputs): per entry, the lists against the oracle's and the walk
    on them by trace replay and tolerance; blocks past an entry's end get empty lists and leave
    their output rows untouched."""
    cfg, kw_kap, kw_osk, causal = _case(seed)
    r = np.random.default_rng(13000 + seed)
    B = cfg["block"]
    Np = cfg["seq_len"]                          # padded length (a multiple of the block)
    lens = [int(v) for v in r.integers(1, Np + 1, size=int(r.integers(2, 6)))]
    cfg = {k: v for k, v in cfg.items() if k != "take"}
    cfg.update(batch=len(lens), seq_len=Np)
    print(f"fuzz varlen {seed}: lens={lens} {cfg} kap={kw_kap} osk={kw_osk} causal={causal}", flush=True)
    x = make(cfg)
    xp = {}
    for n_ in ("q", "k", "v"):
        a = x[n_].copy()
        for b, L in enumerate(lens):
            a[b, :, L:] = np.nan
        xp[n_] = a
    xd = _dev(xp, cfg)
    kp = O.KapParams(**kw_kap)
    op = O.OskParams(**kw_osk)
    scale = float(np.float32(1.0 / np.sqrt(cfg["head_dim"])))
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=B, budget=kp.budget, pool=kp.pool,
                                 agg_mode=kp.agg_mode, order_mode=kp.order_mode, causal=causal,
                                 scale=scale, return_scores=True, seq_lens=lens)
    sentinel = 7.0
    out = torch.full_like(xd["q"], sentinel)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=B,
                                tight_budget=op.tight_budget, cap_mode=op.cap_mode,
                                skip_mode=op.skip_mode, skip_param=op.skip_param, causal=causal,
                                scale=scale, return_lse=True, return_status=True, return_counts=True,
                                out=out, vote_rows=op.vote_rows, seq_lens=lens)
    torch.cuda.synchronize()
    o_all = out.float().cpu().numpy()
    for b, L in enumerate(lens):
        nbb = -(-L // B)
        cb = dict(cfg, batch=1, seq_len=nbb * B, take=L)
        xb = {n_: np.ascontiguousarray(x[n_][b:b + 1, :, :L]) for n_ in ("q", "k", "v")}
        g = dict(idx=idx[b:b + 1, :, :nbb].contiguous(), cnt=cnt[b:b + 1, :, :nbb].contiguous(),
                 hrm=hrm[b:b + 1, :, :nbb].contiguous(), sc=sc[b:b + 1, :, :nbb].contiguous())
        check_lists(oracle_lists(xb, cb, kp, causal=causal), g)
        assert (cnt[b, :, nbb:] == 0).all() and (idx[b, :, nbb:] == -1).all()
        assert (st[b, :, nbb:] == 0).all() and (tc[b, :, nbb:] == 0).all()
        assert np.all(o_all[b, :, L:] == sentinel)
        res = dict(out=o_all[b:b + 1, :, :L], lse=lse[b:b + 1, :, :L].cpu().numpy(),
                   st=st[b:b + 1, :, :nbb].cpu().numpy(), tc=tc[b:b + 1, :, :nbb].cpu().numpy())
        check_osk_units(xb, cb, op, g["idx"].cpu().numpy(), g["cnt"].cpu().numpy(), res, causal=causal)
