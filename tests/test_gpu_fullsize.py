"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

The whole hot path (KAP then OSK on the KAP lists, default skip rule) runs on the full
workload; every list is checked for the invariants that hold at any size, and every
(head, query block) unit is compared with the oracle, on a pool of worker processes
(tests/oracle_pool.py), also at the largest sequence the library takes.  The dense kernel at
128K is compared on sampled units.
"""
import time

import numpy as np
import pytest
import torch

import oracle as O
from synth import config, make
from synth.inputs import shrink
from gpu_helpers import TOL_LSE, out_excess, oshape, scale_of, upload
import block_sparse_attention_kap_amd as cosa
import oracle_pool as oracle_pool_mod

pytestmark = pytest.mark.gpu


def _list_invariants(idx, cnt, hrm, cfg, budget):
    nb = cfg["seq_len"] // cfg["block"]
    n = np.arange(1, nb + 1)
    want = np.minimum(n, np.maximum(1, np.ceil(budget * n))).astype(np.int32)
    assert (cnt == want[None, None, :]).all()
    kmax = idx.shape[-1]
    pos = np.arange(kmax)[None, None, None, :]
    valid = pos < cnt[..., None]
    assert (idx[~valid] == -1).all()
    blk = np.arange(nb)[None, None, :, None]
    assert ((idx >= 0) & (idx <= blk))[valid].all()
    s = np.sort(np.where(valid, idx, -1 - pos), axis=-1)
    assert (np.diff(s, axis=-1) != 0).all()              # distinct entries
    assert (hrm >= 1).all() and (hrm <= cfg["block"]).all()


def _host(t):
    """A device tensor on the host as numpy (bf16 as its raw 16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _every_unit(pool, cfg, share=False, vote_rows=0, splits=1):
    """KAP then OSK on the whole workload in the launch configuration bench.py times, then every
    (head, query block) unit compared with the oracle on the pool's worker processes: the list
    through the tie-band comparator, the walk by status-trace replay, counts, outputs, LSE.
    splits > 1 cuts each head's query blocks into that many jobs (for few heads)."""
    from oracle_pool import check_head
    t0 = time.perf_counter()
    x = make(cfg)
    xd = upload(x, cfg)
    del x
    B = cfg["block"]
    kp = O.KapParams(budget=cfg["budget"])
    op = O.OskParams(tight_budget=cfg["tight_budget"], vote_rows=vote_rows)
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=B, budget=kp.budget, scale=scale_of(cfg),
                                 return_scores=True, share_kv=share)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=B,
                                tight_budget=op.tight_budget, scale=scale_of(cfg), return_lse=True,
                                return_status=True, return_counts=True, vote_rows=vote_rows,
                                shared_lists=share)
    torch.cuda.synchronize()
    idx, cnt, hrm, sc = (t.cpu().numpy() for t in (idx, cnt, hrm, sc))
    st, tc, lse, out = st.cpu().numpy(), tc.cpu().numpy(), lse.cpu().numpy(), _host(out)
    del xd
    torch.cuda.empty_cache()
    _list_invariants(idx, cnt, hrm, cfg, cfg["budget"])
    print(f"{cfg['name']}: GPU done in {time.perf_counter() - t0:.1f}s, checking every unit on "
          f"{pool._processes} workers", flush=True)
    G = cfg["q_heads"] // cfg["kv_heads"]
    kap_kw = dict(budget=kp.budget)
    osk_kw = dict(tight_budget=op.tight_budget, vote_rows=vote_rows)
    jobs = []
    nb = cfg["seq_len"] // B
    # heavier (later) blocks get shorter ranges: cut where the causal work sum(i) splits evenly
    cuts = [0] + [int(nb * (s / splits) ** 0.5) for s in range(1, splits)] + [nb]
    for b in range(cfg["batch"]):
        for h in range(cfg["q_heads"]):
            lh = h // G if share else h
            for lo, hi in zip(cuts[:-1], cuts[1:]):
                part = {} if splits == 1 else dict(blocks=(lo, hi))
                rows = slice(lo * B, hi * B)
                jobs.append(dict(cfg=cfg, kap=kap_kw, osk=osk_kw, b=b, h=h, share=share,
                                 idx=idx[b, lh], cnt=cnt[b, lh], hrm=hrm[b, lh], sc=sc[b, lh],
                                 st=st[b, h], tc=tc[b, h], out=out[b, h][rows], lse=lse[b, h][rows],
                                 **part))
    tot = dict(units=0, skipped=0, replays=0, excess=-1.0, flat=0.0, flat_r=0.0, n_flat=0,
               n_flat_r=0, elements=0, lse=0.0, max_abs_out=0.0)
    bad = []
    for r in pool.imap_unordered(check_head, jobs):
        for kk in ("units", "skipped", "replays", "n_flat", "n_flat_r", "elements"):
            tot[kk] += r[kk]
        for kk in ("excess", "flat", "flat_r", "lse", "max_abs_out"):
            tot[kk] = max(tot[kk], r[kk])
        bad += r["bad"]
        print(f"  head {r['h']}: {r['units']} units, {r['n_bad']} rejected, "
              f"excess {r['excess']:.2e}, {r['seconds']:.1f}s", flush=True)
    line = (f"{cfg['name']}{' shared lists' if share else ''}{' 32-row votes' if vote_rows else ''}: "
            f"{tot} in {time.perf_counter() - t0:.1f}s")
    print(line, flush=True)
    oracle_pool_mod.SUMMARIES.append(line)
    assert not bad, f"rejected: {bad[:5]}"
    assert tot["units"] == cfg["batch"] * cfg["q_heads"] * (cfg["seq_len"] // B)
    assert tot["excess"] <= 0, tot
    assert tot["lse"] <= TOL_LSE[cfg["dtype"]], tot
    return tot


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_full_size_every_unit(ci, oracle_pool):
    """Every unit of the full-size workloads (8K, 32K, 128K, and the block-64 stress workload)
    against the oracle."""
    cfg = config(ci)
    print(f"full-size parity, every unit: {cfg['name']}", flush=True)
    _every_unit(oracle_pool, cfg)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,mode", [(3, "shared_kv"), (4, "shared_kv"), (2, "vote_rows_32")])
def test_full_size_modes_every_unit(ci, mode, oracle_pool):
    """The GQA-shared lists (one list per KV head; at block 64 four query heads per workgroup,
    the second workgroup of a 7-head group one head short) and the 32-row skip votes, every unit
    at full size."""
    cfg = config(ci)
    print(f"full-size parity, every unit: {cfg['name']} {mode}", flush=True)
    _every_unit(oracle_pool, cfg, share=mode == "shared_kv", vote_rows=32 if mode == "vote_rows_32" else 0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,seq_len", [(4, 4096 * 64), (3, 4096 * 128)])
def test_max_blocks_every_unit(ci, seq_len, oracle_pool):
    """The largest sequence the library takes: 4096 blocks (the staged list, the select
    kernel and the proxy workspace at their limits), one query head, every unit."""
    cfg = shrink(config(ci), seq_len, q_heads=1, kv_heads=1)
    assert cfg["seq_len"] // cfg["block"] == 4096
    print(f"maximum-size parity: {cfg['name']}", flush=True)
    _every_unit(oracle_pool, cfg, splits=2 * oracle_pool._processes)


@pytest.mark.parametrize("ci", [3])
def test_full_size_dense_sampled(ci):
    cfg = config(ci)
    x = make(cfg)
    xd = upload(x, cfg)
    out = cosa.dense(xd["q"], xd["k"], xd["v"], block=cfg["block"], scale=scale_of(cfg))
    torch.cuda.synchronize()
    sh = oshape(cfg)
    G = cfg["q_heads"] // cfg["kv_heads"]
    B = cfg["block"]
    nb = cfg["seq_len"] // B
    worst = -1.0
    for h, i in [(0, nb - 1), (G + 1, nb // 2), (31, 3)]:
        blocks = list(range(i + 1))
        o, _ = O.restricted_attention(x["q"][0, h][i * B:(i + 1) * B], x["k"][0, h // G],
                                      x["v"][0, h // G], i, blocks, sh)
        worst = max(worst, out_excess(out[0, h, i * B:(i + 1) * B].float().cpu().numpy(), o, "bf16"))
    assert worst <= 0, worst


def test_full_size_prefill_equals_serial():
    """cosa_prefill at 128K over four groups of KV heads: bitwise the proxy and the walk called
    one after the other (lists, output, LSE)."""
    cfg = config(3)
    print(f"full-size prefill: {cfg['name']}", flush=True)
    xd = upload(make(cfg), cfg)
    B = cfg["block"]
    idx, cnt, hrm = cosa.kap(xd["q"], xd["k"], block=B, budget=cfg["budget"], scale=scale_of(cfg))
    out, lse = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=B,
                        tight_budget=cfg["tight_budget"], scale=scale_of(cfg), return_lse=True)
    torch.cuda.synchronize()
    out2, lse2, (idx2, cnt2, hrm2) = cosa.prefill(
        xd["q"], xd["k"], xd["v"], block=B, budget=cfg["budget"], tight_budget=cfg["tight_budget"],
        head_chunks=4, scale=scale_of(cfg), return_lse=True, return_lists=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2) and torch.equal(hrm, hrm2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
