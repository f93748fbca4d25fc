"""Synthetic ablation of the proxy/kernel co-design, on the GPU.

The technical summary of the paper (gist.science, pt, section 4, ablation studies)
reports that ordering by the proxy alone improves accuracy, that in-kernel skipping
adds sparsity, and that the combination keeps accuracy while tightening the budget.
The datasets and models are not used here; this script measures the same effects on
the synthetic workloads, against the dense kernel on the same inputs:

  A  top-k proxy   plain top-k by block score at the tight budget, natural
                   use of the list (no skipping)          -- a single-criterion mask
  B  KAP order     HRM-first top-k at the tight budget, no skipping
  C  KAP + cap     HRM-first top-k at the moderate budget, walk capped at the
                   tight budget (ordered truncation), no skipping
  D  CoSA          C plus the in-kernel skip test (MASS, eps 1e-3), the tight budget
                   capping the visited blocks (a skipped block saves its P.V without
                   extending the walk: skipping raises the sparsity)
  E  threshold     HRM-first top-k at the moderate budget, no cap, skip test only
                   (MASS, eps 1e-2)
  F  CoSA, groups  D with the skip test voted per group of 32 query rows instead of
                   per block of B rows (one outlier row vetoes less)
  G  CoSA, shared  D with one list per KV head, built from the pooled rows of all its
                   query heads and walked by each of them (GQA-shared lists)
  H  CoSA, computed D with the cap counted in computed blocks instead of visited ones:
                   a skipped block then extends the walk to the next listed block

--sweep instead compares the two skip tests over their thresholds: MASS with eps in
{1e-4, 1e-3, 1e-2, 1e-1} and MAXDIFF with tau in {-8, -4, -2, 0}, each with the
moderate list and no cap (pure threshold skipping) and with the tightened cap.

Every variant computes at most the same number of blocks per query block as A.
Metrics per variant: captured attention mass per query row, exp(LSE - LSE_dense),
as mean and 1st percentile; output error against the dense output (mean and max
abs); fraction of causal blocks visited and computed; OSK time.

    python ablation.py --config 2
    python ablation.py --config 1 --concentrated
    python ablation.py --config 1 --concentrated --sweep
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--seq-len", type=int, default=0, help="shrink the workload to this length")
    ap.add_argument("--concentrated", action="store_true",
                    help="planted keys 12x stronger, query noise 0.2 (skipping fires)")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--sweep", action="store_true", help="MASS / MAXDIFF threshold sweep")
    args = ap.parse_args()

    import numpy as np
    import torch

    import block_sparse_attention_kap_amd as cosa
    from synth import config, make, shrink

    cfg = config(args.config)
    if args.seq_len:
        cfg = shrink(cfg, args.seq_len)
    if args.concentrated:
        cfg.update(salient_gain=12.0, q_noise=0.2)
        cfg["name"] += "+concentrated"
    x = make(cfg)
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(tdt).cuda() for n in ("q", "k", "v"))
    B = cfg["block"]
    D = cfg["head_dim"]
    nb = cfg["seq_len"] // B
    scale = float(np.float32(1.0 / np.sqrt(D)))
    rho, rho_t = cfg["budget"], cfg["tight_budget"]
    od, lsed = cosa.dense(q, k, v, block=B, scale=scale, return_lse=True)
    od = od.float()
    n_cand = cfg["batch"] * cfg["q_heads"] * nb * (nb + 1) // 2

    if args.sweep:
        variants = []
        for cap in (rho, rho_t):
            tag = "no cap" if cap == rho else "cap rho'"
            variants += [(f"MASS eps={e:g}, {tag}", dict(budget=rho, order_mode=0),
                          dict(tight=cap, skip=2, eps=e)) for e in (1e-4, 1e-3, 1e-2, 1e-1)]
            variants += [(f"MAXDIFF tau={t:g}, {tag}", dict(budget=rho, order_mode=0),
                          dict(tight=cap, skip=1, eps=t)) for t in (-8.0, -4.0, -2.0, 0.0)]
            variants += [(f"skip off, {tag}", dict(budget=rho, order_mode=0), dict(tight=cap, skip=0, eps=1e-3))]
    else:
        variants = [
            ("A top-k proxy", dict(budget=rho_t, order_mode=1), dict(tight=rho_t, skip=0, eps=1e-3)),
            ("B KAP order", dict(budget=rho_t, order_mode=0), dict(tight=rho_t, skip=0, eps=1e-3)),
            ("C KAP + cap", dict(budget=rho, order_mode=0), dict(tight=rho_t, skip=0, eps=1e-3)),
            ("D CoSA", dict(budget=rho, order_mode=0), dict(tight=rho_t, skip=2, eps=1e-3, cap=1)),
            ("E threshold", dict(budget=rho, order_mode=0), dict(tight=rho, skip=2, eps=1e-2)),
            ("F CoSA, groups", dict(budget=rho, order_mode=0), dict(tight=rho_t, skip=2, eps=1e-3, votes=32, cap=1)),
            ("G CoSA, shared", dict(budget=rho, order_mode=0, share=True), dict(tight=rho_t, skip=2, eps=1e-3, cap=1)),
            ("H CoSA, computed cap", dict(budget=rho, order_mode=0), dict(tight=rho_t, skip=2, eps=1e-3, cap=0)),
        ]
    rows = []
    for name, kw, ow in variants:
        share = kw.get("share", False)
        idx, cnt, _ = cosa.kap(q, k, block=B, budget=kw["budget"], scale=scale,
                               order_mode=kw["order_mode"], share_kv=share)
        vr = ow.get("votes", 0) if cfg["dtype"] == "bf16" else 0
        cap = ow.get("cap", 1)
        o, lse, tc = cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=ow["tight"],
                              skip_mode=ow["skip"], skip_param=ow["eps"], scale=scale,
                              return_lse=True, return_counts=True, vote_rows=vr,
                              shared_lists=share, cap_mode=cap)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.reps)]
        for a_, b_ in ev:
            a_.record()
            cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=ow["tight"], skip_mode=ow["skip"],
                     skip_param=ow["eps"], scale=scale, out=o, vote_rows=vr, shared_lists=share,
                     cap_mode=cap)
            b_.record()
        torch.cuda.synchronize()
        ms = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev]))
        rec = torch.exp(lse - lsed).flatten()
        err = (o.float() - od).abs()
        t = tc.to(torch.int64).sum(dim=(0, 1, 2)).cpu().numpy().astype(np.float64)
        if vr:
            t[1] /= B // vr          # computed row-group tiles -> block-tile equivalents
        row = dict(variant=name, workload=cfg["name"],
                   mass_mean=round(float(rec.mean()), 5),
                   mass_p01=round(float(torch.quantile(rec[:: max(1, rec.numel() // 1_000_000)].float(), 0.01)), 5),
                   mean_abs=round(float(err.mean()), 5),
                   max_abs=round(float(err.max()), 4),
                   visited=round(int(t[0]) / n_cand, 4), computed=round(int(t[1]) / n_cand, 4),
                   osk_ms=round(ms, 3))
        rows.append(row)
        print(json.dumps(row), flush=True)
    print(f"\n| {cfg['name']} | mass mean | mass p01 | mean abs err | max abs err | visited | computed | OSK ms |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['variant']} | {r['mass_mean']} | {r['mass_p01']} | {r['mean_abs']} | {r['max_abs']} "
              f"| {r['visited']} | {r['computed']} | {r['osk_ms']} |")


if __name__ == "__main__":
    main()
