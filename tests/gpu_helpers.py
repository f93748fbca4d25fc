"""Shared helpers of the GPU parity tests: upload inputs, run the HIP path through
the binding, and compare unit by unit with the oracle (tie band + replay)."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_kap_amd as cosa
import oracle as O
from oracle.compare import check_list, replay_walk
from oracle_pool import output_check

TOL_OUT = {"bf16": 1e-2, "f32": 1e-4}
TOL_LSE = {"bf16": 1e-3, "f32": 1e-5}


# running totals of the flat error measures over the session (printed at its end)
FLAT_STATS = dict(elements=0, flat=0.0, flat_rounded=0.0, n_flat=0, n_flat_rounded=0)


def out_excess(got, ref, dtype):
    """Largest amount by which an output misses its tolerance (<= 0 passes).

    Two bounds, both required.  (1) The output is the storage rounding (RNE) of a value within
    the accumulation tolerance of the oracle (1e-2 for bf16 inputs with fp32 accumulation,
    1e-4 for fp32): its rounding interval meets [ref - tol, ref + tol].  (2) |got - ref| <= tol
    + 2^-9 |ref| for a bf16 output.  The flat errors against the oracle and against the oracle
    rounded to the output dtype are accumulated in FLAT_STATS.
    """
    e, f, fr, nf, nfr = output_check(got, ref, dtype)
    FLAT_STATS["elements"] += int(np.size(ref))
    FLAT_STATS["flat"] = max(FLAT_STATS["flat"], f)
    FLAT_STATS["flat_rounded"] = max(FLAT_STATS["flat_rounded"], fr)
    FLAT_STATS["n_flat"] += nf
    FLAT_STATS["n_flat_rounded"] += nfr
    tol = TOL_OUT[dtype] + (2.0 ** -9 * np.abs(ref) if dtype == "bf16" else 0.0)
    return max(e, float((np.abs(got - ref) - tol).max()))


def scale_of(cfg):
    return float(np.float32(1.0 / np.sqrt(cfg["head_dim"])))


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def upload(x, cfg):
    return {n: to_dev(x[n], cfg["dtype"]) for n in ("q", "k", "v")}


def oshape(cfg, causal=True):
    return O.Shape(cfg["batch"], cfg["q_heads"], cfg["kv_heads"], seq_len(cfg), cfg["head_dim"],
                   cfg["block"], causal, scale_of(cfg), cfg["dtype"])


def gpu_kap(xd, cfg, kp: O.KapParams, causal=True, kmax=None):
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=cfg["block"], budget=kp.budget,
                                 pool=kp.pool, pool_mode=kp.pool_mode, agg_mode=kp.agg_mode,
                                 force_sink=kp.force_sink, force_diag=kp.force_diag,
                                 causal=causal, scale=scale_of(cfg), kmax=kmax,
                                 return_scores=True, sel_mode=kp.sel_mode, mass=kp.mass,
                                 order_mode=kp.order_mode)
    torch.cuda.synchronize()
    return dict(idx=idx, cnt=cnt, hrm=hrm, sc=sc)


def gpu_osk(xd, cfg, idx, cnt, op: O.OskParams, causal=True, page_table=None, kv=None):
    k, v = (xd["k"], xd["v"]) if kv is None else kv
    out, lse, st, tc = cosa.osk(xd["q"], k, v, idx, cnt, block=cfg["block"],
                                tight_budget=op.tight_budget, cap_mode=op.cap_mode,
                                skip_mode=op.skip_mode, skip_param=op.skip_param,
                                page_table=page_table, causal=causal, scale=scale_of(cfg),
                                return_lse=True, return_status=True, return_counts=True,
                                vote_rows=op.vote_rows)
    torch.cuda.synchronize()
    return dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy(), st=st.cpu().numpy(),
                tc=tc.cpu().numpy())


def oracle_lists(x, cfg, kp, causal=True, heads=None, blocks=None):
    """Oracle KAP units for every (batch, head) -> {(b, h): [unit per block]}."""
    sh = oshape(cfg, causal)
    G = cfg["q_heads"] // cfg["kv_heads"]
    res = {}
    for b in range(cfg["batch"]):
        for h in (range(cfg["q_heads"]) if heads is None else heads):
            res[(b, h)] = O.kap_head(x["q"][b, h], x["k"][b, h // G], sh, kp, blocks)
    return res


def num_blocks(cfg):
    """Blocks per sequence; the last one is partial when the block does not divide it."""
    return -(-cfg["seq_len"] // cfg["block"])


def seq_len(cfg):
    return cfg.get("take", cfg["seq_len"])


def pack_lists(units_by_head, cfg, kmax):
    nb = num_blocks(cfg)
    idx = np.full((cfg["batch"], cfg["q_heads"], nb, kmax), -1, np.int32)
    cnt = np.zeros((cfg["batch"], cfg["q_heads"], nb), np.int32)
    for (b, h), units in units_by_head.items():
        for i, u in enumerate(units):
            idx[b, h, i, :u["k"]] = u["list"]
            cnt[b, h, i] = u["k"]
    return idx, cnt


def check_lists(units_by_head, g, blocks=None):
    idx, cnt, hrm, sc = (g[n].cpu().numpy() for n in ("idx", "cnt", "hrm", "sc"))
    bad = []
    n_units = 0
    for (b, h), units in units_by_head.items():
        for u, i in zip(units, range(len(units)) if blocks is None else blocks):
            ok, msg = check_list(u, idx[b, h, i], int(cnt[b, h, i]), int(hrm[b, h, i]), sc[b, h, i])
            n_units += 1
            if not ok:
                bad.append(f"(b={b}, h={h}, i={i}): {msg}")
    assert not bad, f"{len(bad)}/{n_units} lists rejected; first: {bad[:3]}"
    return n_units


def check_osk_units(x, cfg, op, idx, cnt, res, causal=True, heads=None, blocks=None,
                    page_table=None, kv_np=None):
    """Replay the oracle walk against the GPU's status trace for every unit and
    compare outputs.  idx/cnt: numpy lists the GPU consumed."""
    sh = oshape(cfg, causal)
    G = cfg["q_heads"] // cfg["kv_heads"]
    B = cfg["block"]
    nb = -(-seq_len(cfg) // B)
    worst, worst_lse, n_units, n_skip, n_replay = -1.0, 0.0, 0, 0, 0
    bad = []
    kk, vv = (x["k"], x["v"]) if kv_np is None else kv_np
    groups = B // op.vote_rows if 0 < op.vote_rows < B else 1
    rows = B // groups
    for b in range(cfg["batch"]):
        for h in (range(cfg["q_heads"]) if heads is None else heads):
            pt = None if page_table is None else page_table[b]
            for i in (range(nb) if blocks is None else blocks):
                kl = int(cnt[b, h, i])
                st = res["st"][b, h, i].astype(np.int64)
                n_comp, visited = 0, 0
                for g in range(groups):
                    gst = (st >> (2 * g)) & 3 if groups > 1 else st
                    fn = lambda forced, g=g: O.osk_unit(x["q"][b, h], kk[b, h // G], vv[b, h // G], i,
                                                        idx[b, h, i], kl, sh, op, pt, forced,
                                                        g if groups > 1 else None)
                    ok, w, msg, forced = replay_walk(fn, gst)
                    n_units += 1
                    n_replay += len(forced)
                    if not ok:
                        bad.append(f"(b={b}, h={h}, i={i}, group={g}): {msg}")
                        continue
                    n_skip += int((w["status"] == 2).sum())
                    n_comp += w["n_comp"]
                    visited = max(visited, w["visited"])
                    if w["out"].shape[0] == 0:
                        continue                 # a row group past the end of a ragged sequence
                    r0 = i * B + g * rows
                    err = out_excess(res["out"][b, h, r0:r0 + rows], w["out"], cfg["dtype"])
                    lerr = np.abs(res["lse"][b, h, r0:r0 + rows] - w["lse"]).max()
                    worst, worst_lse = max(worst, float(err)), max(worst_lse, float(lerr))
                tc = res["tc"][b, h, i]
                if tc[0] != visited or tc[1] != n_comp:
                    bad.append(f"(b={b}, h={h}, i={i}): counts {tc} vs {visited}, {n_comp}")
    assert not bad, f"{len(bad)}/{n_units} walks rejected; first: {bad[:3]}"
    dt = cfg["dtype"]
    assert worst <= 0.0, f"output error exceeds the tolerance by {worst}"
    assert worst_lse <= TOL_LSE[dt], f"max abs lse error {worst_lse} > {TOL_LSE[dt]}"
    return dict(units=n_units, skipped=n_skip, replays=n_replay, err=worst, lse_err=worst_lse)
