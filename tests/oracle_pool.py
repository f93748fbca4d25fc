"""A pool of worker processes that compares GPU results with the oracle, one (batch, head) at a
time, for the parity tests at the benchmark's full sizes (test infrastructure only).

The workers are forked while the test session is being collected, before anything touches the
GPU, and never use it: each one regenerates a workload's inputs from its seed (cached per
workload) and receives, per job, the GPU's lists, status traces, counts and output rows of one
head.  It checks every query block of that head: the list through the tie-band comparator, the
walk by status-trace replay, and the output and LSE against the oracle's closed form.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

TOL_OUT = {"bf16": 1e-2, "f32": 1e-4}
TOL_LSE = {"bf16": 1e-3, "f32": 1e-5}

_INPUTS: dict = {}
SUMMARIES: list = []   # one line per exhaustive comparison (parent process), printed at the end


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def start():
    """Fork the pool (call before the GPU is initialised in this process)."""
    return mp.get_context("fork").Pool(workers())


def _bf16_neighbours(x32: np.ndarray):
    """The bf16 values just below and above each bf16 value x (as float64)."""
    u = x32.astype(np.float32).view(np.uint32) >> 16
    sign = (u >> 15) & 1
    mag = u & 0x7FFF
    # moving the magnitude away from / toward zero; zero's neighbours are the smallest
    # subnormals of either sign
    away = ((mag + 1) | (sign << 15)).astype(np.uint32) << 16
    toward = np.where(mag == 0, (1 | ((1 - sign) << 15)) << 16,
                      (((mag - 1) | (sign << 15)).astype(np.uint32) << 16)).astype(np.uint32)
    a = away.view(np.float32).astype(np.float64)
    t = toward.view(np.float32).astype(np.float64)
    up = np.where(sign == 0, a, t)
    down = np.where(sign == 0, t, a)
    return down, up


def output_check(got, ref, dtype):
    """Compare GPU outputs with the oracle's (fp64) closed form.

    The tolerance (1e-2 for bf16 inputs with fp32 accumulation, 1e-4 for fp32) bounds the
    error of the value the kernel forms before it stores it; the stored value is that value
    rounded to the output dtype (round to nearest even).  So an output passes iff its rounding
    interval, the reals that round to it, meets [ref - tol, ref + tol]: that is, iff it is the
    storage rounding of some value within the tolerance of the oracle.
    Returns (excess, flat, flat_rounded, n_flat, n_flat_rounded): excess <= 0 iff every
    element passes (the distance by which the worst rounding interval misses the tolerance
    band); flat = max |got - ref|; flat_rounded = max |got - round(ref)| (the oracle rounded to
    the output dtype); n_flat, n_flat_rounded: how many elements exceed the tolerance by those
    two flat measures.
    """
    got = np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    tol = TOL_OUT[dtype]
    g64 = got.astype(np.float64)
    if dtype == "bf16":
        down, up = _bf16_neighbours(got.astype(np.float32))
        r32 = ref.astype(np.float32).view(np.uint32).astype(np.uint64)
        rr = (((r32 + 0x7FFF + ((r32 >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    else:
        g32 = got.astype(np.float32)
        down = np.nextafter(g32, np.float32(-np.inf)).astype(np.float64)
        up = np.nextafter(g32, np.float32(np.inf)).astype(np.float64)
        rr = ref.astype(np.float32)
    lo_edge = (g64 + down) / 2          # the rounding interval of got
    hi_edge = (g64 + up) / 2
    miss = np.maximum(lo_edge - (ref + tol), (ref - tol) - hi_edge)
    excess = float(miss.max()) if miss.size else -1.0
    d = np.abs(g64 - ref)
    dr = np.abs(g64 - rr.astype(np.float64))
    flat = float(d.max()) if ref.size else 0.0
    flat_r = float(dr.max()) if ref.size else 0.0
    return excess, flat, flat_r, int((d > tol).sum()), int((dr > tol).sum())


def _inputs(cfg):
    from synth import make
    key = (cfg["name"], cfg["seed"], cfg["seq_len"], cfg["q_heads"], cfg["kv_heads"])
    if key not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[key] = make(cfg)
    return _INPUTS[key]


def _as_float(a, dtype):
    if dtype == "bf16" and a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def check_head(job: dict) -> dict:
    """Every query block of one (batch b, query head h): list, walk trace, counts, output, LSE.

    job: cfg, kap (KapParams fields), osk (OskParams fields), b, h, share (lists per KV head),
    idx [nb, kmax], cnt [nb], hrm [nb], sc [nb, kmax], st [nb, kmax], tc [nb, 2],
    out [N, D] (uint16 bf16 bits or float32), lse [N].
    """
    from threadpoolctl import threadpool_limits

    import oracle as O
    from oracle.compare import check_list, replay_walk

    t0 = time.perf_counter()
    cfg = job["cfg"]
    x = _inputs(cfg)
    b, h = job["b"], job["h"]
    dt = cfg["dtype"]
    G = cfg["q_heads"] // cfg["kv_heads"]
    kvh = h // G
    B = cfg["block"]
    N = cfg["seq_len"]
    sh = O.Shape(cfg["batch"], cfg["q_heads"], cfg["kv_heads"], N, cfg["head_dim"], B, True,
                 float(np.float32(1.0 / np.sqrt(cfg["head_dim"]))), dt)
    kp = O.KapParams(**job["kap"])
    op = O.OskParams(**job["osk"])
    out = _as_float(job["out"], dt)
    lse = job["lse"]
    # an optional range of query blocks [lo, hi); out and lse then hold rows lo*B .. hi*B - 1
    lo, hi = job.get("blocks", (0, sh.nb))
    row0 = lo * B if "blocks" in job else 0
    bad = []
    res = dict(b=b, h=h, units=0, skipped=0, replays=0, excess=-1.0, flat=0.0, flat_r=0.0,
               n_flat=0, n_flat_r=0, elements=0, lse=0.0, max_abs_out=0.0)
    with threadpool_limits(limits=1):
        blocks = range(lo, hi)
        if job["share"]:
            units = O.kap_kv_group(x["q"][b, kvh * G:(kvh + 1) * G], x["k"][b, kvh], sh, kp, blocks)
        else:
            units = O.kap_head(x["q"][b, h], x["k"][b, kvh], sh, kp, blocks)
        for i, u in zip(blocks, units):
            res["units"] += 1
            ok, msg = check_list(u, job["idx"][i], int(job["cnt"][i]), int(job["hrm"][i]),
                                 job["sc"][i])
            if not ok:
                bad.append(f"list (b={b}, h={h}, i={i}): {msg}")
                continue
            lst, kl = job["idx"][i], int(job["cnt"][i])
            # with 32-row votes every group of rows walks on its own: 2 status bits per group
            groups = B // op.vote_rows if 0 < op.vote_rows < B else 1
            rows_g = B // groups
            n_comp, visited = 0, 0
            for g in range(groups):
                st = job["st"][i].astype(np.int64)
                gst = (st >> (2 * g)) & 3 if groups > 1 else st
                fn = lambda forced, i=i, lst=lst, kl=kl, g=g: O.osk_unit(
                    x["q"][b, h], x["k"][b, kvh], x["v"][b, kvh], i, lst, kl, sh, op,
                    forced=forced, group=g if groups > 1 else None)
                ok, w, msg, forced = replay_walk(fn, gst)
                if not ok:
                    bad.append(f"walk (b={b}, h={h}, i={i}, group={g}): {msg}")
                    continue
                res["replays"] += len(forced)
                res["skipped"] += int((w["status"] == 2).sum())
                n_comp += w["n_comp"]
                visited = max(visited, w["visited"])
                r0 = i * B + g * rows_g
                rows = slice(r0 - row0, min(r0 + rows_g, N) - row0)
                if w["out"].shape[0] == 0:
                    continue
                e, f, fr, nf, nfr = output_check(out[rows], w["out"], dt)
                res["excess"] = max(res["excess"], e)
                res["flat"] = max(res["flat"], f)
                res["flat_r"] = max(res["flat_r"], fr)
                res["n_flat"] += nf
                res["n_flat_r"] += nfr
                res["elements"] += w["out"].size
                res["max_abs_out"] = max(res["max_abs_out"], float(np.abs(w["out"]).max()))
                res["lse"] = max(res["lse"], float(np.abs(lse[rows] - w["lse"]).max()))
            tc = job["tc"][i]
            if tc[0] != visited or tc[1] != n_comp:
                bad.append(f"counts (b={b}, h={h}, i={i}): {tc.tolist()} vs {visited}, {n_comp}")
    res["bad"] = bad[:5]
    res["n_bad"] = len(bad)
    res["seconds"] = time.perf_counter() - t0
    return res
