"""Benchmark of CoSA block-sparse prefill attention (KAP + OSK) on one MI355X.

One step = one layer's prefill attention over all heads: the proxy (pool, score,
select/order) followed by the ordered-skipping kernel on its lists.  Default
workload: the 128K Llama-3-8B GQA shape (32 query / 8 KV heads, head_dim 128,
block 128, bf16, budget 10 %, tightened budget 5 %), synthetic inputs with planted
salient blocks and a local-window bias.  The dense causal kernel is timed on the
same inputs for the speedup.

Prints one JSON line.  value = dense-equivalent TFLOP/s of the step
(4*D*Hq*B*N(N+1)/2 FLOP over the KAP+OSK time); ms_per_step is ms per layer prefill.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload index (synth.CONFIGS)")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-mode", type=int, default=2)
    ap.add_argument("--share-kv", action="store_true",
                    help="one visit list per KV head, walked by its query heads (GQA-shared mode)")
    ap.add_argument("--vote-rows", type=int, default=0, help="0: block skip vote; 32: per 32-row group")
    ap.add_argument("--cap-mode", type=int, default=1,
                    help="the tightened budget caps 1: visited blocks (default), 0: computed blocks")
    ap.add_argument("--no-concentrated", action="store_true",
                    help="skip the extra run on the concentrated 128K variant (where skipping fires)")
    ap.add_argument("--head-chunks", type=int, default=1,
                    help="1: the timed step is the two calls back to back on one stream; above 1 it "
                         "pipelines the proxy and the walk over this many groups of KV heads on two "
                         "streams (cosa_prefill)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the rates this GPU reaches: an HBM copy and a library bf16 GEMM")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def spread(ms):
    """median, min and max of per-step event times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "max": round(float(a.max()), 4)}


def log(msg, quiet=False):
    if not quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("attn.hip", "attn_tiles.hpp", "cosa_common.hpp"):
        with open(os.path.join(ROOT, "block_sparse_attention_kap_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_OPTIONS = {"skip": "mass", "lists": "per_q_head", "vote_rows": 0}


def load_traffic(kernel_hash: str, workload: str, options: dict):
    """HBM traffic of the OSK kernel from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel source, this workload and these walk options; else None."""
    p = os.path.join(ROOT, "profiles", f"osk_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_hash") != kernel_hash or d.get("workload") != workload \
            or d.get("options", TRAFFIC_OPTIONS) != options:
        return None
    return d.get("bytes_per_launch")


_CPU_CTX = {}   # set before the worker processes fork (read-only there)


def _cpu_worker(h: int):
    """One job of the CPU baseline: the oracle on every query block of query head h (pooling,
    proxy scores, order and select, the walk with skip test and cap, the closed-form output),
    with one BLAS thread.  Returns (h, seconds)."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    c = _CPU_CTX
    x, sh, kp, op = c["x"], c["sh"], c["kp"], c["op"]
    G = sh.q_heads // sh.kv_heads
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for b in range(sh.batch):
            O.run_head(x["q"][b, h], x["k"][b, h // G], x["v"][b, h // G], sh, kp, op)
    return h, time.perf_counter() - t0


def cpu_baseline(cfg, x, quiet: bool):
    """Time the oracle (as it stands) on the whole layer: every (query head, query block) unit,
    one job per query head on a pool of worker processes (one per host core, at most 16; one
    BLAS thread each), wall clock from the first job to the last.  The workers are forked
    before the GPU is touched; they share the inputs and never use the GPU."""
    import multiprocessing as mp

    import numpy as np

    import oracle as O
    sh = O.Shape(cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["seq_len"], cfg["head_dim"],
                 cfg["block"], True, float(np.float32(1.0 / np.sqrt(cfg["head_dim"]))), cfg["dtype"])
    kp = O.KapParams(budget=cfg["budget"])
    op = O.OskParams(tight_budget=cfg["tight_budget"])
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    _CPU_CTX.update(x=x, sh=sh, kp=kp, op=op)
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        parts = []
        for h, sec in pool.imap_unordered(_cpu_worker, range(cfg["q_heads"])):
            parts.append(sec)
            if len(parts) % 8 == 0:
                log(f"oracle: {len(parts)} of {cfg['q_heads']} query heads done", quiet)
        total = time.perf_counter() - t0
    _CPU_CTX.clear()
    log(f"oracle: whole layer ({cfg['batch'] * cfg['q_heads']} query heads x {sh.nb} query blocks) "
        f"in {total:.1f}s on {workers} processes ({sum(parts):.1f} core-seconds)", quiet)
    return total, workers, float(sum(parts))


def concentrated_run(args, cfg, q, k, v, idx, cnt, hrm, out, ws, kmax, scale, peak):
    """The same 128K shape with attention concentrated on the planted blocks (planted keys 12x
    stronger, query noise 0.2), where the in-kernel skip test fires: the proxy, then the walk on
    its lists with the skip test (the benchmark's cap mode), with it off, and with the cap
    counted the other way; times, realized fractions and the MFMA fraction on visited tiles.
    The inputs are written into the benchmark's own buffers (no new device allocation)."""
    import numpy as np
    import torch

    import block_sparse_attention_kap_amd as cosa
    from synth import make
    c = dict(cfg, salient_gain=12.0, q_noise=0.2)
    x = make(c)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        t.copy_(torch.from_numpy(x[n]).to(t.dtype))
    del x
    B, D = cfg["block"], cfg["head_dim"]
    nb = cfg["seq_len"] // B
    n_cand = cfg["batch"] * cfg["q_heads"] * nb * (nb + 1) // 2
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    kap = lambda: cosa.kap(q, k, block=B, budget=cfg["budget"], scale=scale, kmax=kmax, workspace=ws,
                           outs=(idx, cnt, hrm))
    kap_ms = timed(kap, args.steps)
    res = {"workload": f"{cfg['name']} with planted keys 12x stronger and query noise 0.2",
           "kap_ms": spread(kap_ms)}
    for name, skip, cap in (("skip", 2, args.cap_mode), ("skip_off", 0, args.cap_mode),
                            ("skip_other_cap", 2, 1 - args.cap_mode)):
        osk = lambda: cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=cfg["tight_budget"],
                               skip_mode=skip, scale=scale, out=out, cap_mode=cap)
        ms = timed(osk, args.steps)
        _, tc = cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=cfg["tight_budget"], skip_mode=skip,
                         scale=scale, return_counts=True, cap_mode=cap)
        t = tc.to(torch.int64).sum(dim=(0, 1, 2)).cpu().numpy()
        vis, comp = int(t[0]), int(t[1])
        flop = 2.0 * B * B * D * (vis + comp)
        res[name] = {"cap": ["computed", "visited"][cap], "osk_ms": spread(ms),
                     "visited_frac": round(vis / n_cand, 4), "computed_frac": round(comp / n_cand, 4),
                     "skipped_of_visited": round((vis - comp) / max(1, vis), 4),
                     "osk_mfma_frac_visited": round(flop / (float(np.mean(ms)) * 1e-3) / 1e12 / peak, 4)}
        log(f"concentrated, {name} ({res[name]['cap']} cap): osk {np.median(ms):.3f} ms, "
            f"computed {res[name]['computed_frac']}, skipped {res[name]['skipped_of_visited']}",
            args.quiet)
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the hot path needs no collective, and the kernels "
              "are measured on a single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.peaks:
        # what the chip delivers outside this library: a 2 GiB device copy (HBM read + write) and a
        # dense bf16 GEMM through torch.matmul (the vendor GEMM library), each timed with events
        res = {}
        n = (2 << 30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        ts = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(src)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        res["hbm_copy_GBps"] = round(2 * n * 4 / (float(np.median(ts)) * 1e-3) / 1e9, 1)
        del src, dst
        for m in (4096, 8192, 16384):
            x = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
            y = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
            for _ in range(3):
                z = x @ y
            ts = []
            for _ in range(10):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                z = x @ y
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            res[f"bf16_gemm_{m}_TFLOPs"] = round(2.0 * m ** 3 / (float(np.median(ts)) * 1e-3) / 1e12, 1)
            del x, y, z
        res["datasheet"] = {"hbm_GBps": 8000, "bf16_dense_TFLOPs": 2500}
        print(json.dumps(res))
        return

    if args.copy_probe_mib:
        # a plain copy of known size: calibrates the HBM byte counters of the profiler
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n * 4}))
        return

    import block_sparse_attention_kap_amd as cosa
    from synth import config, make

    if not os.path.exists(cosa.lib_path()):
        from block_sparse_attention_kap_amd.build import build
        build()
    cfg = config(args.config)
    B, D, N = cfg["block"], cfg["head_dim"], cfg["seq_len"]
    Bt, Hq, Hkv = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    nb = -(-N // B)
    log(f"workload {cfg['name']}: generating inputs", args.quiet)
    t0 = time.perf_counter()
    x = make(cfg)
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s", args.quiet)
    cpu = None
    if not args.no_cpu_baseline and args.config in (1, 2, 3, 4):
        # before anything touches the GPU: the oracle's worker processes fork from here
        cpu = cpu_baseline(cfg, x, args.quiet)
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(tdt).to(dev) for n in ("q", "k", "v"))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    shape = cosa.make_shape(q, k, B, True, scale)
    kparams = cosa.KapParams(cfg["budget"], 0, 0, 0, 0, 0.0, 0, 0, 0, int(args.share_kv))
    ws = torch.empty(cosa.kap_workspace_bytes(shape, kparams), dtype=torch.uint8, device=dev)
    kmax = cosa.list_capacity(shape, cfg["budget"])
    Hl = Hkv if args.share_kv else Hq          # heads the lists are indexed by
    idx = torch.empty((Bt, Hl, nb, kmax), dtype=torch.int32, device=dev)
    cnt = torch.empty((Bt, Hl, nb), dtype=torch.int32, device=dev)
    hrm = torch.empty((Bt, Hl, nb), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        cosa.kap(q, k, block=B, budget=cfg["budget"], scale=scale, kmax=kmax, workspace=ws,
                 outs=(idx, cnt, hrm), share_kv=args.share_kv)
        if ev is not None:
            ev[1].record(stream)
        cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=cfg["tight_budget"],
                 skip_mode=args.skip_mode, scale=scale, out=out, vote_rows=args.vote_rows,
                 cap_mode=args.cap_mode,
                 shared_lists=args.share_kv)
        if ev is not None:
            ev[2].record(stream)

    # groups of KV heads for the pipelined step: the largest divisor of Hkv not above the request
    chunks = max(c for c in range(1, max(1, args.head_chunks) + 1) if Hkv % c == 0)

    def piped_step():
        cosa.prefill(q, k, v, block=B, budget=cfg["budget"], tight_budget=cfg["tight_budget"],
                     head_chunks=chunks, share_kv=args.share_kv, skip_mode=args.skip_mode,
                     cap_mode=args.cap_mode,
                     vote_rows=args.vote_rows, scale=scale, workspace=ws, lists=(idx, cnt, hrm),
                     out=out)

    timed = piped_step if chunks > 1 else step
    for _ in range(args.warmup):
        timed()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        timed()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = wall * 1e3 / args.steps
    # the two stages timed apart (back to back on one stream, events around each)
    for _ in range(args.warmup if chunks > 1 else 0):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    kap_ms = [e[0].elapsed_time(e[1]) for e in evs]
    osk_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    log(f"step {ms_per_step:.3f} ms wall ({chunks} head group(s)), back to back: kap "
        f"{np.median(kap_ms):.3f} ms, osk {np.median(osk_ms):.3f} ms, both {np.median(step_ms):.3f} ms",
        args.quiet)

    # realized work of the OSK (deterministic: same lists every step)
    _, st_counts = cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=cfg["tight_budget"],
                            skip_mode=args.skip_mode, scale=scale, return_counts=True,
                            cap_mode=args.cap_mode,
                            vote_rows=args.vote_rows, shared_lists=args.share_kv)
    torch.cuda.synchronize()
    tcs = st_counts.to(torch.int64).sum(dim=(0, 1, 2)).cpu().numpy()
    visited, computed = int(tcs[0]), int(tcs[1])
    if args.vote_rows:
        computed = computed * args.vote_rows // B   # row-group tiles -> whole-block equivalents
    n_cand = Bt * Hq * nb * (nb + 1) // 2
    osk_flop = 2.0 * B * B * D * (visited + computed)
    osk_avg = float(np.mean(osk_ms))
    kap_avg = float(np.mean(kap_ms))
    osk_tflops = osk_flop / (osk_avg * 1e-3) / 1e12
    f_dense = 4.0 * D * Hq * Bt * N * (N + 1) / 2
    value = f_dense / (ms_per_step * 1e-3) / 1e12
    eb = 2 if cfg["dtype"] == "bf16" else 4
    g = B // 4
    kap_bytes = (Hq + Hkv) * Bt * N * D * eb * (1 + 1 / g)
    khash = source_hash()
    traffic = load_traffic(khash, cfg["name"],
                           {"skip": ["off", "maxdiff", "mass"][args.skip_mode],
                            "lists": "per_kv_head" if args.share_kv else "per_q_head",
                            "vote_rows": args.vote_rows})

    dense_ms = None
    # the dense baseline's tile: its result does not depend on it, and 128-key tiles run it
    # faster than 64-key ones (the baseline is the faster of the two)
    dense_block = 128
    if not args.no_dense:
        dout = torch.empty_like(q)
        cosa.dense(q, k, v, block=dense_block, scale=scale, out=dout)
        torch.cuda.synchronize()
        de = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.dense_reps)]
        for a, b in de:
            a.record(stream)
            cosa.dense(q, k, v, block=dense_block, scale=scale, out=dout)
            b.record(stream)
        torch.cuda.synchronize()
        dense_ms = float(np.mean([a.elapsed_time(b) for a, b in de]))
        log(f"dense {dense_ms:.3f} ms", args.quiet)
        del dout
    # the same lists walked with the skip test off (ordered truncation at the cap only)
    skip_off = None
    if args.skip_mode != 0:
        so_ms = []
        for r in range(args.warmup + args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=cfg["tight_budget"], skip_mode=0,
                     cap_mode=args.cap_mode,
                     scale=scale, out=out, vote_rows=args.vote_rows, shared_lists=args.share_kv)
            b.record(stream)
            if r >= args.warmup:
                so_ms.append((a, b))
        torch.cuda.synchronize()
        so = [a.elapsed_time(b) for a, b in so_ms]
        _, so_counts = cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=cfg["tight_budget"],
                                skip_mode=0, scale=scale, return_counts=True,
                                cap_mode=args.cap_mode,
                                vote_rows=args.vote_rows, shared_lists=args.share_kv)
        torch.cuda.synchronize()
        sc = so_counts.to(torch.int64).sum(dim=(0, 1, 2)).cpu().numpy()
        so_comp = int(sc[1]) * args.vote_rows // B if args.vote_rows else int(sc[1])
        skip_off = {"osk_ms": spread(so), "visited_tiles": int(sc[0]), "computed_tiles": so_comp,
                    "osk_mfma_frac_visited": round(2.0 * B * B * D * (int(sc[0]) + so_comp)
                                                   / (float(np.mean(so)) * 1e-3) / 1e12
                                                   / (PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16"
                                                      else PEAK_F32_TFLOPS), 4)}
        log(f"skip off: osk {np.median(so):.3f} ms", args.quiet)
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_F32_TFLOPS
    conc = None
    if args.config == 3 and not args.no_concentrated and not args.share_kv and not args.vote_rows:
        conc = concentrated_run(args, cfg, q, k, v, idx, cnt, hrm, out, ws, kmax, scale, peak)
    res = {
        "metric": "dense-equivalent TFLOP/s of one 128K layer prefill (KAP+OSK); "
                  "also ms/layer, speedup vs dense, MFMA % on visited blocks",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded planted-structure Q/K/V; no dataset, no weights)",
        "inputs": {"generator": "synth.make", "seed": cfg["seed"], "numpy": np.__version__,
                   "structure": cfg["structure"]},
        "config": {"workload": cfg["name"], "batch": Bt, "q_heads": Hq, "kv_heads": Hkv,
                   "seq_len": N, "head_dim": D, "block": B, "budget": cfg["budget"],
                   "tight_budget": cfg["tight_budget"], "skip": ["off", "maxdiff", "mass"][args.skip_mode],
                   "cap": ["computed", "visited"][args.cap_mode],
                   "skip_eps": 1e-3, "lists": "per_kv_head" if args.share_kv else "per_q_head",
                   "vote_rows": args.vote_rows,
                   "schedule": (f"proxy and walk pipelined over {chunks} groups of KV heads on two streams"
                                if chunks > 1 else "proxy then walk on one stream")},
        "ms_per_layer": round(ms_per_step, 4),
        "kap_ms": round(kap_avg, 4),
        "osk_ms": round(osk_avg, 4),
        "events_ms": {"kap": spread(kap_ms), "osk": spread(osk_ms), "layer_back_to_back": spread(step_ms)},
        "skip_off": skip_off,
        "dense_ms": None if dense_ms is None else round(dense_ms, 3),
        "dense_block": dense_block,
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms_per_step, 3),
        "dense_mfma_frac": None if dense_ms is None else round(f_dense / (dense_ms * 1e-3) / 1e12 / peak, 4),
        "osk_mfma_frac_visited": round(osk_tflops / peak, 4),
        "kap_hbm_frac": round(kap_bytes / (kap_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "realized": {"visited_frac": round(visited / n_cand, 4), "computed_frac": round(computed / n_cand, 4),
                     "visited_tiles": visited, "computed_tiles": computed,
                     "skipped_tiles": visited - computed},
        "roofline": {"bound": "mfma",
                     "kernel": (f"attn2_kernel<{B},{D},{2 if args.vote_rows else 1}> (OSK)"
                                if cfg["dtype"] == "bf16" else f"attn_kernel<f32,{B},{D},sparse> (OSK)"),
                     "achieved": round(osk_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(osk_tflops / peak, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": osk_flop, "kernel_ms": round(osk_avg, 4),
                     "source_hash": khash},
        "concentrated": conc,
        "cpu_baseline": None,
    }
    if cpu is not None:
        total_s, cores, spent = cpu
        res["cpu_baseline"] = {"value": round(f_dense / total_s / 1e12, 6), "unit": "TFLOP/s",
                               "ms_per_layer": round(total_s * 1e3, 1), "cores": cores, "kind": "oracle",
                               "sample": f"whole layer: all {Bt * Hq * nb} (query head, query block) units "
                                         f"(pooling, proxy, order and select, walk with skip test and cap, "
                                         f"closed-form output), one job per query head on {cores} worker "
                                         f"processes with one BLAS thread each ({spent:.1f} core-seconds); "
                                         f"wall clock, no extrapolation"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
