"""Seeded synthetic Q, K, V for the five workloads of the benchmark.

The pages evaluate on RULER and LongBench-v2 with Llama-3.1-8B and Qwen3-8B
backbones.  Neither the datasets nor the weights are used here: these
generators stand in for them with Llama-3-8B attention shapes (32 query heads,
8 KV heads, head_dim 128) and planted structure that gives the proxy something
to find (salient key blocks, a sink block, a local-window bias, a Gaussian
mixture with heavy-tailed outlier rows).

Everything is drawn on the host with ``numpy.random.default_rng(seed)`` in
float32, in the order Q, K, V, then structure, and finally rounded
round-to-nearest-even to the storage dtype.  Arrays are returned as float32
holding dtype-exact values, layout [batch, heads, seq, dim].
"""
from __future__ import annotations

import copy

import numpy as np

# Workload table.  Seeds are 1000 + index.
CONFIGS = [
    dict(name="tiny_fp32_1k", batch=1, q_heads=1, kv_heads=1, seq_len=1024,
         head_dim=64, block=64, dtype="f32", budget=0.5, tight_budget=0.25,
         structure="iid", seed=1000),
    dict(name="llama_gqa_8k", batch=1, q_heads=32, kv_heads=8, seq_len=8192,
         head_dim=128, block=128, dtype="bf16", budget=0.3, tight_budget=0.15,
         structure="salient", n_salient=4, sink=True, window=0, seed=1001),
    dict(name="llama_gqa_32k", batch=1, q_heads=32, kv_heads=8, seq_len=32768,
         head_dim=128, block=128, dtype="bf16", budget=0.2, tight_budget=0.1,
         structure="salient", n_salient=16, sink=False, window=4, seed=1002),
    dict(name="llama_gqa_128k", batch=1, q_heads=32, kv_heads=8,
         seq_len=131072, head_dim=128, block=128, dtype="bf16", budget=0.1,
         tight_budget=0.05, structure="salient", n_salient=64, sink=False,
         window=4, seed=1003),
    dict(name="stress_gqa7_128k_b64", batch=1, q_heads=28, kv_heads=4,
         seq_len=131072, head_dim=128, block=64, dtype="bf16", budget=0.08,
         tight_budget=0.04, structure="mixture", n_components=16,
         outlier_frac=0.005, seed=1004),
]


def config(index: int) -> dict:
    return copy.deepcopy(CONFIGS[index])


def shrink(cfg: dict, seq_len: int, q_heads: int | None = None,
           kv_heads: int | None = None, n_salient: int | None = None) -> dict:
    """Same structure at a smaller size (for parity tests the oracle can finish)."""
    c = copy.deepcopy(cfg)
    c["seq_len"] = seq_len
    if q_heads is not None:
        c["q_heads"] = q_heads
    if kv_heads is not None:
        c["kv_heads"] = kv_heads
    if c.get("structure") == "salient":
        nb = seq_len // c["block"]
        ns = n_salient if n_salient is not None else max(1, c["n_salient"] * seq_len // cfg["seq_len"])
        c["n_salient"] = min(ns, nb - 1)
    c["name"] = f'{cfg["name"]}@{seq_len}'
    return c


def ragged(cfg: dict, seq_len: int) -> dict:
    """The same workload cut to seq_len tokens, which the block need not divide.

    Inputs are drawn at the next multiple of the block and their first seq_len
    rows kept, so the structure of every whole block is unchanged.
    """
    c = copy.deepcopy(cfg)
    blk = c["block"]
    full = -(-seq_len // blk) * blk
    if full != c["seq_len"]:
        c = shrink(c, full)
    c["take"] = seq_len
    c["name"] = f'{cfg["name"]}@{seq_len}'
    return c


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 value (ties to even), in place.

    Inputs are finite.  The result is float32 holding bf16-exact values.
    """
    assert x.dtype == np.float32
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return x


def _unit(rng, *shape_and_dim):
    v = rng.standard_normal(shape_and_dim, dtype=np.float32)
    v /= np.linalg.norm(v, axis=-1, keepdims=True)
    return v


def make(cfg: dict, seed: int | None = None) -> dict:
    """Draw Q, K, V for one workload.  Returns dict(q=, k=, v=) float32 arrays.

    Optional knobs of the "salient" structure (defaults reproduce the workload
    table): ``salient_gain`` (3.0) scales the planted keys, ``q_noise`` (1.0)
    scales the i.i.d. part of Q.  A large gain with a small noise concentrates
    attention so that in-kernel skipping fires.
    """
    rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
    bt, hq, hk = cfg["batch"], cfg["q_heads"], cfg["kv_heads"]
    n, d, blk = cfg["seq_len"], cfg["head_dim"], cfg["block"]
    assert n % blk == 0 and hq % hk == 0
    nb = n // blk
    grp = hq // hk
    q = rng.standard_normal((bt, hq, n, d), dtype=np.float32)
    k = rng.standard_normal((bt, hk, n, d), dtype=np.float32)
    v = rng.standard_normal((bt, hk, n, d), dtype=np.float32)
    st = cfg.get("structure", "iid")
    if st == "salient":
        for b in range(bt):
            u = _unit(rng, hk, d)                       # one query direction per KV head
            gain = cfg.get("salient_gain", 3.0)
            qn = cfg.get("q_noise", 1.0)
            if qn != 1.0:
                q[b] *= qn
            for g in range(hk):
                q[b, g * grp:(g + 1) * grp] += u[g]
                sal = rng.choice(np.arange(1, nb), size=cfg["n_salient"], replace=False)
                blocks = list(sal) + ([0] if cfg.get("sink") else [])
                for j in blocks:
                    jit = 0.1 * rng.standard_normal((blk, d), dtype=np.float32)
                    k[b, g, j * blk:(j + 1) * blk] = gain * np.sqrt(d) * u[g] + jit
            w_len = cfg.get("window", 0)
            if w_len:
                w = _unit(rng, hk, nb, d)                  # one direction per (KV head, q-block)
                # query block i of every Q head in group g moves along 3 w[g, i]
                qv = q[b].reshape(hk, grp, nb, blk, d)
                qv += 3.0 * w[:, None, :, None, :]
                # key block j moves toward the query directions of blocks i in [j, j + w_len]
                cs = np.concatenate([np.zeros((hk, 1, d), np.float32), np.cumsum(3.0 * w, axis=1, dtype=np.float32)], axis=1)
                hi = np.minimum(np.arange(nb) + w_len, nb - 1) + 1
                kbias = cs[:, hi] - cs[:, np.arange(nb)]  # sum over i = j .. min(j+w, nb-1)
                kv = k[b].reshape(hk, nb, blk, d)
                kv += kbias[:, :, None, :]
    elif st == "mixture":
        ncomp = cfg["n_components"]
        for b in range(bt):
            for g in range(hk):
                mu = rng.standard_normal((ncomp, d), dtype=np.float32)
                comp = rng.integers(0, ncomp, size=n)
                n_out = int(round(cfg["outlier_frac"] * n))
                rows = rng.choice(n, size=n_out, replace=False)
                tnoise = (3.0 * rng.standard_t(3, size=(n_out, d))).astype(np.float32)
                k[b, g, rows] = tnoise                  # outlier rows: noise replaced
                k[b, g] += mu[comp]
    elif st != "iid":
        raise ValueError(st)
    if cfg["dtype"] == "bf16":
        for x in (q, k, v):
            round_bf16(x)
    elif cfg["dtype"] != "f32":
        raise ValueError(cfg["dtype"])
    t = cfg.get("take", n)
    if t != n:                                          # ragged length: keep the first t rows
        q, k, v = (np.ascontiguousarray(x[:, :, :t]) for x in (q, k, v))
    return dict(q=q, k=k, v=v)
