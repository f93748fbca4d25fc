"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small workloads (same structure as the benchmark configs, sizes the oracle
finishes in seconds, several tiles, query-block counts that leave a ragged tail
in the XCD-grouped launch) are compared unit by unit:
  - pooled Q and K: bitwise;
  - block-level proxy scores: within fp32 accumulation error;
  - visit lists: the tie-band comparator (exact outside a 1e-5 relative band);
  - OSK status traces: exact, with replay of decisions whose statistic sits within
    the band of the threshold; outputs within 1e-2 (bf16) / 1e-4 (fp32) max abs.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_kap_amd as cosa
import oracle as O
from synth import config, make, ragged, shrink
from gpu_helpers import (TOL_OUT, check_lists, out_excess, check_osk_units, gpu_kap, gpu_osk, num_blocks,
                         oracle_lists, oshape, pack_lists, scale_of, seq_len, to_dev, upload)

pytestmark = pytest.mark.gpu


def _cfgs():
    c0 = config(0)
    c1 = shrink(config(1), 2304, q_heads=8, kv_heads=2, n_salient=3)     # nb = 18
    c2 = shrink(config(2), 4096, q_heads=4, kv_heads=1, n_salient=6)     # window bias
    c4 = shrink(config(4), 4096, q_heads=7, kv_heads=1)                  # B = 64, G = 7
    cc = shrink(config(1), 3072, q_heads=4, kv_heads=1, n_salient=5)     # concentrated: skips fire
    cc.update(salient_gain=12.0, q_noise=0.2)
    c64 = dict(shrink(config(1), 2048, q_heads=2, kv_heads=1, n_salient=2), head_dim=64)
    c32f = dict(shrink(config(2), 2048, q_heads=2, kv_heads=1, n_salient=3), dtype="f32",
                block=128)
    # ragged lengths: a partial last block, and a partial last pooled group (N % g != 0)
    r1 = ragged(c1, 2304 - 88)                                           # 40-row tail, N % 32 = 8
    r4 = ragged(c4, 4096 - 40)                                           # B = 64: 24-row tail
    rc = dict(ragged(cc, 3072 - 100), salient_gain=12.0, q_noise=0.2)    # 28-row tail
    r0 = ragged(c0, 1000)                                                # fp32, 40-row tail
    r64 = ragged(c64, 2048 - 9)                                          # D = 64, N % 16 = 7
    rs = ragged(shrink(config(1), 128, q_heads=2, kv_heads=1, n_salient=0), 100)   # N < B
    # concentrated at block 64 with G = 7 (shared lists: four heads per workgroup, the second
    # workgroup of the group one head short)
    cc64 = dict(shrink(config(1), 3072, q_heads=7, kv_heads=1, n_salient=5), block=64,
                salient_gain=12.0, q_noise=0.2)
    return {"tiny_fp32": c0, "gqa8k_small": c1, "gqa32k_small": c2, "stress_small": c4,
            "concentrated": cc, "d64_bf16": c64, "fp32_b128": c32f, "ragged_gqa": r1,
            "ragged_b64": r4, "ragged_conc": rc, "ragged_fp32": r0, "ragged_d64": r64,
            "ragged_short": rs, "concentrated_b64": cc64}


CFGS = _cfgs()
_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        cfg = CFGS[name]
        x = make(cfg)
        _CACHE[name] = (cfg, x, upload(x, cfg))
    return _CACHE[name]


def _kp(cfg, **kw):
    return O.KapParams(budget=kw.pop("budget", cfg["budget"]), **kw)


def _op(cfg, **kw):
    return O.OskParams(tight_budget=kw.pop("tight_budget", cfg["tight_budget"]), **kw)


# ------------------------------------------------------------------ KAP

def _workspace_views(cfg, kp, ws):
    g = kp.g(oshape(cfg))
    Np = -(-seq_len(cfg) // g)
    D = cfg["head_dim"]
    eb = 2 if cfg["dtype"] == "bf16" else 4
    a256 = lambda n: (n + 255) // 256 * 256
    qbytes = cfg["batch"] * cfg["q_heads"] * Np * D * eb
    kbytes = cfg["batch"] * cfg["kv_heads"] * Np * D * eb
    tdt = torch.bfloat16 if eb == 2 else torch.float32
    qp = ws[:qbytes].view(tdt).view(cfg["batch"], cfg["q_heads"], Np, D)
    kp_ = ws[a256(qbytes):a256(qbytes) + kbytes].view(tdt).view(cfg["batch"], cfg["kv_heads"], Np, D)
    nb = num_blocks(dict(cfg, seq_len=seq_len(cfg)))
    ldp = (nb + 3) // 4 * 4                      # row pitch of P: blocks rounded up to 4
    pbytes = cfg["batch"] * cfg["q_heads"] * Np * ldp * 4
    off = a256(qbytes) + a256(kbytes)
    P = ws[off:off + pbytes].view(torch.float32).view(cfg["batch"], cfg["q_heads"], Np, ldp)[..., :nb]
    return qp.float().cpu().numpy(), kp_.float().cpu().numpy(), P.cpu().numpy()


@pytest.mark.parametrize("name,pool,mode", [
    ("tiny_fp32", 0, 0), ("gqa8k_small", 0, 0), ("stress_small", 0, 0), ("gqa8k_small", 1, 0),
    ("gqa8k_small", 2, 0), ("gqa8k_small", 8, 1), ("fp32_b128", 4, 0), ("d64_bf16", 64, 0),
    ("ragged_gqa", 0, 0), ("ragged_gqa", 8, 1), ("ragged_b64", 0, 0), ("ragged_fp32", 0, 0),
    ("ragged_d64", 0, 0), ("ragged_short", 0, 0),
    # every pooled-keys-per-block branch of the bf16 score kernel (B / g = 8, 32, 16 at D = 64,
    # 32 on a ragged block-64 sequence)
    ("gqa8k_small", 16, 0), ("gqa8k_small", 4, 0), ("d64_bf16", 8, 0), ("ragged_b64", 2, 0),
])
def test_pool_bitwise_and_proxy_scores(name, pool, mode):
    cfg, x, xd = _inputs(name)
    kp = _kp(cfg, pool=pool, pool_mode=mode)
    sh = oshape(cfg)
    params = cosa.KapParams(kp.budget, pool, mode, 0, 0, 0.0, 0, 0, 0)
    shape = cosa.make_shape(xd["q"], xd["k"], cfg["block"], True, scale_of(cfg))
    ws = torch.zeros(cosa.kap_workspace_bytes(shape, params), dtype=torch.uint8, device="cuda")
    cosa.kap(xd["q"], xd["k"], block=cfg["block"], budget=kp.budget, pool=pool, pool_mode=mode,
             scale=scale_of(cfg), workspace=ws)
    torch.cuda.synchronize()
    qp, kpp, P = _workspace_views(cfg, kp, ws)
    g = kp.g(sh)
    G = cfg["q_heads"] // cfg["kv_heads"]
    for b in range(cfg["batch"]):
        for h in range(cfg["q_heads"]):
            want = O.pool_rows(x["q"][b, h], g, mode, cfg["dtype"])
            assert np.array_equal(qp[b, h], want), f"pooled Q head {h}"
        for hk in range(cfg["kv_heads"]):
            want = O.pool_rows(x["k"][b, hk], g, mode, cfg["dtype"])
            assert np.array_equal(kpp[b, hk], want), f"pooled K head {hk}"
    rb = cfg["block"] // g
    worst = 0.0
    for h in range(min(cfg["q_heads"], 3)):
        qh = O.pool_rows(x["q"][0, h], g, mode, cfg["dtype"])
        kh = O.pool_rows(x["k"][0, h // G], g, mode, cfg["dtype"])
        for i in range(sh.nb):
            Pw = O.proxy_block_scores(qh, kh, i, sh, g)
            got = P[0, h, i * rb:(i + 1) * rb, :i + 1]
            want = Pw[:, :i + 1]
            err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
            worst = max(worst, float(err.max()))
    assert worst <= 2e-5, worst


@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32", {}), ("gqa8k_small", {}), ("gqa32k_small", {}), ("stress_small", {}),
    ("concentrated", {}), ("d64_bf16", {}), ("fp32_b128", {}),
    ("gqa8k_small", dict(agg_mode=O.AGG_MAX)), ("gqa8k_small", dict(pool=1)),
    ("gqa8k_small", dict(pool=2, budget=0.55)), ("gqa32k_small", dict(force_sink=True, force_diag=True)),
    ("stress_small", dict(pool_mode=O.POOL_STRIDE)), ("gqa8k_small", dict(budget=1.0)),
    ("tiny_fp32", dict(sel_mode=O.SEL_CUMMASS, mass=0.7)),
    ("gqa8k_small", dict(sel_mode=O.SEL_CUMMASS, mass=0.5, budget=0.6)),
    ("gqa32k_small", dict(sel_mode=O.SEL_CUMMASS, mass=0.9, budget=0.5)),
    ("stress_small", dict(sel_mode=O.SEL_CUMMASS, mass=0.8, budget=1.0)),
    ("gqa32k_small", dict(order_mode=O.ORDER_SCORE)), ("tiny_fp32", dict(order_mode=O.ORDER_SCORE)),
    ("ragged_gqa", {}), ("ragged_b64", {}), ("ragged_conc", {}), ("ragged_fp32", {}),
    ("ragged_d64", {}), ("ragged_short", {}), ("ragged_gqa", dict(pool=1)),
    ("ragged_gqa", dict(sel_mode=O.SEL_CUMMASS, mass=0.8, budget=0.6)),
])
def test_kap_lists_match_oracle(name, kw):
    cfg, x, xd = _inputs(name)
    kp = _kp(cfg, **kw)
    g = gpu_kap(xd, cfg, kp)
    units = oracle_lists(x, cfg, kp)
    n = check_lists(units, g)
    assert n == cfg["batch"] * cfg["q_heads"] * -(-seq_len(cfg) // cfg["block"])


@pytest.mark.parametrize("name", ["gqa8k_small", "ragged_gqa"])
def test_kap_lists_noncausal(name):
    cfg, x, xd = _inputs(name)
    kp = _kp(cfg)
    g = gpu_kap(xd, cfg, kp, causal=False)
    check_lists(oracle_lists(x, cfg, kp, causal=False), g)


# ------------------------------------------------------------------ OSK on the oracle's lists

@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32", {}), ("gqa8k_small", {}), ("gqa32k_small", {}), ("stress_small", {}),
    ("concentrated", {}), ("concentrated", dict(skip_mode=O.SKIP_MAXDIFF, skip_param=-2.0)),
    ("concentrated", dict(cap_mode=O.VISITED)), ("concentrated", dict(tight_budget=0.5)),
    ("gqa8k_small", dict(skip_mode=O.SKIP_OFF)), ("d64_bf16", {}), ("fp32_b128", {}),
    ("concentrated", dict(skip_param=0.05, tight_budget=0.3)),
    ("concentrated", dict(vote_rows=32)), ("concentrated", dict(vote_rows=32, cap_mode=O.VISITED)),
    ("concentrated", dict(vote_rows=32, skip_mode=O.SKIP_MAXDIFF, skip_param=-2.0)),
    ("stress_small", dict(vote_rows=32)), ("gqa8k_small", dict(vote_rows=32, skip_mode=O.SKIP_OFF)),
    ("ragged_gqa", {}), ("ragged_b64", {}), ("ragged_conc", {}), ("ragged_conc", dict(vote_rows=32)),
    ("ragged_conc", dict(skip_mode=O.SKIP_MAXDIFF, skip_param=-2.0)), ("ragged_fp32", {}),
    ("ragged_d64", {}), ("ragged_short", {}), ("ragged_b64", dict(vote_rows=32)),
])
def test_osk_on_oracle_lists(name, kw):
    cfg, x, xd = _inputs(name)
    if name in ("concentrated", "ragged_conc"):
        # a loose cap, so that the walk reaches blocks the skip test can drop
        kw.setdefault("tight_budget", 0.5)
    conc = name in ("concentrated", "ragged_conc")
    kp = _kp(cfg, budget=max(cfg["budget"], 0.5) if conc else cfg["budget"])
    op = _op(cfg, **kw)
    units = oracle_lists(x, cfg, kp)
    kmax = max(u["k"] for us in units.values() for u in us)
    idx, cnt = pack_lists(units, cfg, kmax)
    res = gpu_osk(xd, cfg, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), op)
    stats = check_osk_units(x, cfg, op, idx, cnt, res)
    print(name, kw, stats)
    if conc and op.skip_mode != O.SKIP_OFF:
        assert stats["skipped"] > 0


@pytest.mark.parametrize("name", ["gqa32k_small", "ragged_gqa", "ragged_fp32"])
def test_osk_noncausal(name):
    cfg, x, xd = _inputs(name)
    kp, op = _kp(cfg), _op(cfg)
    units = oracle_lists(x, cfg, kp, causal=False)
    kmax = max(u["k"] for us in units.values() for u in us)
    idx, cnt = pack_lists(units, cfg, kmax)
    res = gpu_osk(xd, cfg, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), op, causal=False)
    check_osk_units(x, cfg, op, idx, cnt, res, causal=False)


def test_osk_page_table_remap():
    # K and V stored in a permuted page order; the list holds logical blocks.
    cfg, x, xd = _inputs("gqa8k_small")
    kp, op = _kp(cfg), _op(cfg)
    B, nb = cfg["block"], cfg["seq_len"] // cfg["block"]
    perm = np.random.default_rng(5).permutation(nb).astype(np.int32)   # logical j -> physical
    kph = np.empty_like(x["k"])
    vph = np.empty_like(x["v"])
    for j in range(nb):
        kph[:, :, perm[j] * B:(perm[j] + 1) * B] = x["k"][:, :, j * B:(j + 1) * B]
        vph[:, :, perm[j] * B:(perm[j] + 1) * B] = x["v"][:, :, j * B:(j + 1) * B]
    units = oracle_lists(x, cfg, kp)
    kmax = max(u["k"] for us in units.values() for u in us)
    idx, cnt = pack_lists(units, cfg, kmax)
    pt = np.tile(perm, (cfg["batch"], 1))
    res = gpu_osk(xd, cfg, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), op,
                  page_table=torch.from_numpy(pt).cuda(),
                  kv=(to_dev(kph, cfg["dtype"]), to_dev(vph, cfg["dtype"])))
    check_osk_units(x, cfg, op, idx, cnt, res, page_table=pt, kv_np=(kph, vph))


def test_osk_malformed_lists_stop_the_walk():
    cfg, x, xd = _inputs("gqa8k_small")
    op = _op(cfg, skip_mode=O.SKIP_OFF, tight_budget=1.0)
    nb = cfg["seq_len"] // cfg["block"]
    kmax = 4
    idx = np.full((1, cfg["q_heads"], nb, kmax), -1, np.int32)
    cnt = np.zeros((1, cfg["q_heads"], nb), np.int32)
    for i in range(nb):
        idx[0, :, i, 0] = i
        idx[0, :, i, 1] = i + 1          # not a candidate of block i (causal): walk stops here
        cnt[0, :, i] = 3
    cnt[0, 0, 5] = 0                     # empty list: zeros and -inf
    res = gpu_osk(xd, cfg, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), op)
    B = cfg["block"]
    assert (res["st"][0, :, :, 1:] == 0).all()
    assert (res["st"][0, 1:, :, 0] == 1).all()
    assert res["st"][0, 0, 5, 0] == 0
    assert np.all(res["out"][0, 0, 5 * B:6 * B] == 0) and np.all(np.isneginf(res["lse"][0, 0, 5 * B:6 * B]))
    sh = oshape(cfg)
    G = cfg["q_heads"] // cfg["kv_heads"]
    for h in (1, 3):
        for i in (0, 7, nb - 1):
            o, _ = O.restricted_attention(x["q"][0, h][i * B:(i + 1) * B], x["k"][0, h // G],
                                          x["v"][0, h // G], i, [i], sh)
            assert out_excess(res["out"][0, h, i * B:(i + 1) * B], o, "bf16") <= 0


# ------------------------------------------------------------------ end to end

@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}), ("gqa8k_small", {}), ("gqa32k_small", {}),
                                     ("stress_small", {}), ("concentrated", {}),
                                     ("gqa32k_small", dict(sel_mode=O.SEL_CUMMASS, mass=0.8)),
                                     ("ragged_gqa", {}), ("ragged_b64", {}), ("ragged_conc", {}),
                                     ("ragged_short", {})])
def test_end_to_end(name, kw):
    cfg, x, xd = _inputs(name)
    kp, op = _kp(cfg, **kw), _op(cfg)
    g = gpu_kap(xd, cfg, kp)
    check_lists(oracle_lists(x, cfg, kp), g)
    res = gpu_osk(xd, cfg, g["idx"], g["cnt"], op)
    check_osk_units(x, cfg, op, g["idx"].cpu().numpy(), g["cnt"].cpu().numpy(), res)


@pytest.mark.parametrize("name", ["gqa32k_small", "ragged_gqa"])
def test_full_budget_without_skipping_is_dense(name):
    cfg, x, xd = _inputs(name)
    kp = _kp(cfg, budget=1.0)
    op = _op(cfg, tight_budget=1.0, skip_mode=O.SKIP_OFF)
    g = gpu_kap(xd, cfg, kp)
    res = gpu_osk(xd, cfg, g["idx"], g["cnt"], op)
    sh = oshape(cfg)
    G = cfg["q_heads"] // cfg["kv_heads"]
    for h in range(cfg["q_heads"]):
        ref, lse = O.dense_attention(x["q"][0, h], x["k"][0, h // G], x["v"][0, h // G], sh)
        assert out_excess(res["out"][0, h], ref, "bf16") <= 0
        assert np.abs(res["lse"][0, h] - lse).max() <= 1e-3


@pytest.mark.parametrize("name,causal", [("tiny_fp32", True), ("gqa8k_small", True),
                                         ("stress_small", True), ("d64_bf16", True),
                                         ("fp32_b128", True), ("gqa8k_small", False),
                                         ("ragged_gqa", True), ("ragged_gqa", False),
                                         ("ragged_b64", True), ("ragged_fp32", True),
                                         ("ragged_fp32", False), ("ragged_d64", True),
                                         ("ragged_short", True), ("ragged_short", False)])
def test_dense_matches_oracle(name, causal):
    cfg, x, xd = _inputs(name)
    out, lse = cosa.dense(xd["q"], xd["k"], xd["v"], block=cfg["block"], causal=causal,
                          scale=scale_of(cfg), return_lse=True)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    sh = oshape(cfg, causal)
    G = cfg["q_heads"] // cfg["kv_heads"]
    for h in range(min(cfg["q_heads"], 4)):
        ref, rl = O.dense_attention(x["q"][0, h], x["k"][0, h // G], x["v"][0, h // G], sh)
        assert out_excess(out[0, h], ref, cfg["dtype"]) <= 0
        assert np.abs(lse[0, h] - rl).max() <= (1e-3 if cfg["dtype"] == "bf16" else 1e-5)


def test_bitwise_deterministic():
    cfg, x, xd = _inputs("gqa32k_small")
    kp, op = _kp(cfg), _op(cfg)
    a = gpu_kap(xd, cfg, kp)
    b = gpu_kap(xd, cfg, kp)
    for n in ("idx", "cnt", "hrm", "sc"):
        assert torch.equal(a[n], b[n])
    ra = gpu_osk(xd, cfg, a["idx"], a["cnt"], op)
    rb = gpu_osk(xd, cfg, a["idx"], a["cnt"], op)
    for n in ("out", "lse", "st", "tc"):
        assert np.array_equal(ra[n], rb[n])
    d1 = cosa.dense(xd["q"], xd["k"], xd["v"], block=cfg["block"])
    d2 = cosa.dense(xd["q"], xd["k"], xd["v"], block=cfg["block"])
    assert torch.equal(d1, d2)


def test_ragged_rejects_page_table():
    # pages are whole blocks: a ragged sequence cannot be paged
    cfg, x, xd = _inputs("ragged_gqa")
    nb = num_blocks(dict(cfg, seq_len=seq_len(cfg)))
    idx = torch.zeros((1, cfg["q_heads"], nb, 1), dtype=torch.int32, device="cuda")
    cnt = torch.ones((1, cfg["q_heads"], nb), dtype=torch.int32, device="cuda")
    pt = torch.arange(nb, dtype=torch.int32, device="cuda")[None]
    with pytest.raises(cosa.CosaError):
        cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=cfg["block"], tight_budget=1.0,
                 page_table=pt)


# ------------------------------------------------------------------ varlen batches

VARLEN_LENS = [2216, 1000, 2304, 130]


def _varlen_inputs():
    """Four entries of one padded batch.  Padding rows hold NaN, so any read of them
    would reach the outputs."""
    if "varlen" not in _CACHE:
        cfg = dict(shrink(config(1), 2304, q_heads=4, kv_heads=1, n_salient=3), batch=len(VARLEN_LENS))
        x = make(cfg)
        xp = {}
        for n_ in ("q", "k", "v"):
            a = x[n_].copy()
            for b, L in enumerate(VARLEN_LENS):
                a[b, :, L:] = np.nan
            xp[n_] = a
        _CACHE["varlen"] = (cfg, x, upload(xp, cfg))
    return _CACHE["varlen"]


def _entry(cfg, x, b):
    L = VARLEN_LENS[b]
    cb = dict(cfg, batch=1, seq_len=-(-L // cfg["block"]) * cfg["block"], take=L)
    return cb, {n_: np.ascontiguousarray(x[n_][b:b + 1, :, :L]) for n_ in ("q", "k", "v")}


@pytest.mark.parametrize("kw", [{}, dict(vote_rows=32), dict(causal=False)])
def test_varlen_batch_matches_oracle_per_entry(kw):
    cfg, x, xd = _varlen_inputs()
    causal = kw.pop("causal", True)
    B = cfg["block"]
    kp = _kp(cfg, budget=0.5)
    op = _op(cfg, tight_budget=0.5, **kw)
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=B, budget=kp.budget, causal=causal,
                                 scale=scale_of(cfg), return_scores=True, seq_lens=VARLEN_LENS)
    sentinel = 7.0
    out = torch.full_like(xd["q"], sentinel)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=B,
                                tight_budget=op.tight_budget, skip_mode=op.skip_mode,
                                skip_param=op.skip_param, causal=causal, scale=scale_of(cfg),
                                return_lse=True, return_status=True, return_counts=True, out=out,
                                vote_rows=op.vote_rows, seq_lens=VARLEN_LENS)
    torch.cuda.synchronize()
    o_all = out.float().cpu().numpy()
    for b, L in enumerate(VARLEN_LENS):
        cb, xb = _entry(cfg, x, b)
        nbb = -(-L // B)
        g = dict(idx=idx[b:b + 1, :, :nbb].contiguous(), cnt=cnt[b:b + 1, :, :nbb].contiguous(),
                 hrm=hrm[b:b + 1, :, :nbb].contiguous(), sc=sc[b:b + 1, :, :nbb].contiguous())
        check_lists(oracle_lists(xb, cb, kp, causal=causal), g)
        # blocks past the end of the entry: empty lists, nothing visited, rows untouched
        assert (cnt[b, :, nbb:] == 0).all() and (idx[b, :, nbb:] == -1).all()
        assert (st[b, :, nbb:] == 0).all() and (tc[b, :, nbb:] == 0).all()
        assert np.all(o_all[b, :, L:] == sentinel)
        res = dict(out=o_all[b:b + 1, :, :L], lse=lse[b:b + 1, :, :L].cpu().numpy(),
                   st=st[b:b + 1, :, :nbb].cpu().numpy(), tc=tc[b:b + 1, :, :nbb].cpu().numpy())
        check_osk_units(xb, cb, op, g["idx"].cpu().numpy(), g["cnt"].cpu().numpy(), res, causal=causal)


def test_varlen_shared_lists_block64():
    """A varlen batch at block 64 with lists shared by the KV head's query heads (four heads per
    workgroup): bitwise the per-head walk of the same lists, NaN padding never read."""
    lens = [3000, 1000, 4096, 70]
    cfg = dict(shrink(config(4), 4096, q_heads=7, kv_heads=1), batch=len(lens))
    x = make(cfg)
    for n_ in ("q", "k", "v"):
        x[n_] = x[n_].copy()
        for b, L in enumerate(lens):
            x[n_][b, :, L:] = np.nan
    xd = upload(x, cfg)
    B, G = cfg["block"], cfg["q_heads"] // cfg["kv_heads"]
    idx, cnt, _ = cosa.kap(xd["q"], xd["k"], block=B, budget=cfg["budget"], scale=scale_of(cfg),
                           share_kv=True, seq_lens=lens)
    kw = dict(block=B, tight_budget=cfg["tight_budget"], scale=scale_of(cfg), return_lse=True,
              return_status=True, return_counts=True, seq_lens=lens)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, shared_lists=True, **kw)
    idx_h = idx.repeat_interleave(G, dim=1).contiguous()
    cnt_h = cnt.repeat_interleave(G, dim=1).contiguous()
    out2, lse2, st2, tc2 = cosa.osk(xd["q"], xd["k"], xd["v"], idx_h, cnt_h, **kw)
    torch.cuda.synchronize()
    assert torch.equal(st, st2) and torch.equal(tc, tc2)
    for b, L in enumerate(lens):
        assert torch.equal(out[b, :, :L], out2[b, :, :L])
        assert torch.equal(lse[b, :, :L], lse2[b, :, :L])
        assert torch.isfinite(out[b, :, :L].float()).all()


def test_varlen_entry_equals_single_sequence_call():
    # an entry of a varlen batch gives bitwise what a batch-1 call on its rows gives
    cfg, x, xd = _varlen_inputs()
    B = cfg["block"]
    idx, cnt, hrm = cosa.kap(xd["q"], xd["k"], block=B, budget=0.3, scale=scale_of(cfg),
                             seq_lens=VARLEN_LENS)
    out = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=B, tight_budget=0.15,
                   scale=scale_of(cfg), seq_lens=VARLEN_LENS)
    dn = cosa.dense(xd["q"], xd["k"], xd["v"], block=B, scale=scale_of(cfg), seq_lens=VARLEN_LENS)
    for b, L in enumerate(VARLEN_LENS):
        q1, k1, v1 = (xd[n_][b:b + 1, :, :L].contiguous() for n_ in ("q", "k", "v"))
        nbb = -(-L // B)
        km = min(idx.shape[3], nbb)            # a list holds at most nb entries
        i1, c1, h1 = cosa.kap(q1, k1, block=B, budget=0.3, scale=scale_of(cfg), kmax=km)
        o1 = cosa.osk(q1, k1, v1, i1, c1, block=B, tight_budget=0.15, scale=scale_of(cfg))
        d1 = cosa.dense(q1, k1, v1, block=B, scale=scale_of(cfg))
        assert torch.equal(idx[b:b + 1, :, :nbb, :km], i1) and (idx[b, :, :nbb, km:] == -1).all()
        assert torch.equal(cnt[b:b + 1, :, :nbb], c1)
        assert torch.equal(hrm[b:b + 1, :, :nbb], h1)
        assert torch.equal(out[b:b + 1, :, :L], o1)
        assert torch.equal(dn[b:b + 1, :, :L], d1)


PAGED_LENS = [1024, 512, 2304, 256]   # whole blocks of 128 in a 2304-row layout (18 pages)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_page_table_reads_pages_past_each_entry(dtype):
    """A paged varlen batch: the logical blocks of every entry live in the last of the 18 pages
    of its KV head, in a random order, so those of the shorter entries lie past the end of the
    entry's own tokens; pages no entry names, and query rows past each entry, hold NaN.  Each entry is
    compared with the oracle walking the same physical pages through the same table."""
    cfg = dict(shrink(config(1), 2304, q_heads=4, kv_heads=1, n_salient=3), batch=len(PAGED_LENS),
               dtype=dtype)
    x = make(cfg)
    B = cfg["block"]
    nb = cfg["seq_len"] // B
    rng = np.random.default_rng(77)
    pt = np.zeros((len(PAGED_LENS), nb), np.int32)
    kph, vph = np.full_like(x["k"], np.nan), np.full_like(x["v"], np.nan)
    qn = x["q"].copy()
    past_end = 0
    for b, L in enumerate(PAGED_LENS):
        nbb = L // B
        pages = rng.permutation(np.arange(nb - nbb, nb)).astype(np.int32)   # the last nbb pages
        pt[b, :nbb] = pages
        past_end += int((pages >= nbb).sum())
        for j, pg in enumerate(pages):
            kph[b, :, pg * B:(pg + 1) * B] = x["k"][b, :, j * B:(j + 1) * B]
            vph[b, :, pg * B:(pg + 1) * B] = x["v"][b, :, j * B:(j + 1) * B]
        qn[b, :, L:] = np.nan
    assert past_end == 8 + 4 + 2
    kp = _kp(cfg, budget=0.5)
    op = _op(cfg, tight_budget=0.5)
    entries = [dict(cfg, batch=1, seq_len=L) for L in PAGED_LENS]
    units = [oracle_lists({n_: x[n_][b:b + 1, :, :L] for n_ in ("q", "k")}, entries[b], kp)
             for b, L in enumerate(PAGED_LENS)]
    kmax = max(u["k"] for us in units for uu in us.values() for u in uu)
    idx = np.full((len(PAGED_LENS), cfg["q_heads"], nb, kmax), -1, np.int32)
    cnt = np.zeros((len(PAGED_LENS), cfg["q_heads"], nb), np.int32)
    for b, L in enumerate(PAGED_LENS):
        ib, cb_ = pack_lists(units[b], entries[b], kmax)
        idx[b, :, :L // B], cnt[b, :, :L // B] = ib[0], cb_[0]
    out, lse, st, tc = cosa.osk(to_dev(qn, dtype), to_dev(kph, dtype), to_dev(vph, dtype),
                                torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), block=B,
                                tight_budget=op.tight_budget, scale=scale_of(cfg),
                                page_table=torch.from_numpy(pt).cuda(), seq_lens=PAGED_LENS,
                                return_lse=True, return_status=True, return_counts=True)
    torch.cuda.synchronize()
    o_all, lse, st, tc = out.float().cpu().numpy(), lse.cpu().numpy(), st.cpu().numpy(), tc.cpu().numpy()
    for b, L in enumerate(PAGED_LENS):
        nbb = L // B
        assert np.isfinite(o_all[b, :, :L]).all()
        res = dict(out=o_all[b:b + 1, :, :L], lse=lse[b:b + 1, :, :L], st=st[b:b + 1, :, :nbb],
                   tc=tc[b:b + 1, :, :nbb])
        check_osk_units({"q": x["q"][b:b + 1, :, :L]}, entries[b], op, idx[b:b + 1, :, :nbb],
                        cnt[b:b + 1, :, :nbb], res, page_table=pt[b:b + 1, :nbb],
                        kv_np=(kph[b:b + 1], vph[b:b + 1]))


def test_binding_rejects_mismatched_tensors():
    """Sizes the library takes from q (batch, seq, head dim) must hold for k, v and out: the
    binding raises before any call instead of letting a kernel read or write past an end."""
    cfg, x, xd = _inputs("gqa8k_small")
    q, k, v = xd["q"], xd["k"], xd["v"]
    B = cfg["block"]
    idx, cnt, _ = cosa.kap(q, k, block=B, budget=0.3)
    bad_k = [k[:, :, :-B].contiguous(), k[:, :, :, :64].contiguous(),
             torch.cat([k, k], dim=0), k.float()]
    for kk in bad_k:
        with pytest.raises(cosa.CosaError):
            cosa.kap(q, kk, block=B, budget=0.3)
        with pytest.raises(cosa.CosaError):
            cosa.osk(q, kk, kk, idx, cnt, block=B, tight_budget=0.15)
        with pytest.raises(cosa.CosaError):
            cosa.dense(q, kk, kk, block=B)
        with pytest.raises(cosa.CosaError):
            cosa.prefill(q, kk, kk, block=B, budget=0.3, tight_budget=0.15)
    with pytest.raises(cosa.CosaError):
        cosa.osk(q, k, v[:, :, :-B].contiguous(), idx, cnt, block=B, tight_budget=0.15)
    with pytest.raises(cosa.CosaError):
        cosa.dense(q, k, v, block=B, out=torch.empty_like(q)[:, :, :-B].contiguous())
    with pytest.raises(cosa.CosaError):
        cosa.dense(q, k, v, block=B, out=torch.empty_like(q, dtype=torch.float32))
    with pytest.raises(cosa.CosaError):
        cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=0.15, out=torch.empty_like(q)[:, :1])
    with pytest.raises(cosa.CosaError):
        cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=0.15,
                 page_table=torch.zeros((1, 3), dtype=torch.int32, device="cuda"))
    with pytest.raises(cosa.CosaError):
        cosa.osk(q, k, v, idx.cpu(), cnt, block=B, tight_budget=0.15)


def test_varlen_dense_matches_oracle():
    cfg, x, xd = _varlen_inputs()
    out, lse = cosa.dense(xd["q"], xd["k"], xd["v"], block=cfg["block"], scale=scale_of(cfg),
                          return_lse=True, seq_lens=VARLEN_LENS)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b, L in enumerate(VARLEN_LENS):
        cb, xb = _entry(cfg, x, b)
        sh = oshape(cb)
        for h in range(cfg["q_heads"]):
            ref, rl = O.dense_attention(xb["q"][0, h], xb["k"][0, 0], xb["v"][0, 0], sh)
            assert out_excess(out[b, h, :L], ref, "bf16") <= 0
            assert np.abs(lse[b, h, :L] - rl).max() <= 1e-3


# ------------------------------------------------------------------ GQA-shared lists

def _oracle_kv_lists(x, cfg, kp, causal=True):
    sh = oshape(cfg, causal)
    G = cfg["q_heads"] // cfg["kv_heads"]
    return {(b, g): O.kap_kv_group(x["q"][b, g * G:(g + 1) * G], x["k"][b, g], sh, kp)
            for b in range(cfg["batch"]) for g in range(cfg["kv_heads"])}


@pytest.mark.parametrize("name,kw", [("gqa8k_small", {}), ("stress_small", {}), ("ragged_gqa", {}),
                                     ("gqa32k_small", dict(sel_mode=O.SEL_CUMMASS, mass=0.8, budget=0.5)),
                                     ("gqa8k_small", dict(pool=2))])
def test_shared_kv_lists_match_oracle(name, kw):
    cfg, x, xd = _inputs(name)
    kp = _kp(cfg, **kw)
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=cfg["block"], budget=kp.budget, pool=kp.pool,
                                 scale=scale_of(cfg), return_scores=True, sel_mode=kp.sel_mode,
                                 mass=kp.mass, share_kv=True)
    torch.cuda.synchronize()
    assert idx.shape[1] == cfg["kv_heads"]
    n = check_lists(_oracle_kv_lists(x, cfg, kp), dict(idx=idx, cnt=cnt, hrm=hrm, sc=sc))
    assert n == cfg["batch"] * cfg["kv_heads"] * -(-seq_len(cfg) // cfg["block"])


@pytest.mark.parametrize("name,cap_mode", [("gqa8k_small", 0), ("stress_small", 0), ("concentrated", 0),
                                           ("concentrated", 1), ("ragged_gqa", 0), ("ragged_conc", 0),
                                           ("concentrated_b64", 0), ("concentrated_b64", 1),
                                           ("ragged_b64", 0)])
def test_osk_walks_shared_kv_lists(name, cap_mode):
    """Shared lists: the query heads of a KV head share each K/V tile in one workgroup (two
    heads at block 128, four at block 64, the last workgroup of an odd group part empty),
    each with its own state, vote and cap; the walk of every head is bitwise the one of the
    per-head kernel handed the same list."""
    cfg, x, xd = _inputs(name)
    conc = name.startswith("concentrated")
    kp = _kp(cfg, budget=0.5 if conc else cfg["budget"])
    op = _op(cfg, tight_budget=0.5 if conc else cfg["tight_budget"], cap_mode=cap_mode)
    G = cfg["q_heads"] // cfg["kv_heads"]
    idx, cnt, _ = cosa.kap(xd["q"], xd["k"], block=cfg["block"], budget=kp.budget,
                           scale=scale_of(cfg), share_kv=True)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=cfg["block"],
                                tight_budget=op.tight_budget, cap_mode=op.cap_mode,
                                skip_mode=op.skip_mode, skip_param=op.skip_param,
                                scale=scale_of(cfg), return_lse=True, return_status=True,
                                return_counts=True, shared_lists=True)
    # the same lists handed to every query head explicitly: bitwise the same walk
    idx_h = idx.repeat_interleave(G, dim=1).contiguous()
    cnt_h = cnt.repeat_interleave(G, dim=1).contiguous()
    out2, lse2, st2, tc2 = cosa.osk(xd["q"], xd["k"], xd["v"], idx_h, cnt_h, block=cfg["block"],
                                    tight_budget=op.tight_budget, cap_mode=op.cap_mode,
                                    skip_mode=op.skip_mode, skip_param=op.skip_param,
                                    scale=scale_of(cfg), return_lse=True, return_status=True,
                                    return_counts=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(st, st2)
    assert torch.equal(lse, lse2) and torch.equal(tc, tc2)
    res = dict(out=out.float().cpu().numpy(), lse=lse.cpu().numpy(), st=st.cpu().numpy(),
               tc=tc.cpu().numpy())
    stats = check_osk_units(x, cfg, op, idx_h.cpu().numpy(), cnt_h.cpu().numpy(), res)
    if conc:
        assert stats["skipped"] > 0
