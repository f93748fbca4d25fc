"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

The whole hot path (KAP then OSK on the KAP lists, default skip rule) runs on the
full workload; every list is checked for the invariants that hold at any size, and
a stratified sample of query blocks (two query heads on different KV heads; the
last, first and spread query blocks) is compared with the oracle one unit at a time.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle.compare import check_list, replay_walk
from synth import config, make
from synth.inputs import shrink
from gpu_helpers import TOL_LSE, gpu_kap, out_excess, oshape, scale_of, upload
import block_sparse_attention_kap_amd as cosa

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


def _run_and_compare(cfg, heads, blocks):
    """KAP then OSK on the whole workload; list invariants everywhere, the sampled units
    (heads x blocks) against the oracle one at a time."""
    x = make(cfg)
    xd = upload(x, cfg)
    kp = O.KapParams(budget=cfg["budget"])
    op = O.OskParams(tight_budget=cfg["tight_budget"])
    g = gpu_kap(xd, cfg, kp)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], g["idx"], g["cnt"], block=cfg["block"],
                                tight_budget=op.tight_budget, scale=scale_of(cfg), return_lse=True,
                                return_status=True, return_counts=True)
    torch.cuda.synchronize()
    idx, cnt, hrm, sc = (g[n].cpu().numpy() for n in ("idx", "cnt", "hrm", "sc"))
    st, tc = st.cpu().numpy(), tc.cpu().numpy()
    _list_invariants(idx, cnt, hrm, cfg, cfg["budget"])
    nb = cfg["seq_len"] // cfg["block"]
    n = np.arange(1, nb + 1)
    kprime = np.minimum(cnt[0], np.maximum(1, np.ceil(cfg["tight_budget"] * n)).astype(np.int32))
    assert (tc[0, :, :, 1] <= kprime).all() and (tc[0, :, :, 1] >= 1).all()
    del xd
    sh = oshape(cfg)
    G = cfg["q_heads"] // cfg["kv_heads"]
    B = cfg["block"]
    worst, worst_lse = -1.0, 0.0
    for h in heads:
        units = O.kap_head(x["q"][0, h], x["k"][0, h // G], sh, kp, blocks)
        for u, i in zip(units, blocks):
            ok, msg = check_list(u, idx[0, h, i], int(cnt[0, h, i]), int(hrm[0, h, i]), sc[0, h, i])
            assert ok, f"list (h={h}, i={i}): {msg}"
            fn = lambda forced: O.osk_unit(x["q"][0, h], x["k"][0, h // G], x["v"][0, h // G], i,
                                           idx[0, h, i], int(cnt[0, h, i]), sh, op, forced=forced)
            ok, w, msg, _ = replay_walk(fn, st[0, h, i])
            assert ok, f"walk (h={h}, i={i}): {msg}"
            assert tc[0, h, i, 0] == w["visited"] and tc[0, h, i, 1] == w["n_comp"]
            o = out[0, h, i * B:(i + 1) * B].float().cpu().numpy()
            lz = lse[0, h, i * B:(i + 1) * B].cpu().numpy()
            worst = max(worst, out_excess(o, w["out"], cfg["dtype"]))
            worst_lse = max(worst_lse, float(np.abs(lz - w["lse"]).max()))
    print(f"{cfg['name']}: sampled {len(heads) * len(blocks)} units, tolerance excess {worst:.3e}, "
          f"lse err {worst_lse:.3e}, skipped {(st == 2).sum()} of {(st > 0).sum()} visited", flush=True)
    assert worst <= 0 and worst_lse <= TOL_LSE[cfg["dtype"]]


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_full_size_sampled(ci):
    cfg = config(ci)
    print(f"full-size parity: {cfg['name']}", flush=True)
    G = cfg["q_heads"] // cfg["kv_heads"]
    nb = cfg["seq_len"] // cfg["block"]
    blocks = sorted(set([nb - 1, nb - 2, nb - 3, nb - 4, 0, 1, nb // 2, nb // 3, nb // 5]))
    _run_and_compare(cfg, [0, G + 1], blocks)


@pytest.mark.parametrize("ci,seq_len", [(4, 4096 * 64), (3, 4096 * 128)])
def test_max_blocks_sampled(ci, seq_len):
    """The largest sequence the library takes: 4096 blocks (the staged list, the select
    kernel and the proxy workspace at their limits), one query head."""
    cfg = shrink(config(ci), seq_len, q_heads=1, kv_heads=1)
    assert cfg["seq_len"] // cfg["block"] == 4096
    print(f"maximum-size parity: {cfg['name']}", flush=True)
    _run_and_compare(cfg, [0], [4095, 4094, 4000, 2048, 1000, 1, 0])


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


@pytest.mark.parametrize("ci,mode", [(3, "shared_kv"), (4, "shared_kv"), (2, "vote_rows_32")])
def test_full_size_modes_sampled(ci, mode):
    """The GQA-shared lists (one list per KV head; at block 64 four query heads per workgroup,
    the second workgroup of a 7-head group one head short) and the 32-row skip votes at full
    size."""
    cfg = config(ci)
    print(f"full-size parity: {cfg['name']} {mode}", flush=True)
    x = make(cfg)
    xd = upload(x, cfg)
    share = mode == "shared_kv"
    vr = 32 if mode == "vote_rows_32" else 0
    kp = O.KapParams(budget=cfg["budget"])
    op = O.OskParams(tight_budget=cfg["tight_budget"], vote_rows=vr)
    idx, cnt, hrm, sc = cosa.kap(xd["q"], xd["k"], block=cfg["block"], budget=kp.budget,
                                 scale=scale_of(cfg), return_scores=True, share_kv=share)
    out, lse, st, tc = cosa.osk(xd["q"], xd["k"], xd["v"], idx, cnt, block=cfg["block"],
                                tight_budget=op.tight_budget, scale=scale_of(cfg), return_lse=True,
                                return_status=True, return_counts=True, vote_rows=vr,
                                shared_lists=share)
    torch.cuda.synchronize()
    idx, cnt, hrm, sc = (t.cpu().numpy() for t in (idx, cnt, hrm, sc))
    st, tc = st.cpu().numpy(), tc.cpu().numpy()
    hl = cfg["kv_heads"] if share else cfg["q_heads"]
    assert idx.shape[1] == hl
    _list_invariants(idx, cnt, hrm, cfg, cfg["budget"])
    del xd
    sh = oshape(cfg)
    G = cfg["q_heads"] // cfg["kv_heads"]
    B = cfg["block"]
    nb = cfg["seq_len"] // B
    blocks = sorted(set([nb - 1, nb - 2, 0, 1, nb // 2, nb // 3]))
    worst, worst_lse = -1.0, 0.0
    for h in sorted({0, G - 1, G + 1}):
        kvh = h // G
        lh = kvh if share else h
        if share:
            units = O.kap_kv_group(x["q"][0, kvh * G:(kvh + 1) * G], x["k"][0, kvh], sh, kp, blocks)
        else:
            units = O.kap_head(x["q"][0, h], x["k"][0, kvh], sh, kp, blocks)
        for u, i in zip(units, blocks):
            ok, msg = check_list(u, idx[0, lh, i], int(cnt[0, lh, i]), int(hrm[0, lh, i]), sc[0, lh, i])
            assert ok, f"list (h={h}, i={i}): {msg}"
            groups = B // vr if vr else 1
            rows = B // groups
            for g in range(groups):
                gst = (st[0, h, i].astype(np.int64) >> (2 * g)) & 3 if vr else st[0, h, i]
                fn = lambda forced, g=g: O.osk_unit(x["q"][0, h], x["k"][0, kvh], x["v"][0, kvh], i,
                                                    idx[0, lh, i], int(cnt[0, lh, i]), sh, op,
                                                    forced=forced, group=g if vr else None)
                ok, w, msg, _ = replay_walk(fn, gst)
                assert ok, f"walk (h={h}, i={i}, group={g}): {msg}"
                r0 = i * B + g * rows
                o = out[0, h, r0:r0 + rows].float().cpu().numpy()
                lz = lse[0, h, r0:r0 + rows].cpu().numpy()
                worst = max(worst, out_excess(o, w["out"], cfg["dtype"]))
                worst_lse = max(worst_lse, float(np.abs(lz - w["lse"]).max()))
    print(f"{cfg['name']} {mode}: tolerance excess {worst:.3e}, lse err {worst_lse:.3e}", flush=True)
    assert worst <= 0 and worst_lse <= TOL_LSE[cfg["dtype"]]


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
