"""GPU: cosa_prefill (proxy and walk pipelined over groups of KV heads on two streams) gives
bitwise what cosa_proxy_select followed by cosa_ordered_sparse_attn gives on the whole layer:
lists, outputs and LSE, for several head groupings, block sizes, ragged and varlen batches,
shared lists and skip settings.  The serial calls are themselves pinned to the
oracle by the parity tests."""
import numpy as np
import pytest
import torch

import block_sparse_attention_kap_amd as cosa
from synth import config, make, ragged, shrink
from gpu_helpers import scale_of, upload

pytestmark = pytest.mark.gpu

VARLEN = [2216, 1000, 2304, 130]


def _cfg(name):
    if name == "gqa8k_small":
        return shrink(config(1), 2304, q_heads=8, kv_heads=4, n_salient=3)
    if name == "stress_small":
        return shrink(config(4), 4096, q_heads=7, kv_heads=1)
    if name == "ragged_gqa":
        return ragged(shrink(config(1), 2304, q_heads=8, kv_heads=2, n_salient=3), 2304 - 88)
    if name == "concentrated":
        c = shrink(config(1), 3072, q_heads=4, kv_heads=2, n_salient=5)
        c.update(salient_gain=12.0, q_noise=0.2)
        return c
    if name == "varlen":
        return dict(shrink(config(1), 2304, q_heads=4, kv_heads=2, n_salient=3), batch=len(VARLEN))
    if name == "fp32":
        return dict(shrink(config(2), 2048, q_heads=4, kv_heads=2, n_salient=3), dtype="f32", block=128)
    raise KeyError(name)


_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        cfg = _cfg(name)
        x = make(cfg)
        if name == "varlen":   # padding rows hold NaN: a read of them would reach the outputs
            for n_ in ("q", "k", "v"):
                x[n_] = x[n_].copy()
                for b, L in enumerate(VARLEN):
                    x[n_][b, :, L:] = np.nan
        _CACHE[name] = (cfg, x, upload(x, cfg))
    return _CACHE[name]


def _both(cfg, xd, head_chunks, seq_lens=None, **kw):
    """The serial calls and the pipelined call on the same inputs."""
    q, k, v = xd["q"], xd["k"], xd["v"]
    B = cfg["block"]
    budget = kw.pop("budget", cfg["budget"])
    tight = kw.pop("tight_budget", cfg["tight_budget"])
    share = kw.pop("share_kv", False)
    causal = kw.pop("causal", True)
    idx, cnt, hrm = cosa.kap(q, k, block=B, budget=budget, scale=scale_of(cfg), share_kv=share,
                             seq_lens=seq_lens, causal=causal)
    out, lse = cosa.osk(q, k, v, idx, cnt, block=B, tight_budget=tight, scale=scale_of(cfg),
                        return_lse=True, shared_lists=share, seq_lens=seq_lens, causal=causal, **kw)
    torch.cuda.synchronize()
    ref = dict(out=out.clone(), lse=lse.clone(), idx=idx.clone(), cnt=cnt.clone(), hrm=hrm.clone())
    out2, lse2, (idx2, cnt2, hrm2) = cosa.prefill(
        q, k, v, block=B, budget=budget, tight_budget=tight, head_chunks=head_chunks,
        share_kv=share, scale=scale_of(cfg), return_lse=True, return_lists=True,
        seq_lens=seq_lens, causal=causal, **kw)
    torch.cuda.synchronize()
    return ref, dict(out=out2, lse=lse2, idx=idx2, cnt=cnt2, hrm=hrm2)


def _same(ref, got, rows=None):
    for key in ("idx", "cnt", "hrm"):
        assert torch.equal(ref[key], got[key]), key
    if rows is None:
        assert torch.equal(ref["out"], got["out"])
        assert torch.equal(ref["lse"], got["lse"])
    else:
        for b, L in enumerate(rows):
            assert torch.equal(ref["out"][b, :, :L], got["out"][b, :, :L])
            assert torch.equal(ref["lse"][b, :, :L], got["lse"][b, :, :L])


@pytest.mark.parametrize("name,chunks,kw", [
    ("gqa8k_small", 1, {}), ("gqa8k_small", 2, {}), ("gqa8k_small", 4, {}),
    ("gqa8k_small", 2, dict(share_kv=True)), ("stress_small", 1, {}), ("ragged_gqa", 2, {}),
    ("concentrated", 2, dict(budget=0.5, tight_budget=0.5)),
    ("concentrated", 2, dict(budget=0.5, tight_budget=0.3, cap_mode=1)),
    ("concentrated", 1, dict(budget=0.5, tight_budget=0.5, vote_rows=32)),
    ("gqa8k_small", 2, dict(causal=False)), ("fp32", 2, {}),
])
def test_prefill_equals_serial(name, chunks, kw):
    print(f"prefill: {name} chunks={chunks} {kw}", flush=True)
    cfg, x, xd = _inputs(name)
    ref, got = _both(cfg, xd, chunks, **kw)
    _same(ref, got)


def test_prefill_varlen_batch():
    cfg, x, xd = _inputs("varlen")
    ref, got = _both(cfg, xd, 2, seq_lens=VARLEN)
    _same(ref, got, rows=VARLEN)


def test_prefill_back_to_back_reuses_buffers():
    """Two calls in a row on the same lists and workspace: the second proxy waits for the
    first call's walks before it overwrites the lists."""
    cfg, x, xd = _inputs("gqa8k_small")
    B = cfg["block"]
    kw = dict(block=B, budget=cfg["budget"], tight_budget=cfg["tight_budget"], head_chunks=4,
              scale=scale_of(cfg), return_lists=True)
    out1, lists = cosa.prefill(xd["q"], xd["k"], xd["v"], **kw)
    first = out1.clone()
    out2, _ = cosa.prefill(xd["q"], xd["k"], xd["v"], lists=lists, **kw)
    torch.cuda.synchronize()
    assert torch.equal(first, out2)


def test_prefill_rejects_bad_grouping():
    cfg, x, xd = _inputs("gqa8k_small")
    with pytest.raises(cosa.CosaError):
        cosa.prefill(xd["q"], xd["k"], xd["v"], block=cfg["block"], budget=cfg["budget"],
                     tight_budget=cfg["tight_budget"], head_chunks=3, scale=scale_of(cfg))
