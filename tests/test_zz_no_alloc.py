"""The proxy entry point that allocates nothing (cosa_proxy_select_noalloc), called through
the C ABI, against cosa_proxy_select on the same inputs: bitwise the same lists, counts, HRM
counts and scores, on calls in a row whose second input is smaller than the first (the
static scratch then still holds the first call's data)."""
import pytest
import torch

import block_sparse_attention_kap_amd as cosa
from synth import config, make, shrink
from gpu_helpers import scale_of, upload

pytestmark = pytest.mark.gpu

SCRATCH = cosa._lib.COSA_NOALLOC_SCRATCH_MIB << 20


def _pair(xd, cfg, budget=None, **kw):
    B = cfg["block"]
    budget = cfg["budget"] if budget is None else budget
    ref = cosa.kap(xd["q"], xd["k"], block=B, budget=budget, scale=scale_of(cfg),
                   return_scores=True, **kw)
    got = cosa.kap_noalloc(xd["q"], xd["k"], block=B, budget=budget, scale=scale_of(cfg),
                           return_scores=True, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("visit_idx", "visit_cnt", "hrm_cnt", "visit_score"), ref, got):
        assert torch.equal(a, b), name


def _layer_bytes(xd, cfg, **kw):
    sh = cosa.make_shape(xd["q"], xd["k"], cfg["block"], True, scale_of(cfg), kw.get("seq_lens"))
    kp = cosa.KapParams(cfg["budget"], 0, 0, 0, 0, 0.9, 0, 0, 0, int(kw.get("share_kv", False)))
    return cosa.kap_workspace_bytes(sh, kp)


def test_noalloc_equals_workspace_call_large_then_small():
    big = shrink(config(3), 65536)                       # 32/8 heads at 64K: cut into slices
    small = shrink(config(1), 4096, q_heads=8, kv_heads=2, n_salient=3)
    print("no-alloc proxy: 64K layer (sliced), then a 4K layer", flush=True)
    xb = upload(make(big), big)
    assert _layer_bytes(xb, big) > SCRATCH
    _pair(xb, big)
    _pair(xb, big, share_kv=True)
    del xb
    xs = upload(make(small), small)
    assert _layer_bytes(xs, small) < SCRATCH
    _pair(xs, small)
    _pair(xs, small, budget=0.5, share_kv=True)


def test_noalloc_varlen_then_block64():
    """A varlen batch (sliced per entry), then a smaller block-64 problem with G = 7."""
    lens = [3000, 1000, 4096, 130]
    cfg = dict(shrink(config(1), 4096, q_heads=8, kv_heads=2, n_salient=3), batch=len(lens))
    print("no-alloc proxy: varlen batch, then block 64", flush=True)
    xd = upload(make(cfg), cfg)
    _pair(xd, cfg, seq_lens=lens)
    c4 = shrink(config(4), 2048, q_heads=7, kv_heads=1)
    x4 = upload(make(c4), c4)
    _pair(x4, c4)
    _pair(x4, c4, share_kv=True)


def test_noalloc_rejects_a_head_larger_than_the_scratch():
    """4096 blocks of 128 tokens: one query head's block scores alone need 256 MiB, more than
    the static array; the call returns COSA_ERR_SCRATCH and launches nothing."""
    q = torch.empty((1, 1, 4096 * 128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cosa.CosaError) as e:
        cosa.kap_noalloc(q, q, block=128, budget=0.1)
    assert e.value.status == cosa._lib.COSA_ERR_SCRATCH
